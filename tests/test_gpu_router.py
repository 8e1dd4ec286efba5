"""Router scores on the matrix cores against the oracle, element by element,
at shapes that select each kernel: the wide 256-token x 96-expert tiles (at
least 256 of them), the 128 x 64 tiles, and the few-token kernel -- with
ragged token and expert counts, expert counts that are not a multiple of 4
(scalar stores), and a hidden size with an odd number of 32-element K steps
(the K sweeps start at two offsets and wrap around).  Each shape also runs on
the pre-split weight planes, which must give bitwise the same logits."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_02_amd as moe
from _parity import LOGIT_TOL, THREADS, device, host, normwise

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,H", [(6000, 1000, 256),    # wide: 24 x 11 tiles, last ones ragged
                                   (6000, 1003, 288),    # wide, E % 4 != 0, 9 K steps
                                   (8192, 768, 6144),    # wide: the full-scale shape, 256 tiles
                                   (700, 130, 320),      # 128 x 64 tiles
                                   (40, 100, 512)])      # few tokens
@pytest.mark.parametrize("planes", [False, True])
def test_router_logits_match_oracle(T, E, H, planes):
    dev = device()
    print(f"\n[case] router T={T} E={E} H={H} planes={planes}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(T * 31 + E)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.randn(E, H, generator=g) * 0.02
    logits = torch.full((T, E), float("nan"), device=dev)
    xd, wd = x.to(dev), w.to(dev)
    moe.moe_router_logits(xd, wd, logits)
    if planes:
        wp = torch.empty((3, E, H), dtype=torch.bfloat16, device=dev)
        moe.moe_router_split_weights(wd, wp)
        from_planes = torch.full((T, E), float("nan"), device=dev)
        moe.moe_router_logits(xd, wd, from_planes, wp)
        torch.cuda.synchronize()
        assert torch.equal(from_planes, logits)   # bitwise
        logits = from_planes
    torch.cuda.synchronize()
    got = host(logits).astype(np.float64)
    if T * E * H > 2e9:   # full-scale: the oracle computes sampled tokens
        rows = np.unique(np.r_[0:8, T - 8:T, np.random.default_rng(0).choice(T, 48, False)])
    else:
        rows = np.arange(T)
    xs = x.float().numpy()[rows]
    wn = w.numpy()
    ref = oracle.router_logits(xs, wn, threads=THREADS)
    assert np.isfinite(got).all()
    assert normwise(got[rows], ref) <= LOGIT_TOL
    # every product is exact (x bf16, the weight split into three bf16
    # planes), so the error is the fp32 accumulation's: within H unit
    # roundoffs of the sum of |x w|
    bound = H * 2.0 ** -24 * (np.abs(xs).astype(np.float64) @ np.abs(wn).astype(np.float64).T)
    assert (np.abs(got[rows] - ref) <= bound + 1e-30).all()


@pytest.mark.parametrize("E,H", [(768, 6144), (13, 40)])
def test_router_split_is_exact(E, H):
    # hi + mid + lo == w exactly, each plane a bf16 value, hi the truncation of
    # w; includes zeros, signed zeros, tiny and huge magnitudes (the split is
    # exact for |w| >= 2^-110, where no remainder is subnormal)
    dev = device()
    print(f"\n[case] router split E={E} H={H}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(E * 7 + H)
    w = torch.randn(E, H, generator=g) * 0.02
    flat = w.view(-1)
    special = torch.tensor([0.0, -0.0, 1e-30, -1.234567 * 2.0 ** -109, 3e38, -1.5, 2.0 ** -100,
                            1.0 + 2.0 ** -23])
    flat[:special.numel()] = special
    wp = torch.empty((3, E, H), dtype=torch.bfloat16, device=dev)
    moe.moe_router_split_weights(w.to(dev), wp)
    torch.cuda.synchronize()
    p = wp.cpu().double()
    np.testing.assert_array_equal((p[0] + p[1] + p[2]).numpy(), w.double().numpy())
    hi_bits = wp[0].cpu().view(torch.int16).numpy().astype(np.uint16)
    w_bits = (w.view(torch.int32).numpy().astype(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(hi_bits, w_bits)


@pytest.mark.parametrize("T,E,H", [(40, 100, 512), (700, 130, 320), (6000, 1003, 288)])
def test_router_logits_misaligned_pointers(T, E, H):
    # x and w_router offset by 4 bytes from a 16-byte boundary (the API takes
    # element-aligned pointers): the matrix-core kernels move 16-byte pieces,
    # so these shapes go to the FMA kernel and must still match the oracle
    dev = device()
    print(f"\n[case] router misaligned T={T} E={E} H={H}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(T + E + H)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.randn(E, H, generator=g) * 0.02
    xb = torch.zeros(T * H + 8, dtype=torch.bfloat16, device=dev)
    wb = torch.zeros(E * H + 4, dtype=torch.float32, device=dev)
    xd = xb[2:2 + T * H].view(T, H)
    wd = wb[1:1 + E * H].view(E, H)
    xd.copy_(x)
    wd.copy_(w)
    assert xd.data_ptr() % 16 == 4 and wd.data_ptr() % 16 == 4
    logits = torch.full((T, E), float("nan"), device=dev)
    moe.moe_router_logits(xd, wd, logits)
    torch.cuda.synchronize()
    rows = np.arange(min(T, 64))
    got = host(logits).astype(np.float64)[rows]
    xs, wn = x.float().numpy()[rows], w.numpy()
    ref = oracle.router_logits(xs, wn, threads=THREADS)
    bound = H * 2.0 ** -24 * (np.abs(xs).astype(np.float64) @ np.abs(wn).astype(np.float64).T)
    assert (np.abs(got - ref) <= bound + 1e-30).all()
