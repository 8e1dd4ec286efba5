"""Router scores on the matrix cores against the oracle, element by element,
at shapes that select each kernel: the wide 256-token x 96-expert tiles (at
least 256 of them), the 128 x 64 tiles, and the few-token kernel -- with
ragged token and expert counts, expert counts that are not a multiple of 4
(scalar stores), and a hidden size with an odd number of 32-element K steps
(the K sweeps start at two offsets and wrap around)."""
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
def test_router_logits_match_oracle(T, E, H):
    dev = device()
    print(f"\n[case] router T={T} E={E} H={H}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(T * 31 + E)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.randn(E, H, generator=g) * 0.02
    logits = torch.full((T, E), float("nan"), device=dev)
    moe.moe_router_logits(x.to(dev), w.to(dev), logits)
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
