"""GPU parity of the HIP path (through the C ABI) against the oracle, at
sizes the oracle finishes in seconds: several tiles, ragged tails, and the
degenerate routings of the method."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_02_amd as moe
import workload
from _parity import (TOL, check_end_to_end, device, forward, host, inputs_on_host, normwise,
                     stage_checks)

pytestmark = pytest.mark.gpu


# Paths of forward(): "fast" = the default buffers (dispatch indices only, the
# expert GEMM gathering rows from x, combine folding in the identity experts:
# moe_expert_ffn_gather + moe_combine_identity); "stages" = every stage's
# buffer kept (grouped copy x_perm, y_acc: moe_expert_ffn, moe_zero_experts,
# moe_combine).
PATHS = {"fast": {}, "stages": {"grouped_copy": True, "separate_identity": True}}


def _run(cfg, bias=None, path="fast"):
    dev = device()
    print(f"\n[case] {cfg} path={path}", flush=True)
    inp = workload.make_inputs(cfg, dev)
    if bias is not None:
        inp["bias"] = torch.as_tensor(bias, dtype=torch.float32, device=dev)
    buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev,
                            **PATHS[path])
    forward(cfg, inp, buf)
    return inp, buf


def _e2e(cfg, inp, buf, tokens=None):
    h = inputs_on_host(inp)
    err, flips = check_end_to_end(cfg, h["x"], h["w_router"], h["bias"], h["w13"], h["w2"],
                                  host(buf["y"]), host(buf["topk_idx"]), tokens)
    print(f"end-to-end normwise {err:.3e}, flipped tokens {flips}", flush=True)
    assert err <= TOL[cfg.dtype]
    return err


@pytest.mark.parametrize("N,Z,base", [(16, 0, "tiny_fp32"), (0, 16, "tiny_fp32"),
                                      (24, 0, "mid_bf16"), (0, 24, "mid_bf16")])
@pytest.mark.parametrize("path", list(PATHS))
def test_pool_of_one_expert_kind(N, Z, base, path):
    """Degenerate pools: FFN experts only (an ordinary MoE layer, Z = 0) and
    zero-computation experts only (N = 0: no FFN rows, the expert GEMMs
    enqueue nothing and y = x times the summed gates)."""
    cfg = workload.CONFIGS[base].replace(N=N, Z=Z, T=200)
    inp, buf = _run(cfg, path=path)
    S = int(host(buf["offsets"])[-1])
    assert S == (200 * cfg.K if Z == 0 else 0)
    if N == 0:
        g = host(buf["topk_gate"]).astype(np.float64).sum(1)
        ref = inputs_on_host(inp)["x"].astype(np.float64) * g[:, None]
        assert normwise(host(buf["y"]), ref) <= TOL[cfg.dtype]
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("path", list(PATHS))
def test_tiny_fp32_layer(path):
    cfg = workload.CONFIGS["tiny_fp32"]
    inp, buf = _run(cfg, path=path)
    print(stage_checks(cfg, inp, buf))
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("path", list(PATHS))
def test_mid_bf16_layer(path):
    cfg = workload.CONFIGS["mid_bf16"]
    inp, buf = _run(cfg, path=path)
    counts = host(buf["counts"])[:cfg.N]
    order = np.argsort(counts)
    experts = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    print(stage_checks(cfg, inp, buf, ffn_experts=experts))
    tokens = np.r_[0:24, cfg.T - 24:cfg.T, np.random.default_rng(0).choice(cfg.T, 48, False)]
    _e2e(cfg, inp, buf, np.unique(tokens))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 63, 65, 333])
def test_ragged_token_counts(T, dtype):
    cfg = workload.MoEConfig("ragged", T=T, H=256, N=8, Z=4, I=128, K=3, dtype=dtype,
                             sigma_w=0.05, bias_lo=-0.1, bias_hi=0.1, scale=1.5)
    inp, buf = _run(cfg)
    stage_checks(cfg, inp, buf)
    _e2e(cfg, inp, buf)


def test_multi_tile_experts_bf16():
    # ~660 rows per FFN expert: several 256-row m-tiles and a ragged last one
    cfg = workload.MoEConfig("multitile", T=2000, H=384, N=4, Z=2, I=192, K=2, dtype="bf16",
                             sigma_w=0.05, bias_lo=-0.01, bias_hi=0.01, scale=1.0)
    inp, buf = _run(cfg)
    assert host(buf["counts"])[:cfg.N].max() > 512
    stage_checks(cfg, inp, buf)
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("path", list(PATHS))
def test_multi_tile_experts_full_tile_kernel_bf16(path):
    # hidden 512 and intermediate 256 are shapes the full-tile kernel takes:
    # ~660 rows per FFN expert give two full 256-row m-tiles (K sweeps of 8
    # steps for gate/up, 4 for down: one six-step pass plus a tail, and a
    # tail alone) and a ragged partial one, through both dispatch paths
    cfg = workload.MoEConfig("multitile_full", T=2000, H=512, N=4, Z=2, I=256, K=2, dtype="bf16",
                             sigma_w=0.05, bias_lo=-0.01, bias_hi=0.01, scale=1.0)
    inp, buf = _run(cfg, path=path)
    assert host(buf["counts"])[:cfg.N].max() > 512
    stage_checks(cfg, inp, buf)
    _e2e(cfg, inp, buf)


def test_k_equals_e_picks_every_expert():
    cfg = workload.MoEConfig("k_eq_e", T=70, H=128, N=5, Z=3, I=64, K=8, dtype="bf16",
                             sigma_w=0.05, bias_lo=-0.1, bias_hi=0.1, scale=1.0)
    inp, buf = _run(cfg)
    stage_checks(cfg, inp, buf)
    assert (host(buf["counts"]) == cfg.T).all()
    np.testing.assert_allclose(host(buf["topk_gate"]).sum(1), 1.0, atol=1e-5)
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("path", list(PATHS))
def test_more_than_64_picks_per_token(path):
    # K = 70 of E = 96: the routing kernel writes its picks in two chunks of
    # lanes (64 + 6), and combine takes its general kernel (K > 16)
    cfg = workload.MoEConfig("k70", T=50, H=128, N=64, Z=32, I=64, K=70, dtype="bf16",
                             sigma_w=0.05, bias_lo=-0.1, bias_hi=0.1, scale=1.25)
    inp, buf = _run(cfg, path=path)
    stage_checks(cfg, inp, buf)
    assert host(buf["counts"]).sum() == cfg.T * cfg.K
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("path", list(PATHS))
def test_rows_wider_than_one_pass(path):
    # H = 8320 > 8 x 1024: combine loops over the row (its one-piece-per-thread
    # kernel takes rows of at most 8192)
    cfg = workload.MoEConfig("h8320", T=20, H=8320, N=4, Z=2, I=64, K=3, dtype="bf16",
                             sigma_w=0.01, bias_lo=-0.1, bias_hi=0.1, scale=1.0)
    inp, buf = _run(cfg, path=path)
    stage_checks(cfg, inp, buf)
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("T", [40, 300])
def test_largest_expert_pool(T):
    # E = 1024, the most the routing kernel takes: 16 keys per lane, a
    # 1024-bin pick histogram, 16 expert tiles in the router (T = 300) or 64
    # 16-expert blocks of the few-token router (T = 40).
    cfg = workload.MoEConfig("e1024", T=T, H=256, N=768, Z=256, I=128, K=12, dtype="bf16",
                             sigma_w=0.05, bias_lo=-0.1, bias_hi=0.1, scale=1.0)
    inp, buf = _run(cfg)
    stage_checks(cfg, inp, buf)
    counts = host(buf["counts"])
    assert counts.sum() == cfg.T * cfg.K and counts.max() <= cfg.T
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("path", list(PATHS))
def test_all_zero_expert_routing_returns_scaled_x(path):
    cfg = workload.MoEConfig("all_zero", T=130, H=256, N=6, Z=4, I=128, K=3, dtype="bf16",
                             sigma_w=0.05, bias_lo=0.0, bias_hi=0.0, scale=1.0)
    bias = np.zeros(cfg.E, np.float32)
    bias[cfg.N:] = 1e3
    inp, buf = _run(cfg, bias, path)
    assert (host(buf["topk_idx"]) >= cfg.N).all()
    assert int(host(buf["offsets"])[-1]) == 0
    assert (host(buf["slot_row"]) == -1).all()
    x = host(inp["x"]).astype(np.float64)
    g = host(buf["topk_gate"]).astype(np.float64).sum(1, keepdims=True)
    assert normwise(host(buf["y"]), x * g) <= TOL["bf16"]
    _e2e(cfg, inp, buf)


@pytest.mark.parametrize("path", list(PATHS))
def test_all_ffn_routing_has_no_identity_term(path):
    cfg = workload.MoEConfig("all_ffn", T=130, H=256, N=6, Z=4, I=128, K=3, dtype="bf16",
                             sigma_w=0.05, bias_lo=0.0, bias_hi=0.0, scale=2.0)
    bias = np.zeros(cfg.E, np.float32)
    bias[cfg.N:] = -1e3
    inp, buf = _run(cfg, bias, path)
    assert (host(buf["topk_idx"]) < cfg.N).all()
    if buf["y_acc"] is not None:
        assert (host(buf["y_acc"]) == 0).all()
    stage_checks(cfg, inp, buf)
    _e2e(cfg, inp, buf)


def test_route_ties_signed_zero_and_masking_are_bit_exact():
    dev = device()
    rng = np.random.default_rng(11)
    T, E, K = 200, 96, 8
    # quantised logits: many exact ties; signed zeros; some masked experts
    l = (rng.integers(-4, 5, (T, E)) * 0.125).astype(np.float32)
    l[l == 0] = np.where(rng.random((l == 0).sum()) < 0.5, -0.0, 0.0)
    b = np.zeros(E, np.float32)
    b[rng.choice(E, 10, False)] = -np.inf
    lt = torch.from_numpy(l).to(dev)
    bt = torch.from_numpy(b).to(dev)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)
    moe.moe_route(lt, bt, K, idx, gate, counts, status)
    torch.cuda.synchronize()
    i_ref, g_ref, c_ref = oracle.route(l, b, K)
    np.testing.assert_array_equal(host(idx), i_ref)
    np.testing.assert_array_equal(host(counts), c_ref)
    assert normwise(host(gate), g_ref) <= 1e-6
    assert int(host(status)[0]) == 0
    # K beyond the unmasked experts: masked ones follow, lowest id first
    moe.moe_route(lt, bt, 90, torch.empty((T, 90), dtype=torch.int32, device=dev),
                  torch.empty((T, 90), dtype=torch.float32, device=dev), counts, status)
    torch.cuda.synchronize()
    assert int(host(status)[0]) == 0


def test_route_flags_nan_keys():
    dev = device()
    l = torch.zeros((4, 24), dtype=torch.float32, device=dev)
    l[2, 5] = float("nan")
    b = torch.zeros(24, dtype=torch.float32, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)
    moe.moe_route(l, b, 4, torch.empty((4, 4), dtype=torch.int32, device=dev),
                  torch.empty((4, 4), dtype=torch.float32, device=dev),
                  torch.empty(24, dtype=torch.int32, device=dev), status)
    torch.cuda.synchronize()
    assert int(host(status)[0]) == 1


def _route(l, b, K, status=None):
    dev = device()
    T, E = l.shape
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev) if status is None else status
    moe.moe_route(torch.from_numpy(l).to(dev), torch.from_numpy(b).to(dev), K, idx, gate, counts,
                  status)
    torch.cuda.synchronize()
    return host(idx), host(gate), host(counts), int(host(status)[0])


def test_route_minus_inf_logits_are_masked_experts():
    # A -inf logit (or key) is a masked expert, not an error: it is never
    # picked before a finite key, and its gate is 0 when K exceeds the
    # unmasked experts.  Full pool (768 experts, K = 12), both selection
    # paths: a token with 5 finite logits takes masked experts by lowest id.
    rng = np.random.default_rng(21)
    T, E, K = 150, 768, 12
    l = (rng.standard_normal((T, E)) * 0.5).astype(np.float32)
    l[rng.random((T, E)) < 0.3] = -np.inf
    l[7] = -np.inf
    l[7, [3, 100, 400, 700, 767]] = [0.1, -0.2, 0.3, 0.0, 1.0]
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, gate, counts, status = _route(l, b, K)
    i_ref, g_ref, c_ref = oracle.route(l, b, K)
    np.testing.assert_array_equal(idx, i_ref)
    np.testing.assert_array_equal(counts, c_ref)
    assert normwise(gate, g_ref) <= 1e-6
    assert (gate[7, 5:] == 0).all() and status == 0


def test_route_flags_undefined_softmax():
    # +inf logit, NaN logit, or every logit -inf: the gates are undefined
    for case in ("+inf", "nan", "all -inf"):
        l = np.zeros((4, 24), np.float32)
        if case == "+inf":
            l[1, 3] = np.inf
        elif case == "nan":
            l[2, 5] = np.nan
        else:
            l[3, :] = -np.inf
        _, _, _, status = _route(l, np.zeros(24, np.float32), 4)
        assert status == 1, case
    # -inf on some experts only, and a -inf bias: no flag
    l = np.zeros((4, 24), np.float32)
    l[0, :20] = -np.inf
    b = np.zeros(24, np.float32)
    b[21] = -np.inf
    _, _, _, status = _route(l, b, 4)
    assert status == 0


def test_permute_rows_stay_in_bounds_with_inconsistent_counts():
    # counts that are not the histogram of topk_idx give a meaningless
    # grouping, but every row written stays inside [0, T*K)
    dev = device()
    T, E, N, K = 300, 96, 64, 8
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    it = torch.from_numpy(idx).to(dev)
    x = torch.zeros((T, 256), dtype=torch.bfloat16, device=dev)
    for bad in (np.zeros(E, np.int32), np.full(E, 1 << 20, np.int32)):
        offsets = torch.empty(N + 1, dtype=torch.int32, device=dev)
        row_src = torch.full((T * K + 64,), -7, dtype=torch.int32, device=dev)
        slot_row = torch.empty(T * K, dtype=torch.int32, device=dev)
        moe.moe_permute(x, it, torch.from_numpy(bad).to(dev), N, offsets, None, row_src,
                        slot_row)
        torch.cuda.synchronize()
        sr = host(slot_row)
        assert ((sr == -1) | ((sr >= 0) & (sr < T * K))).all()
        assert (sr == -1).sum() == (idx >= N).sum()
        assert (host(row_src)[T * K:] == -7).all()


def test_forward_is_bitwise_deterministic():
    cfg = workload.CONFIGS["mid_bf16"].replace(T=1024)
    inp, buf = _run(cfg)
    y1 = buf["y"].clone()
    yp1 = buf["y_perm"].clone()
    forward(cfg, inp, buf)
    assert torch.equal(buf["y"], y1)
    S = int(host(buf["offsets"])[-1])
    assert torch.equal(buf["y_perm"][:S], yp1[:S])


@pytest.mark.parametrize("path", list(PATHS))
def test_rows_past_the_grouped_rows_are_untouched(path):
    cfg = workload.CONFIGS["tiny_fp32"].replace(T=100)
    dev = device()
    inp = workload.make_inputs(cfg, dev)
    buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev,
                            **PATHS[path])
    grouped_copy = buf["x_perm"] is not None
    if grouped_copy:
        buf["x_perm"].fill_(123.0)
    buf["y_perm"].fill_(-7.0)
    buf["row_src"].fill_(-5)
    forward(cfg, inp, buf)
    S = int(host(buf["offsets"])[-1])
    assert S < cfg.T * cfg.K
    if grouped_copy:
        assert (host(buf["x_perm"][S:]) == 123.0).all()
    assert (host(buf["y_perm"][S:]) == -7.0).all()
    assert (host(buf["row_src"][S:]) == -5).all()


@pytest.mark.parametrize("T,H,I,heavy,boost", [(4000, 256, 128, (0, 1), 1.5),
                                               (2000, 640, 320, (2,), 6.0)])
def test_heavy_experts_many_m_tiles(T, H, I, heavy, boost):
    # Experts with 8-16 m-tiles of 256 rows next to light ones.  Case 1: two
    # experts with ~3000 rows each (12 m-tiles, a ragged last one) and 2
    # column tiles per GEMM.  Case 2: one expert with 2000 rows (8 m-tiles,
    # the last of 208 rows) and 5 column tiles.
    N, Z, K = 6, 2, len(heavy) if len(heavy) > 1 else 2
    cfg = workload.MoEConfig("heavy", T=T, H=H, N=N, Z=Z, I=I, K=K, dtype="bf16", sigma_w=0.05,
                             bias_lo=0.0, bias_hi=0.0, scale=1.25)
    bias = np.zeros(N + Z, np.float32)
    bias[list(heavy)] = boost
    inp, buf = _run(cfg, bias)
    counts = host(buf["counts"])[:N]
    print("rows per FFN expert", counts.tolist(), flush=True)
    assert all(counts[e] >= 7 * 256 + 1 for e in heavy)
    assert any(counts[e] < 8 * 256 for e in range(N) if e not in heavy)
    stage_checks(cfg, inp, buf)
    _e2e(cfg, inp, buf)


def test_two_stream_forward_matches_serial():
    # For large batches forward() runs the identity experts on a second
    # stream; combine must wait for them.  Two different batches alternate and
    # y_acc is poisoned before every call, so a combine that read y_acc early
    # would see NaN or the other batch's values.
    cfg = workload.CONFIGS["mid_bf16"].replace(T=2048)
    assert cfg.T >= moe.OVERLAP_MIN_TOKENS
    dev = device()
    inps = [workload.make_inputs(cfg.replace(seed=s), dev) for s in (0, 1)]
    buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev,
                            separate_identity=True)

    def run(fn, inp):
        buf["y_acc"].fill_(float("nan"))
        y = fn(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K, cfg.scale,
               buf)
        return y.clone()

    ref = [run(moe.forward_serial, inp) for inp in inps]
    for _ in range(3):
        for i, inp in enumerate(inps):
            got = run(moe.forward, inp)
            torch.cuda.synchronize()
            assert torch.equal(got, ref[i])
    assert not torch.equal(ref[0], ref[1])


@pytest.mark.parametrize("name,T,heavy", [("tiny_fp32", None, None), ("mid_bf16", 1500, None),
                                          ("mid_bf16", 1200, (3,))])
def test_row_gather_matches_grouped_copy(name, T, heavy):
    # The expert GEMM reading x[row_src // K] must give the same bits as the
    # GEMM on the grouped copy: same rows, same kernels, same order.  The
    # third case sends ~1100 rows to one expert (full 256-row tiles).
    cfg = workload.CONFIGS[name]
    if T is not None:
        cfg = cfg.replace(T=T)
    dev = device()
    inp = workload.make_inputs(cfg, dev)
    if heavy is not None:
        bias = np.zeros(cfg.E, np.float32)
        bias[list(heavy)] = 4.0
        inp["bias"] = torch.as_tensor(bias, device=dev)
    out = {}
    for copy in (True, False):
        buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev,
                                grouped_copy=copy)
        forward(cfg, inp, buf)
        S = int(host(buf["offsets"])[-1])
        out[copy] = (buf["y_perm"][:S].clone(), buf["y"].clone(), host(buf["counts"]))
    if heavy is not None:
        assert out[True][2][heavy[0]] > 4 * 256
    assert torch.equal(out[True][0], out[False][0])
    assert torch.equal(out[True][1], out[False][1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_row_gather_clamps_out_of_range_sources(dtype):
    # row_src entries outside [0, T*K) read a clamped token row of x, never
    # past it: compare with moe_expert_ffn on x_perm built from the same
    # clamped rows.
    T, K, H, I, N = 40, 3, 256, 128, 4
    dev = device()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn(T, H, generator=g).to(td).to(dev)
    w13 = (torch.randn(N, 2 * I, H, generator=g) * 0.05).to(td).to(dev)
    w2 = (torch.randn(N, H, I, generator=g) * 0.05).to(td).to(dev)
    rows_cap = T * K
    S = 90
    offsets = torch.tensor([0, 30, 30, 75, S], dtype=torch.int32, device=dev)
    rs = torch.randint(0, T * K, (rows_cap,), generator=g, dtype=torch.int32)
    rs[[0, 7, 31, 60, 89]] = torch.tensor([-1, -(2 ** 31), T * K, 2 ** 31 - 1, T * K + 5],
                                          dtype=torch.int32)
    tok = (rs.clamp(min=0).long() // K).clamp(max=T - 1)
    rs = rs.to(dev)
    x_perm = x[tok.to(dev)].contiguous()
    ws = torch.empty(moe.moe_expert_ffn_workspace_bytes(rows_cap, N, I, td), dtype=torch.uint8,
                     device=dev)
    y_ref = torch.zeros(rows_cap, H, dtype=td, device=dev)
    y_got = torch.zeros(rows_cap, H, dtype=td, device=dev)
    moe.moe_expert_ffn(x_perm, offsets, w13, w2, y_ref, ws)
    moe.moe_expert_ffn_gather(x, K, rs, offsets, w13, w2, y_got, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_got[:S], y_ref[:S])
    assert (host(y_got[S:]) == 0).all()


@pytest.mark.parametrize("name,T,zero_bias", [("tiny_fp32", None, 0.0), ("mid_bf16", 2048, 0.0),
                                              ("mid_bf16", 65, 0.0), ("mid_bf16", 300, 50.0),
                                              ("mid_bf16", 300, -50.0)])
def test_combine_identity_matches_six_calls(name, T, zero_bias):
    # moe_combine_identity computes the identity experts' term inside combine
    # with the fp32 operations of moe_zero_experts + moe_combine, so y must
    # be bitwise equal.  T = 2048 puts the six-call path on its two streams;
    # a bias of +50 / -50 on the identity experts routes every pick to them /
    # none of them (an empty / a full FFN slot list).
    cfg = workload.CONFIGS[name]
    if T is not None:
        cfg = cfg.replace(T=T)
    dev = device()
    inp = workload.make_inputs(cfg, dev)
    if zero_bias:
        bias = np.zeros(cfg.E, np.float32)
        bias[cfg.N:] = zero_bias
        inp["bias"] = torch.as_tensor(bias, device=dev)
    ys = {}
    for sep in (False, True):
        buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev,
                                separate_identity=sep)
        assert (buf["y_acc"] is None) == (not sep)
        forward(cfg, inp, buf)
        ys[sep] = buf["y"].clone()
    S = int(host(buf["offsets"])[-1])
    if zero_bias > 0:
        assert S == 0
    if zero_bias < 0:
        assert S == cfg.T * cfg.K
    assert torch.equal(ys[False], ys[True])
    if zero_bias == 0.0 and name == "mid_bf16" and T == 65:
        _e2e(cfg, inp, buf)
