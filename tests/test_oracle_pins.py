"""Pins of the oracle against things other than itself.

Each test checks one oracle stage against a library routine, a closed form,
an invariant, a special case or brute force -- never against a retyped copy
of the oracle's own loops -- chosen so that a dropped term, a wrong sign or
index, or a transposed operand fails at least one of them.  The numbers the
pages print are in tests/golden/longcat_flash_shapes.txt.
"""
import os

import numpy as np
import pytest
import scipy.special as sp

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _golden_shapes():
    out = {}
    with open(os.path.join(GOLDEN, "longcat_flash_shapes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = float(v)
    return out


# ------------------------------------------------------------------ logits --

def test_logits_match_blas_fp64():
    r = _rng(1)
    x = r.standard_normal((37, 200)).astype(np.float32)
    wr = (r.standard_normal((29, 200)) * 0.05).astype(np.float32)
    got = oracle.router_logits(x, wr)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T     # BLAS, other order
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # the threaded front-end splits rows only
    np.testing.assert_array_equal(oracle.router_logits(x, wr, threads=4), got)


def test_logits_transposition_detected():
    # a non-square case where x @ wr and wr @ x.T cannot be confused
    x = np.arange(6, dtype=np.float32).reshape(2, 3)
    wr = np.array([[1, 0, 0], [0, 0, 2], [1, 1, 1], [0, -1, 0]], np.float32)
    got = oracle.router_logits(x, wr)
    np.testing.assert_array_equal(got, [[0, 4, 3, -1], [3, 10, 12, -4]])


# ------------------------------------------------------------------ top-K ----

def _lib_topk(logits32, bias, K):
    key = (logits32 + bias[None, :]).astype(np.float32)   # one fp32 add, like the oracle
    return np.argsort(-key, axis=1, kind="stable")[:, :K].astype(np.int32)


@pytest.mark.parametrize("T,E,K", [(50, 24, 4), (33, 96, 8), (9, 768, 12), (5, 7, 7), (4, 1, 1)])
def test_topk_matches_stable_sort(T, E, K):
    r = _rng(T * E + K)
    l = r.standard_normal((T, E)).astype(np.float32)
    b = r.uniform(-0.1, 0.1, E).astype(np.float32)
    idx, gate, counts = oracle.route(l, b, K)
    np.testing.assert_array_equal(idx, _lib_topk(l, b, K))


def test_topk_ties_pick_lower_index():
    # quantised keys make many exact ties
    r = _rng(7)
    l = (r.integers(-3, 4, (64, 40)) * 0.25).astype(np.float32)
    b = np.zeros(40, np.float32)
    idx, _, _ = oracle.route(l, b, 6)
    np.testing.assert_array_equal(idx, _lib_topk(l, b, 6))
    # all keys equal -> experts 0..K-1 in order
    idx, _, _ = oracle.route(np.zeros((3, 10), np.float32), np.zeros(10, np.float32), 4)
    np.testing.assert_array_equal(idx, np.tile(np.arange(4), (3, 1)))


def test_topk_signed_zero_is_a_tie():
    l = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    idx, _, _ = oracle.route(l, np.zeros(4, np.float32), 3)
    np.testing.assert_array_equal(idx, [[0, 1, 3]])
    l = np.array([[0.0, -0.0, -0.0, 1.0]], np.float32)
    idx, _, _ = oracle.route(l, np.zeros(4, np.float32), 3)
    np.testing.assert_array_equal(idx, [[3, 0, 1]])


def test_topk_minus_inf_masks_and_nan_raises():
    l = np.array([[0.5, 0.1, 0.9, 0.3, 0.2]], np.float32)
    b = np.array([0, -np.inf, -np.inf, 0, 0], np.float32)
    idx, gate, _ = oracle.route(l, b, 4)
    # finite keys first in key order, then the masked ones by ascending id
    np.testing.assert_array_equal(idx, [[0, 3, 4, 1]])
    # the gate still comes from the unbiased logit of the masked expert
    np.testing.assert_allclose(gate[0, 3], sp.softmax(l[0].astype(np.float64))[1], rtol=1e-14)
    with pytest.raises(oracle.OracleError):
        oracle.route(np.array([[0.0, np.nan, 1.0]], np.float32), np.zeros(3, np.float32), 1)


def test_key_is_an_fp32_sum():
    # 1 + 2**-24 rounds to 1 in fp32: the two keys tie and the lower id wins,
    # although the exact sums differ
    l = np.array([[1.0, 1.0]], np.float32)
    b = np.array([0.0, 2.0 ** -24], np.float32)
    idx, _, _ = oracle.route(l, b, 1)
    assert idx[0, 0] == 0
    b = np.array([0.0, 2.0 ** -23], np.float32)
    idx, _, _ = oracle.route(l, b, 1)
    assert idx[0, 0] == 1


# ------------------------------------------------------------------ gates ----

def test_gates_are_softmax_of_unbiased_logits():
    r = _rng(3)
    l = r.standard_normal((40, 24)).astype(np.float32)
    b = r.uniform(-2, 2, 24).astype(np.float32)     # large bias: selection moves, gates must not
    idx, gate, _ = oracle.route(l, b, 5)
    p = sp.softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(gate, np.take_along_axis(p, idx, 1), rtol=1e-13)
    assert (gate > 0).all() and (gate.sum(1) <= 1 + 1e-12).all()
    np.testing.assert_allclose(oracle.gates(l, idx), gate, rtol=0, atol=0)


def test_gates_sum_to_one_when_k_equals_e():
    r = _rng(4)
    l = (r.standard_normal((16, 24)) * 3).astype(np.float32)
    _, gate, _ = oracle.route(l, np.zeros(24, np.float32), 24)
    np.testing.assert_allclose(gate.sum(1), 1.0, rtol=0, atol=8 * np.finfo(np.float64).eps)


# ----------------------------------------------------------------- counts ----

def test_counts_are_the_histogram():
    r = _rng(5)
    T, E, K = 300, 96, 8
    l = r.standard_normal((T, E)).astype(np.float32)
    idx, _, counts = oracle.route(l, r.uniform(-0.1, 0.1, E).astype(np.float32), K)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert counts.sum() == T * K and counts.max() <= T
    assert all(len(set(row)) == K for row in idx.tolist())


# ---------------------------------------------------------------- permute ----

def test_permute_is_the_stable_sort_and_round_trips():
    r = _rng(6)
    T, E, K, N = 200, 24, 4, 16
    l = r.standard_normal((T, E)).astype(np.float32)
    idx, _, counts = oracle.route(l, np.zeros(E, np.float32), K)
    offsets, row_src, slot_row = oracle.permute(idx, N)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(row_src, order[flat[order] < N])
    np.testing.assert_array_equal(np.diff(offsets), counts[:N])
    assert offsets[0] == 0 and offsets[N] == row_src.size == (flat < N).sum()
    # round trip: every FFN slot maps to a row that maps back to it
    ffn = np.nonzero(flat < N)[0]
    np.testing.assert_array_equal(row_src[slot_row[ffn]], ffn)
    assert (slot_row[flat >= N] == -1).all()
    x = r.standard_normal((T, 8)).astype(np.float32)
    x_perm = x[row_src // K]
    np.testing.assert_array_equal(x_perm[slot_row[ffn]], x[ffn // K])


def test_permute_empty_and_all_one_expert():
    idx = np.full((5, 1), 3, np.int32)          # every token on the identity expert 3 (N = 3)
    offsets, row_src, slot_row = oracle.permute(idx, 3)
    assert row_src.size == 0 and (offsets == 0).all() and (slot_row == -1).all()
    idx = np.full((5, 1), 1, np.int32)
    offsets, row_src, slot_row = oracle.permute(idx, 3)
    np.testing.assert_array_equal(offsets, [0, 0, 5, 5])
    np.testing.assert_array_equal(row_src, np.arange(5))


# -------------------------------------------------------------------- FFN ----

def test_ffn_closed_form_unit_vectors():
    # I != H so a transposed w2 or swapped gate/up rows change the answer
    H, I = 8, 3
    a, b, c = [1, 6, 3], [2, 2, 7], [5, 0, 4]
    al, be, ga = [1.5, -2.0, 0.75], [0.5, 3.0, -1.25], [2.0, -0.5, 4.0]
    w13 = np.zeros((2 * I, H), np.float32)
    w2 = np.zeros((H, I), np.float32)
    for j in range(I):
        w13[j, a[j]] = al[j]
        w13[I + j, b[j]] = be[j]
        w2[c[j], j] = ga[j]
    x = np.array([0.3, -1.1, 2.0, 0.7, -0.4, 1.3, -2.5, 0.9], np.float32)
    expect = np.zeros(H)
    for j in range(I):
        g = al[j] * np.float64(x[a[j]])
        expect[c[j]] += ga[j] * (g * sp.expit(g)) * (be[j] * np.float64(x[b[j]]))
    np.testing.assert_allclose(oracle.ffn_row(x, w13, w2), expect, rtol=1e-14, atol=1e-15)


def test_ffn_silu_values():
    # one unit of intermediate: out[0] = silu(x0) * x1
    w13 = np.array([[1, 0], [0, 1]], np.float32)
    w2 = np.array([[1], [0]], np.float32)
    for x0, ref in [(0.0, 0.0), (2.0, 2 * sp.expit(2.0)), (-3.0, -3 * sp.expit(-3.0)),
                    (30.0, 30 * sp.expit(30.0)), (-60.0, -60 * sp.expit(-60.0))]:
        out = oracle.ffn_row(np.array([x0, 1.0], np.float32), w13, w2)
        np.testing.assert_allclose(out, [ref, 0.0], rtol=1e-14, atol=1e-300)


def test_ffn_linearity_properties():
    r = _rng(8)
    H, I = 24, 10
    x = r.standard_normal(H).astype(np.float32)
    w13 = (r.standard_normal((2 * I, H)) * 0.3).astype(np.float32)
    # dyadic values so w2a + w2b is exact in fp32
    w2a = (r.integers(-8, 9, (H, I)) / 16).astype(np.float32)
    w2b = (r.integers(-8, 9, (H, I)) / 16).astype(np.float32)
    fa, fb = oracle.ffn_row(x, w13, w2a), oracle.ffn_row(x, w13, w2b)
    np.testing.assert_allclose(oracle.ffn_row(x, w13, w2a + w2b), fa + fb, rtol=1e-12, atol=1e-14)
    up0 = w13.copy()
    up0[I:] = 0
    assert (oracle.ffn_row(x, up0, w2a) == 0).all()
    up2 = w13.copy()
    up2[I:] *= 2
    np.testing.assert_array_equal(oracle.ffn_row(x, up2, w2a), 2 * fa)


# ------------------------------------------------- zero experts / combine ----

def _tiny(seed=0, T=48, H=32, N=6, Z=3, I=8, K=3):
    r = _rng(seed)
    x = r.standard_normal((T, H)).astype(np.float32)
    wr = (r.standard_normal((N + Z, H)) * 0.2).astype(np.float32)
    b = r.uniform(-0.1, 0.1, N + Z).astype(np.float32)
    w13 = (r.standard_normal((N, 2 * I, H)) * 0.2).astype(np.float32)
    w2 = (r.standard_normal((N, H, I)) * 0.2).astype(np.float32)
    return x, wr, b, w13, w2, K


def _brute_force(x, wr, b, w13, w2, K, s, sel=None):
    """Per token, loop over every expert of the pool with weight 0 for the
    unpicked ones.  Library pieces: BLAS matmul, a stable sort, scipy's
    softmax and logistic function.  sel [T, K]: the experts each token
    keeps (default: the top K of the fp32 keys)."""
    N = w13.shape[0]
    I = w2.shape[2]
    E = wr.shape[0]
    l32 = (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)
    if sel is None:
        sel = _lib_topk(l32, b, K)
    p = sp.softmax(l32.astype(np.float64), axis=1)
    y = np.zeros(x.shape, np.float64)
    for t in range(x.shape[0]):
        xt = x[t].astype(np.float64)
        for e in range(E):
            w = p[t, e] if e in sel[t] else 0.0
            if e < N:
                g = w13[e, :I].astype(np.float64) @ xt
                u = w13[e, I:].astype(np.float64) @ xt
                f = w2[e].astype(np.float64) @ (g * sp.expit(g) * u)
                y[t] += s * w * f
            else:
                y[t] += w * xt
    return y


@pytest.mark.parametrize("seed,s", [(0, 1.0), (1, 2.0), (2, 0.37)])
def test_layer_matches_brute_force(seed, s):
    x, wr, b, w13, w2, K = _tiny(seed)
    got = oracle.layer(x, wr, b, w13, w2, K, s)["y"]
    ref = _brute_force(x, wr, b, w13, w2, K, s)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def _swept_shapes(n=16, seed=11):
    """Random small pools: T, H, N (0 allowed), Z (0 allowed), I, K (up to
    E), compensation scale; a fixed list, so a failure names its case."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        N, Z = int(r.integers(0, 9)), int(r.integers(0, 6))
        if N + Z == 0:
            continue
        out.append(dict(seed=int(r.integers(0, 10**6)), T=int(r.integers(1, 40)),
                        H=int(r.integers(1, 24)), N=N, Z=Z, I=int(r.integers(1, 10)),
                        K=int(r.integers(1, N + Z + 1)), s=float(np.round(r.uniform(0.1, 3.0), 3))))
    return out


@pytest.mark.parametrize("c", _swept_shapes(),
                         ids=lambda c: "T{T}-H{H}-N{N}-Z{Z}-I{I}-K{K}".format(**c))
def test_layer_matches_brute_force_on_swept_shapes(c):
    # Technical Report notes, Key claims [§2.1, §2.3.2]: the layer output is
    # the gate-weighted sum over the kept experts of the pool, FFN outputs
    # scaled by the compensation factor; brute force loops over the whole
    # pool with weight 0 for the experts a token does not keep.
    x, wr, b, w13, w2, K = _tiny(c["seed"], T=c["T"], H=c["H"], N=c["N"], Z=c["Z"], I=c["I"],
                                 K=c["K"])
    got = oracle.layer(x, wr, b, w13, w2, K, c["s"])
    ref = _brute_force(x, wr, b, w13, w2, K, c["s"])
    np.testing.assert_allclose(got["y"], ref, rtol=0, atol=1e-12 * max(np.abs(ref).max(), 1e-30))
    # counts sum to T*K over the pool, and the FFN rows are the FFN picks
    assert int(got["counts"].sum()) == c["T"] * K
    assert int(got["offsets"][-1]) == int((got["idx"] < c["N"]).sum())


def test_layer_with_routing_on_the_oracles_own_choice_is_the_layer():
    # the flip-rule reference row, fed the choice the oracle made itself,
    # must be the oracle's layer output bit for bit
    x, wr, b, w13, w2, K = _tiny(7)
    ref = oracle.layer(x, wr, b, w13, w2, K, 1.3)
    got = oracle.layer_with_routing(x, ref["logits32"], ref["idx"], w13, w2, 1.3)
    np.testing.assert_array_equal(got, ref["y"])


def test_layer_with_routing_follows_a_swapped_expert_set():
    # Technical Report notes, Key claims [§2.1]: the output is the gate-weighted
    # sum over the experts a token keeps.  Swap, for some tokens, the K-th
    # pick for the first unpicked expert (an FFN expert for one token, an
    # identity expert for another) and compare with brute force over the
    # pool restricted to the swapped sets.
    x, wr, b, w13, w2, K = _tiny(8, T=20, N=6, Z=3, K=3)
    N = w13.shape[0]
    ref = oracle.layer(x, wr, b, w13, w2, K, 0.8)
    key = (ref["logits32"] + b[None, :]).astype(np.float32)
    sel = ref["idx"].copy()
    order = np.argsort(-key, axis=1, kind="stable")
    swapped_to = {}
    for t in range(x.shape[0]):
        nxt = order[t, K]                      # the best expert the token did not keep
        kind = "ffn" if nxt < N else "identity"
        if kind not in swapped_to:
            sel[t, K - 1] = nxt
            swapped_to[kind] = t
    assert set(swapped_to) == {"ffn", "identity"}
    got = oracle.layer_with_routing(x, ref["logits32"], sel, w13, w2, 0.8)
    want = _brute_force(x, wr, b, w13, w2, K, 0.8, sel=sel)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())
    # the swapped tokens really changed, the others did not
    for t in swapped_to.values():
        assert np.abs(got[t] - ref["y"][t]).max() > 1e-6
    keep = np.setdiff1d(np.arange(x.shape[0]), list(swapped_to.values()))
    np.testing.assert_array_equal(got[keep], ref["y"][keep])


def test_all_zero_expert_routing_returns_x_times_gate_sum():
    x, wr, b, w13, w2, K = _tiny(3)
    N = w13.shape[0]
    b = b.copy()
    b[N:] += 1e3                 # every pick lands on an identity expert (K <= Z)
    r = oracle.layer(x, wr, b, w13, w2, K, 1.0)
    assert (r["idx"] >= N).all() and r["row_src"].size == 0
    np.testing.assert_allclose(r["y"], x.astype(np.float64) * r["gate"].sum(1, keepdims=True),
                               rtol=1e-15, atol=0)


def test_all_ffn_routing_has_no_identity_term():
    x, wr, b, w13, w2, K = _tiny(4)
    N = w13.shape[0]
    b = b.copy()
    b[N:] -= 1e3
    r = oracle.layer(x, wr, b, w13, w2, K, 1.5)
    assert (r["idx"] < N).all() and (r["y_acc"] == 0).all()
    ref = _brute_force(x, wr, b, w13, w2, K, 1.5)
    np.testing.assert_allclose(r["y"], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_zero_scale_leaves_only_identity_experts():
    x, wr, b, w13, w2, K = _tiny(5)
    r = oracle.layer(x, wr, b, w13, w2, K, 0.0)
    np.testing.assert_array_equal(r["y"], r["y_acc"])
    N = w13.shape[0]
    gz = np.where(r["idx"] >= N, r["gate"], 0).sum(1, keepdims=True)
    np.testing.assert_allclose(r["y_acc"], gz * x.astype(np.float64), rtol=1e-15, atol=0)


def test_layer_is_deterministic():
    x, wr, b, w13, w2, K = _tiny(6)
    r1 = oracle.layer(x, wr, b, w13, w2, K, 1.0)
    r2 = oracle.layer(x, wr, b, w13, w2, K, 1.0, threads=3)
    for k in ("logits", "idx", "gate", "y_perm", "y"):
        np.testing.assert_array_equal(r1[k], r2[k])


# --------------------------------------------------- numbers on the pages ----

def test_config_shapes_match_the_pages():
    g = _golden_shapes()
    for name in ("prefill_bf16", "decode_bf16", "skewed_bf16"):
        c = workload.CONFIGS[name]
        assert (c.H, c.I, c.N, c.Z, c.K) == (g["hidden"], g["expert_intermediate"],
                                             g["ffn_experts"], g["zero_experts"], g["top_k"])


def test_activated_parameter_span_fixes_three_matrices_per_expert():
    """The activation span the pages print (18.6B..31.3B per token) is what
    the 12 picks of 28 layers add when they all land on FFN experts: it fixes
    the parameters of one expert at 3*H*I, i.e. the gate, up and down matrices
    the oracle's expert takes (a two-matrix FFN would give 8.5B)."""
    g = _golden_shapes()
    H, I = int(g["hidden"]), int(g["expert_intermediate"])
    # the parameter count of one expert as the oracle's expert consumes it
    w13 = np.zeros((2 * I, H), np.float32)
    w2 = np.zeros((H, I), np.float32)
    assert (oracle.ffn_row(np.ones(H, np.float32), w13, w2) == 0).all()
    per_expert = w13.size + w2.size
    span = g["layers"] * g["top_k"] * per_expert / 1e9
    assert abs(span - (g["activated_max_b"] - g["activated_min_b"])) < 0.05
    # and the average implies ~0.66 of picks on FFN experts
    share = (g["activated_avg_b"] - g["activated_min_b"]) / span
    assert abs(share - 0.662) < 0.002


def test_ffn_share_matches_the_pages_average():
    """With the full-scale router and bias reading (bias on fp32 logits), the
    share of picks landing on FFN experts is the ~0.66 the pages' average
    activation implies (27B between 18.6B and 31.3B)."""
    cfg = workload.CONFIGS["prefill_bf16"]
    x = workload.make_x(cfg, T=256).float().numpy()
    wr = workload.make_router(cfg).numpy()
    b = workload.make_bias(cfg).numpy()
    l32 = oracle.router_logits(x, wr, threads=os.cpu_count() or 1).astype(np.float32)
    idx, _, _ = oracle.route(l32, b, cfg.K)
    share = (idx < cfg.N).mean()
    assert abs(share - 0.662) < 0.025, share


# --------------------------------------------------------- bias controller --

def _counts_case():
    # 6 FFN experts + 3 identity experts; T = 40 tokens, K = 3 picks each
    counts = np.array([12, 30, 20, 0, 8, 10, 15, 10, 15], np.int32)
    assert counts.sum() == 40 * 3
    return counts, 40, 6


def test_bias_update_errors_sum_to_the_activation_gap():
    # summed over FFN experts the proportional step is kp * (target - FFN picks per token)
    counts, T, N = _counts_case()
    for target in (1.0, 2.0, 2.5):
        b, _, _ = oracle.bias_update(counts, T, N, target, 0.7, 0.0, 0.0, np.zeros(9),
                                     np.zeros(N), np.zeros(N))
        assert b[:N].sum() == pytest.approx(0.7 * (target - counts[:N].sum() / T), abs=1e-12)


def test_bias_update_pushes_against_the_load():
    counts, T, N = _counts_case()
    target = counts[:N].sum() / T          # on target in total: only the balance moves
    b, _, _ = oracle.bias_update(counts, T, N, target, 1.0, 0.0, 0.0, np.zeros(9), np.zeros(N),
                                 np.zeros(N))
    share = target / N
    load = counts[:N] / T
    assert np.all(np.sign(b[:N]) == -np.sign(load - share))   # overloaded down, idle up
    assert np.argmin(b[:N]) == np.argmax(load) and np.argmax(b[:N]) == np.argmin(load)


def test_bias_update_fixed_point_and_identity_experts_untouched():
    T, N = 64, 8
    counts = np.array([24] * N + [17, 99, 0], np.int32)       # every FFN expert at 24 / 64
    b0 = _rng(3).uniform(-0.3, 0.3, N + 3)
    b, integ, prev = oracle.bias_update(counts, T, N, 24 * N / T, 1.3, 0.4, 0.9, b0,
                                        np.zeros(N), np.zeros(N))
    np.testing.assert_array_equal(b, b0)                       # on target: nothing moves
    np.testing.assert_array_equal(integ, 0)
    counts[:N] = [40, 0, 30, 10, 20, 24, 24, 44]
    b, _, _ = oracle.bias_update(counts, T, N, 2.7, 1.3, 0.4, 0.9, b0, np.zeros(N), np.zeros(N))
    np.testing.assert_array_equal(b[N:], b0[N:])              # identity experts: never updated
    assert np.all(b[:N] != b0[:N])


def test_bias_update_integral_and_derivative_terms():
    counts, T, N = _counts_case()
    z = np.zeros(N)
    # integral only, constant counts: the n-th step is n times the first
    b, i, p = oracle.bias_update(counts, T, N, 2.0, 0.0, 0.3, 0.0, np.zeros(9), z, z)
    d1 = b[:N].copy()
    steps = [d1]
    for _ in range(3):
        nb, i, p = oracle.bias_update(counts, T, N, 2.0, 0.0, 0.3, 0.0, b, i, p)
        steps.append(nb[:N] - b[:N])
        b = nb
    for n, d in enumerate(steps, 1):
        np.testing.assert_allclose(d, n * d1, rtol=1e-12, atol=1e-15)
    # derivative only, constant counts: a kick on the first step, nothing after
    b, i, p = oracle.bias_update(counts, T, N, 2.0, 0.0, 0.0, 0.5, np.zeros(9), z, z)
    nb, _, _ = oracle.bias_update(counts, T, N, 2.0, 0.0, 0.0, 0.5, b, i, p)
    np.testing.assert_array_equal(nb, b)
    assert np.abs(b[:N]).max() > 0


@pytest.mark.parametrize("target", [2.0, 3.0])
def test_bias_controller_holds_the_activated_ffn_count(target):
    # Closed loop on the oracle's own router (tiny layer, K = 4 of 16 + 8):
    # the FFN picks per token settle at the target from either side of the
    # uncontrolled share (~2.59) and the FFN experts' loads even out.
    cfg = workload.CONFIGS["tiny_fp32"]
    x = workload.make_x(cfg).numpy()
    l32 = oracle.router_logits(x, workload.make_router(cfg).numpy()).astype(np.float32)
    T, N, K = cfg.T, cfg.N, cfg.K
    bias = workload.make_bias(cfg).numpy().astype(np.float64)
    integ, prev = np.zeros(N), np.zeros(N)
    hist = []
    for _ in range(200):
        _, _, counts = oracle.route(l32, bias.astype(np.float32), K)
        hist.append(counts[:N].sum() / T)
        bias, integ, prev = oracle.bias_update(counts, T, N, target, 1.0, 0.05, 0.2, bias, integ,
                                               prev)
    h = np.array(hist)
    assert abs(h[0] - 2.59) < 0.05
    assert abs(h[-50:].mean() - target) < 0.01 and np.abs(h[-50:] - target).max() < 0.05
    load = counts[:N] / T
    assert load.std() / load.mean() < 0.1


def test_bias_update_derivative_opposes_a_rising_load():
    # kd only: from a balanced batch (no error, no kick) to one where expert 0
    # takes more tokens and expert 1 fewer: expert 0's bias must fall, 1's rise.
    T, N = 32, 4
    z = np.zeros(N)
    bal = np.array([16, 16, 16, 16, 32], np.int32)
    b, i, p = oracle.bias_update(bal, T, N, 2.0, 0.0, 0.0, 0.8, np.zeros(5), z, z)
    np.testing.assert_array_equal(b, 0)
    moved = np.array([24, 8, 16, 16, 32], np.int32)
    nb, _, _ = oracle.bias_update(moved, T, N, 2.0, 0.0, 0.0, 0.8, b, i, p)
    assert nb[0] < 0 < nb[1] and nb[2] == nb[3] == 0


# ------------------------------------------------ router weight similarity --
# Pairwise cosine similarity of the experts' router weight rows, the router
# stability diagnostic (Technical Report notes, Key claims and Method
# [§3.1.3 Router Stability]).

def test_similarity_matches_scipy_cosine_distance():
    from scipy.spatial.distance import cdist
    w = _rng(60).standard_normal((23, 41)).astype(np.float32)
    sim, mean = oracle.router_similarity(w)
    ref = 1.0 - cdist(w.astype(np.float64), w.astype(np.float64), "cosine")
    np.testing.assert_allclose(sim, ref, rtol=0, atol=1e-12)
    off = ref[~np.eye(23, dtype=bool)]
    assert abs(mean - off.mean()) < 1e-12


def test_similarity_of_a_regular_simplex():
    # E unit vectors centred on their mean: every pair has cosine -1/(E-1),
    # rotated into a wider space so rows are not axis-aligned.
    E, H = 9, 30
    v = np.eye(E) - 1.0 / E
    q, _ = np.linalg.qr(_rng(61).standard_normal((H, H)))
    w = (v @ q[:E, :]).astype(np.float32)
    sim, mean = oracle.router_similarity(w)
    off = sim[~np.eye(E, dtype=bool)]
    np.testing.assert_allclose(off, -1.0 / (E - 1), atol=1e-6)
    np.testing.assert_allclose(np.diag(sim), 1.0, atol=1e-12)
    assert abs(mean + 1.0 / (E - 1)) < 1e-6


def test_similarity_orthogonal_and_identical_rows():
    q, _ = np.linalg.qr(_rng(62).standard_normal((16, 16)))
    sim, mean = oracle.router_similarity(q[:10].astype(np.float32))
    np.testing.assert_allclose(sim, np.eye(10), atol=1e-6)
    assert abs(mean) < 1e-6
    row = _rng(63).standard_normal(50).astype(np.float32)
    sim, mean = oracle.router_similarity(np.stack([row, 3 * row, 0.5 * row]))
    np.testing.assert_allclose(sim, 1.0, atol=1e-12)
    assert abs(mean - 1.0) < 1e-12


def test_similarity_scale_sign_and_zero_rows():
    w = _rng(64).standard_normal((12, 33)).astype(np.float32)
    sim, _ = oracle.router_similarity(w)
    w2 = w.copy()
    w2[3] *= 4.0    # exact in fp32
    w2[5] *= -1.0
    w2[7] = 0.0
    sim2, mean2 = oracle.router_similarity(w2)
    sign = np.ones(12)
    sign[5] = -1.0
    expect = sim * sign[:, None] * sign[None, :]
    expect[7, :] = 0.0
    expect[:, 7] = 0.0
    np.testing.assert_allclose(sim2, expect, atol=1e-12)
    assert abs(mean2 - expect[~np.eye(12, dtype=bool)].mean()) < 1e-12
    assert sim2[7, 7] == 0.0


def test_similarity_separates_collapsed_from_random_routers():
    r = _rng(65)
    E, H = 64, 256
    _, m_rand = oracle.router_similarity(r.standard_normal((E, H)).astype(np.float32))
    assert abs(m_rand) < 4.0 / np.sqrt(H) / np.sqrt(E)
    common = r.standard_normal(H)
    w = (common + 0.1 * r.standard_normal((E, H))).astype(np.float32)
    _, m_col = oracle.router_similarity(w)
    assert m_col > 0.95
    sim, mean = oracle.router_similarity(w[:1])
    assert sim.shape == (1, 1) and abs(sim[0, 0] - 1.0) < 1e-12 and mean == 0.0
