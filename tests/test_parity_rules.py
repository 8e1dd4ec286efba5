"""CPU checks of the parity rules the GPU tests apply (no GPU needed).

The end-to-end check lets a token keep a different expert set than the
oracle only when the oracle's top-K margin (K-th minus (K+1)-th fp32 key) is
below 1e-5, and then compares that token with the oracle's output for the set
the GPU chose.  These tests plant such flips in an oracle-made "GPU" result,
so the flip branch runs even though no GPU run has produced a flip.
"""
import types

import numpy as np
import pytest

import oracle
from _parity import FLIP_MARGIN, check_end_to_end, margins


def _layer(seed=11, T=40, H=32, N=6, Z=3, I=8, K=3):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H)).astype(np.float32)
    wr = (r.standard_normal((N + Z, H)) * 0.2).astype(np.float32)
    b = r.uniform(-0.1, 0.1, N + Z).astype(np.float32)
    w13 = (r.standard_normal((N, 2 * I, H)) * 0.2).astype(np.float32)
    w2 = (r.standard_normal((N, H, I)) * 0.2).astype(np.float32)
    return types.SimpleNamespace(K=K, scale=1.25), x, wr, b, w13, w2


def _near_tie(cfg, x, wr, b, t, gap):
    """Move the bias of token t's (K+1)-th expert so that its fp32 key sits
    `gap` below the K-th one (t keeps its picks).  Returns the new bias."""
    l32 = oracle.router_logits(x, wr).astype(np.float32)
    key = l32[t] + b
    order = np.argsort(-key, kind="stable")
    a, c = order[cfg.K - 1], order[cfg.K]
    b = b.copy()
    b[c] = np.float32(key[a] - np.float32(gap) - l32[t, c])
    m = margins(l32[t:t + 1], b, cfg.K)[0]
    assert 0 < m < 2 * gap + 1e-7, m
    return b


def _flip(idx, logits32, bias, K, t):
    """idx with token t's K-th pick replaced by its (K+1)-th best key."""
    key = logits32[t] + bias
    order = np.argsort(-key, kind="stable")
    out = idx.copy()
    out[t, np.nonzero(out[t] == order[K - 1])[0][0]] = order[K]
    return out


def test_no_flip_is_exact():
    cfg, x, wr, b, w13, w2 = _layer()
    ref = oracle.layer(x, wr, b, w13, w2, cfg.K, cfg.scale)
    err, flips = check_end_to_end(cfg, x, wr, b, w13, w2, ref["y"], ref["idx"])
    assert err == 0.0 and flips == 0


def test_flip_below_the_margin_is_accepted_and_compared_with_its_own_set():
    cfg, x, wr, b, w13, w2 = _layer()
    t = 5
    b = _near_tie(cfg, x, wr, b, t, 4e-6)
    ref = oracle.layer(x, wr, b, w13, w2, cfg.K, cfg.scale)
    idx_gpu = _flip(ref["idx"], ref["logits32"], b, cfg.K, t)
    assert (np.sort(idx_gpu[t]) != np.sort(ref["idx"][t])).any()
    # a "GPU" that took the other set and computed its row correctly
    y_gpu = oracle.layer_with_routing(x, ref["logits32"], idx_gpu, w13, w2, cfg.scale)
    err, flips = check_end_to_end(cfg, x, wr, b, w13, w2, y_gpu, idx_gpu)
    assert flips == 1 and err <= 1e-12
    # the same flip with the row of the oracle's own set is caught: the
    # reference row really is recomputed for the GPU's set
    y_bad = y_gpu.copy()
    y_bad[t] = ref["y"][t]
    err_bad, _ = check_end_to_end(cfg, x, wr, b, w13, w2, y_bad, idx_gpu)
    assert err_bad > 1e-4


def test_flip_above_the_margin_is_rejected():
    cfg, x, wr, b, w13, w2 = _layer()
    ref = oracle.layer(x, wr, b, w13, w2, cfg.K, cfg.scale)
    m = margins(ref["logits32"], b, cfg.K)
    t = int(np.argmax(m))
    assert m[t] > FLIP_MARGIN
    idx_gpu = _flip(ref["idx"], ref["logits32"], b, cfg.K, t)
    y_gpu = oracle.layer_with_routing(x, ref["logits32"], idx_gpu, w13, w2, cfg.scale)
    with pytest.raises(AssertionError, match="routing differs"):
        check_end_to_end(cfg, x, wr, b, w13, w2, y_gpu, idx_gpu)


def test_flip_just_above_the_margin_is_rejected():
    cfg, x, wr, b, w13, w2 = _layer()
    t = 9
    b = _near_tie(cfg, x, wr, b, t, 3e-5)
    ref = oracle.layer(x, wr, b, w13, w2, cfg.K, cfg.scale)
    assert margins(ref["logits32"][t:t + 1], b, cfg.K)[0] >= FLIP_MARGIN
    idx_gpu = _flip(ref["idx"], ref["logits32"], b, cfg.K, t)
    y_gpu = oracle.layer_with_routing(x, ref["logits32"], idx_gpu, w13, w2, cfg.scale)
    with pytest.raises(AssertionError, match="routing differs"):
        check_end_to_end(cfg, x, wr, b, w13, w2, y_gpu, idx_gpu)
