"""GPU parity of the router weight similarity (moe_router_similarity) against
the oracle.

The GPU forms the Gram matrix of w_router with fp32 products and fp32
accumulation (matrix cores, K split into partial tiles summed in order), then
divides by fp32 norms.  The rounding error of an fp32 dot product of length H
grows like sqrt(H) unit roundoffs of sum |w_i[h] w_j[h]| <= |w_i| |w_j|, so
each cosine may differ from the oracle's fp64 value by about sqrt(H) * 2^-24;
the bar is four times that, plus 1e-6 for the normalisation roundings.  The
mean is compared with the same bar.  Exact properties: sim is bitwise
symmetric, a zero row gives exact zeros, and two runs agree bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_02_amd as moe
import workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _atol(H):
    return 4.0 * math.sqrt(H) * 2.0 ** -24 + 1e-6


def _run(w, ws_fill=None):
    E, H = w.shape
    wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(DEV)
    sim = torch.empty((E, E), dtype=torch.float32, device=DEV)
    mean = torch.empty(1, dtype=torch.float32, device=DEV)
    nbytes = moe.moe_router_similarity_workspace_bytes(E, H)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    if ws_fill is not None:
        ws.fill_(ws_fill)
    moe.moe_router_similarity(wd, sim, mean, ws)
    torch.cuda.synchronize()
    return sim.cpu().numpy(), float(mean.cpu().item())


def _check(w, sim, mean):
    E, H = w.shape
    ref, ref_mean = oracle.router_similarity(w)
    tol = _atol(H)
    np.testing.assert_allclose(sim, ref, rtol=0, atol=tol)
    assert abs(mean - ref_mean) <= tol
    np.testing.assert_array_equal(sim, sim.T)


@pytest.mark.parametrize("E,H", [(24, 256), (96, 2048), (130, 100), (1, 8), (65, 4), (200, 36)])
def test_similarity_matches_oracle(E, H):
    w = np.random.default_rng(E * 1000 + H).standard_normal((E, H)).astype(np.float32)
    print(f"similarity E={E} H={H}", flush=True)
    sim, mean = _run(w)
    _check(w, sim, mean)


def test_similarity_of_the_full_scale_router():
    cfg = workload.CONFIGS["prefill_bf16"]
    w = workload.make_router(cfg).numpy()          # [768, 6144], N(0, 0.006)
    print("similarity full-scale router 768 x 6144", flush=True)
    sim, mean = _run(w)
    _check(w, sim, mean)
    # Independent random rows: cosines spread like N(0, 1/H) around zero.
    off = sim[~np.eye(cfg.E, dtype=bool)]
    assert abs(off.std() * math.sqrt(cfg.H) - 1.0) < 0.05
    sim2, mean2 = _run(w, ws_fill=0xFF)            # stale workspace (NaN bytes) is not read
    np.testing.assert_array_equal(sim, sim2)
    assert mean == mean2


def test_similarity_zero_scaled_and_collapsed_rows():
    r = np.random.default_rng(71)
    E, H = 100, 512
    w = r.standard_normal((E, H)).astype(np.float32)
    w[3] = 0.0
    w[5] *= -8.0
    w[77] = w[10] * 2.0
    sim, mean = _run(w)
    _check(w, sim, mean)
    assert not sim[3].any() and not sim[:, 3].any()
    assert abs(sim[10, 77] - 1.0) <= _atol(H)
    common = r.standard_normal(H)
    wc = (common + 0.05 * r.standard_normal((E, H))).astype(np.float32)
    sim, mean = _run(wc)
    _check(wc, sim, mean)
    assert mean > 0.99
