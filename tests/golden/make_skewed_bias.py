"""Write ``skewed_bias_seed0.txt``: the selection bias of the skewed workload.

The skewed workload wants about 40 % of all picks on the zero-computation
experts (spread evenly over them: all identity experts treated as one group,
as the LongCat-Flash Technical Report notes describe for the load-balance
loss, Key claims [§2.1.2]) and FFN expert loads that follow Zipf(1.1) over a
seeded permutation of the experts.  A token picks an expert at most once, so
a load cannot exceed T: the Zipf targets are capped at T and the excess is
water-filled over the uncapped experts.

The bias is found offline with frequency feedback on the oracle's routing --
the same idea as the PID-adjusted bias of the pages (Key claims [§2.1.1]),
used here only to build an input: raise the bias of experts that receive too
few tokens, lower it where they receive too many, on the oracle's fp32 logits
of the workload's own x and router weights.

This script calls only ``oracle`` and ``workload``.  Run from the repo root:
    python tests/golden/make_skewed_bias.py
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np
from scipy.stats import norm

_ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, _ROOT)

import oracle  # noqa: E402
import workload  # noqa: E402

ZERO_SHARE = 0.40
ZIPF_S = 1.1
ITERS = 80
STEP = 0.1


def targets(cfg) -> np.ndarray:
    """Target pick count per expert id (FFN ids 0..N-1, identity ids N..E-1)."""
    total = cfg.T * cfg.K
    zero_total = ZERO_SHARE * total
    ffn_total = total - zero_total
    ranks = np.arange(1, cfg.N + 1, dtype=np.float64)
    w = ranks ** (-ZIPF_S)
    tgt = np.zeros(cfg.N)
    capped = np.zeros(cfg.N, bool)
    while True:  # water-filling under the cap T
        free = ffn_total - cfg.T * capped.sum()
        tgt = np.where(capped, cfg.T, free * w / w[~capped].sum())
        over = (tgt > cfg.T) & ~capped
        if not over.any():
            break
        capped |= over
    perm = workload.zipf_permutation(cfg)
    out = np.empty(cfg.E)
    out[perm] = tgt                      # expert perm[r] gets rank r+1's load
    out[cfg.N:] = zero_total / cfg.Z
    return out


def main() -> None:
    cfg = workload.CONFIGS["skewed_bf16"]
    t0 = time.time()
    x = workload.make_x(cfg).float().numpy()
    wr = workload.make_router(cfg).numpy()
    threads = max(1, min(16, os.cpu_count() or 1))
    logits32 = oracle.router_logits(x, wr, threads=threads).astype(np.float32)
    print(f"oracle logits: {time.time() - t0:.1f}s", flush=True)
    tgt = targets(cfg)
    sig = float(logits32.std())
    p = np.clip(tgt / cfg.T, 1e-6, 1 - 1e-6)
    b = (-sig * norm.ppf(1.0 - p)).astype(np.float64)
    b -= b.mean()
    for it in range(ITERS):
        _, _, counts = oracle.route(logits32, b.astype(np.float32), cfg.K)
        err = np.log((counts + 1.0) / (tgt + 1.0))
        b -= STEP * sig * err
        b -= b.mean()
        if it % 10 == 0 or it == ITERS - 1:
            zs = counts[cfg.N:].sum() / (cfg.T * cfg.K)
            dev = np.abs(counts - tgt) / np.maximum(tgt, 1)
            print(f"iter {it}: zero share {zs:.4f}  median dev {np.median(dev):.4f}  "
                  f"max dev {dev.max():.3f}", flush=True)
    bias = b.astype(np.float32)
    _, _, counts = oracle.route(logits32, bias, cfg.K)
    zs = counts[cfg.N:].sum() / (cfg.T * cfg.K)
    ffn = np.sort(counts[:cfg.N])[::-1]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skewed_bias_seed0.txt")
    with open(out, "w") as f:
        f.write("# Selection bias of the skewed workload (T=16384, H=6144, 512 FFN + 256 identity\n")
        f.write("# experts, K=12, seed 0), one fp32 value per expert id as a hex float.\n")
        f.write("# Written by tests/golden/make_skewed_bias.py (oracle routing feedback).\n")
        f.write(f"# On the oracle's logits: zero-expert share {zs:.4f}; FFN loads max {ffn[0]}, "
                f"rank2 {ffn[1]}, rank3 {ffn[2]}, median {int(np.median(ffn))}, min {ffn[-1]}.\n")
        for v in bias:
            f.write(float(v).hex() + "\n")
    print(f"wrote {out}; zero share {zs:.4f}; top loads {ffn[:6].tolist()}; min {ffn[-1]}; "
          f"bias range {bias.min():.3f}..{bias.max():.3f}; {time.time() - t0:.1f}s")


if __name__ == "__main__":
    main()
