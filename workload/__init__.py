"""Seeded synthetic inputs for the MoE layer forward pass.

This module draws random numbers and holds the shape table; it holds none of
the layer's arithmetic.  Both the HIP path and the oracle get their inputs
from here (the oracle receives host copies of exactly the bytes the GPU sees).

Shapes follow the LongCat-Flash Technical Report notes ("Key claims", report
§2.1 and §2.4 Model Configurations): hidden 6144, per-expert FFN intermediate
2048, 512 FFN + 256 zero-computation experts, K = 12 at full scale.  No
trained checkpoint or dataset is involved; every tensor is synthetic:

* ``x`` [T, H] ~ N(0, 1), ``w_router`` [E, H] ~ N(0, sigma_w), ``bias`` [E] ~
  U(lo, hi): numpy PCG64 streams keyed by (seed, tensor id), drawn in fp32 on
  the host, so they are the same on every machine;
* ``w13`` [N, 2I, H] (rows 0..I-1 gate, I..2I-1 up) and ``w2`` [N, H, I] ~
  N(0, sigma_w): torch's Philox generator on the device that holds them, one
  stream per (seed, tensor id, expert), so experts are independent and a
  subset can be drawn alone;
* bf16 configurations round the fp32 draws to bf16 (round to nearest even).

The skewed configuration's bias is not drawn: it is read from
``tests/golden/skewed_bias_seed0.txt``, written by
``tests/golden/make_skewed_bias.py`` (feedback calibration on the oracle's
routing so that ~40 % of picks land on zero-computation experts and FFN loads
follow a capped Zipf(1.1) law over a seeded permutation of the experts).
"""
from __future__ import annotations

import dataclasses
import os

import numpy as np
import torch

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SKEWED_BIAS_FILE = os.path.join(_ROOT, "tests", "golden", "skewed_bias_seed0.txt")

# stream ids, one per tensor
X, W_ROUTER, BIAS, W13, W2, PERM = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    H: int          # hidden size
    N: int          # FFN (SwiGLU) experts, ids 0..N-1
    Z: int          # zero-computation (identity) experts, ids N..N+Z-1
    I: int          # per-expert intermediate size
    K: int          # experts kept per token
    dtype: str      # "f32" or "bf16": activations, expert weights, output
    sigma_w: float  # std of router and expert weights
    bias_lo: float
    bias_hi: float
    scale: float    # variance-compensation factor on FFN expert outputs
    seed: int = 0
    bias_mode: str = "uniform"   # or "skewed" (calibrated, read from file)

    @property
    def E(self) -> int:
        return self.N + self.Z

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # tiny fp32 layer: 16 FFN + 8 identity experts, K = 4
    "tiny_fp32": MoEConfig("tiny_fp32", T=256, H=256, N=16, Z=8, I=128, K=4, dtype="f32",
                           sigma_w=0.02, bias_lo=-0.1, bias_hi=0.1, scale=1.0),
    # mid bf16 layer: 64 + 32 experts, K = 8
    "mid_bf16": MoEConfig("mid_bf16", T=4096, H=2048, N=64, Z=32, I=1024, K=8, dtype="bf16",
                          sigma_w=0.02, bias_lo=-0.1, bias_hi=0.1, scale=1.0),
    # full-scale LongCat-Flash MoE shapes, prefill-shaped batch
    "prefill_bf16": MoEConfig("prefill_bf16", T=8192, H=6144, N=512, Z=256, I=2048, K=12,
                              dtype="bf16", sigma_w=0.006, bias_lo=-0.05, bias_hi=0.05,
                              scale=1.0),
    # same seed, so the same experts; decode-shaped batch (weights streamed,
    # 1-3 rows per expert; its tokens are the first 64 of the prefill batch)
    "decode_bf16": MoEConfig("decode_bf16", T=64, H=6144, N=512, Z=256, I=2048, K=12,
                             dtype="bf16", sigma_w=0.006, bias_lo=-0.05, bias_hi=0.05,
                             scale=1.0),
    # same experts; calibrated skewed routing, compensation factor 2.0
    "skewed_bf16": MoEConfig("skewed_bf16", T=16384, H=6144, N=512, Z=256, I=2048, K=12,
                             dtype="bf16", sigma_w=0.006, bias_lo=-0.05, bias_hi=0.05,
                             scale=2.0, bias_mode="skewed"),
}


def _np_stream(seed: int, tensor: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, expert))))


def _torch_seed(seed: int, tensor: int, expert: int) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=(tensor, expert))
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _round(t: torch.Tensor, cfg: MoEConfig) -> torch.Tensor:
    return t if cfg.dtype == "f32" else t.to(torch.bfloat16)


def make_x(cfg: MoEConfig, T: int | None = None) -> torch.Tensor:
    """[T, H] activations on the host (fp32 or bf16)."""
    T = cfg.T if T is None else T
    a = _np_stream(cfg.seed, X).standard_normal((T, cfg.H), dtype=np.float32)
    return _round(torch.from_numpy(a), cfg)


def make_router(cfg: MoEConfig) -> torch.Tensor:
    """[E, H] fp32 router weights on the host."""
    a = _np_stream(cfg.seed, W_ROUTER).standard_normal((cfg.E, cfg.H), dtype=np.float32)
    a *= np.float32(cfg.sigma_w)
    return torch.from_numpy(a)


def make_bias(cfg: MoEConfig) -> torch.Tensor:
    """[E] fp32 selection bias on the host."""
    if cfg.bias_mode == "skewed":
        return torch.from_numpy(load_skewed_bias(cfg.E))
    a = _np_stream(cfg.seed, BIAS).uniform(cfg.bias_lo, cfg.bias_hi, cfg.E).astype(np.float32)
    return torch.from_numpy(a)


def load_skewed_bias(E: int) -> np.ndarray:
    vals = []
    with open(SKEWED_BIAS_FILE) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float.fromhex(line))
    a = np.asarray(vals, np.float32)
    if a.shape != (E,):
        raise ValueError(f"{SKEWED_BIAS_FILE}: expected {E} values, found {a.shape[0]}")
    return a


def zipf_permutation(cfg: MoEConfig) -> np.ndarray:
    """Seeded permutation of the FFN experts: perm[r] is the expert of load rank r+1."""
    return _np_stream(cfg.seed, PERM).permutation(cfg.N).astype(np.int64)


def make_expert_weights(cfg: MoEConfig, device="cpu", experts=None):
    """Expert weights on ``device``: w13 [n, 2I, H] and w2 [n, H, I] for the
    experts listed (all N by default), one Philox stream per expert."""
    experts = list(range(cfg.N)) if experts is None else list(experts)
    dt = cfg.torch_dtype
    n = len(experts)
    w13 = torch.empty((n, 2 * cfg.I, cfg.H), dtype=dt, device=device)
    w2 = torch.empty((n, cfg.H, cfg.I), dtype=dt, device=device)
    g = torch.Generator(device=device)
    for i, e in enumerate(experts):
        g.manual_seed(_torch_seed(cfg.seed, W13, e))
        w13[i].copy_(torch.randn((2 * cfg.I, cfg.H), generator=g, device=device,
                                 dtype=torch.float32).mul_(cfg.sigma_w))
        g.manual_seed(_torch_seed(cfg.seed, W2, e))
        w2[i].copy_(torch.randn((cfg.H, cfg.I), generator=g, device=device,
                                dtype=torch.float32).mul_(cfg.sigma_w))
    return w13, w2


def make_inputs(cfg: MoEConfig, device="cpu") -> dict:
    """All layer inputs, resident on ``device``."""
    w13, w2 = make_expert_weights(cfg, device)
    return dict(x=make_x(cfg).to(device), w_router=make_router(cfg).to(device),
                bias=make_bias(cfg).to(device), w13=w13, w2=w2)
