"""The seeded input generator: reproducible, independent streams, and the
skewed workload's calibrated bias realises the routing it was built for."""
import hashlib
import os

import numpy as np
import torch

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_streams_are_reproducible_and_independent():
    cfg = workload.CONFIGS["tiny_fp32"]
    a, b = workload.make_x(cfg), workload.make_x(cfg)
    assert torch.equal(a, b)
    w1, w2 = workload.make_expert_weights(cfg, "cpu", experts=[3, 5])
    v1, v2 = workload.make_expert_weights(cfg, "cpu", experts=[5])
    assert torch.equal(w1[1], v1[0]) and torch.equal(w2[1], v2[0])   # per-expert streams
    assert not torch.equal(w1[0], w1[1])
    r = workload.make_router(cfg)
    assert r.shape == (cfg.E, cfg.H) and abs(float(r.std()) - cfg.sigma_w) < 0.002
    b = workload.make_bias(cfg)
    assert float(b.min()) >= cfg.bias_lo and float(b.max()) <= cfg.bias_hi


def test_bf16_configs_round_to_nearest_even():
    cfg = workload.CONFIGS["mid_bf16"]
    x = workload.make_x(cfg, T=4)
    assert x.dtype == torch.bfloat16
    raw = workload.make_x(cfg.replace(dtype="f32"), T=4)
    np.testing.assert_array_equal(x.float().numpy(), raw.to(torch.bfloat16).float().numpy())


def test_decode_tokens_are_the_first_prefill_tokens():
    p, d = workload.CONFIGS["prefill_bf16"], workload.CONFIGS["decode_bf16"]
    assert torch.equal(workload.make_x(p, T=64), workload.make_x(d))
    assert torch.equal(workload.make_router(p), workload.make_router(d))


def test_host_streams_digest():
    """x and the router weights of the full-scale workloads are drawn on the
    host; the skewed bias file was calibrated on exactly these bytes."""
    cfg = workload.CONFIGS["skewed_bf16"]
    h = hashlib.sha256()
    h.update(workload.make_x(cfg, T=8).view(torch.int16).numpy().tobytes())
    h.update(workload.make_router(cfg)[:16].numpy().tobytes())
    with open(os.path.join(GOLDEN, "host_stream_digest.txt")) as f:
        want = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")][0]
    assert h.hexdigest() == want


def test_skewed_bias_realises_the_target_routing():
    cfg = workload.CONFIGS["skewed_bf16"]
    T = 2048                                  # a prefix of the batch: shares are per token
    x = workload.make_x(cfg, T=T).float().numpy()
    wr = workload.make_router(cfg).numpy()
    b = workload.make_bias(cfg).numpy()
    l32 = oracle.router_logits(x, wr, threads=os.cpu_count() or 1).astype(np.float32)
    idx, _, counts = oracle.route(l32, b, cfg.K)
    zero_share = (idx >= cfg.N).mean()
    assert abs(zero_share - 0.40) < 0.01
    ffn = np.sort(counts[:cfg.N])[::-1]
    perm = workload.zipf_permutation(cfg)
    assert counts[perm[0]] == T                      # rank 1 is capped at every token
    assert ffn[1] / T > 0.55 and ffn[2] / T > 0.35   # 11214 and 7179 of 16384
    # loads fall with the Zipf rank
    ranked = counts[perm]
    assert np.corrcoef(np.log(np.arange(1, cfg.N + 1)), np.log(ranked + 1))[0, 1] < -0.95
