"""The bench's accounting, on the CPU: the algorithmic bytes and FLOPs the
rooflines divide by, the fractions made from them, and the rule that a
stored HBM-counter measurement is used only for the kernel source it was
taken on."""
import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workload  # noqa: E402


def _prefill_counts():
    cfg = workload.CONFIGS["prefill_bf16"]
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[:cfg.N] = 127          # 512 active experts, 65,024 rows
    counts[:144] += 1             # 65,168 rows, as in the measured layer
    return cfg, counts, int(counts[:cfg.N].sum())


def test_gemm_bytes_and_flops_of_the_prefill_layer():
    cfg, counts, S = _prefill_counts()
    assert S == 65168
    alg = bench.algorithmic(cfg, counts, S)
    # weights of every active expert once, activation rows in and out once
    assert alg["active"] == 512
    assert alg["gateup_bytes"] == 512 * 2 * 2048 * 6144 * 2 + S * (6144 + 2048) * 2 == 26837516288
    assert alg["down_bytes"] == 512 * 6144 * 2048 * 2 + S * (2048 + 6144) * 2 == 13952614400
    assert alg["gateup_flops"] == 2.0 * S * 6144 * 4096
    assert alg["down_flops"] == alg["gateup_flops"] / 2


def test_identity_picks_and_idle_experts_cost_nothing():
    cfg = workload.CONFIGS["mid_bf16"]
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[cfg.N:] = 100          # identity experts only
    alg = bench.algorithmic(cfg, counts, 0)
    assert alg["active"] == 0 and alg["gateup_bytes"] == 0 and alg["down_flops"] == 0
    counts[3] = 5                 # one FFN expert with 5 rows
    alg = bench.algorithmic(cfg, counts, 5)
    assert alg["active"] == 1
    assert alg["gateup_bytes"] == 2 * cfg.I * cfg.H * 2 + 5 * (cfg.H + cfg.I) * 2


def test_fractions_follow_from_bytes_flops_and_time():
    alg = dict(gateup_bytes=8e9, down_bytes=4e9, gateup_flops=2.5e12, down_flops=1.25e12)
    gu, dn, ffn = bench.gemm_fracs(alg, 1.0, 1.0)     # 1 ms each
    assert gu["hbm_frac"] == 1.0 and dn["hbm_frac"] == 0.5
    assert gu["mfma_frac"] == 1.0 and dn["mfma_frac"] == 0.5
    assert ffn["floor_ms"] == pytest.approx(1.5) and ffn["frac_of_floor"] == 0.75
    assert ffn["binding_roof"] == "hbm"
    gu, dn, ffn = bench.gemm_fracs(dict(alg, gateup_bytes=1e9, down_bytes=1e9), 1.0, 1.0)
    assert ffn["binding_roof"] == "mfma"


def test_source_hash_ignores_comments_only():
    a = "int f(int x) {  // doubles\n  return 2 * x;\n}\n"
    b = "// a header\nint f(int x) {\n\n  return 2 * x;   // the same code\n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"

    def h(text, tmp):
        p = os.path.join(tmp, "src.hip")
        with open(p, "w") as f:
            f.write(text)
        return bench.code_sha256(p)
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        assert h(a, tmp) == h(b, tmp)
        assert h(a, tmp) != h(c, tmp)


def test_stored_traffic_is_used_only_for_its_source_and_workload(tmp_path, monkeypatch):
    src = tmp_path / "ffn.hip"
    src.write_text("__global__ void k() {}\n")
    rec = {"workload": "prefill_bf16", "code_sha256": bench.code_sha256(str(src)),
           "bytes_per_launch": 123}
    rec_path = tmp_path / "traffic.json"
    rec_path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec_path))
    monkeypatch.setattr(bench, "FFN_SOURCE", str(src))
    assert bench.measured_traffic("prefill_bf16") == 123
    assert bench.measured_traffic("skewed_bf16") is None
    src.write_text("// a comment\n__global__ void k() {}   // another\n")
    assert bench.measured_traffic("prefill_bf16") == 123
    src.write_text("__global__ void k() { return; }\n")
    assert bench.measured_traffic("prefill_bf16") is None


def test_call_floors_of_the_prefill_layer():
    cfg, counts, S = _prefill_counts()
    names = [n for ns in bench.CALLS.values() for n in ns]
    kern = {n: (1, 1.0) for n in names}          # every kernel: one launch of 1 ms
    calls = bench.call_floors(cfg, counts, S, kern)
    T, H, E, K = cfg.T, cfg.H, cfg.E, cfg.K
    r = calls["moe_router_logits"]
    assert r["bytes"] == T * H * 2 + E * H * 4 + T * E * 4 == 144703488
    assert r["gflop"] == pytest.approx(3 * 2 * T * E * H / 1e9, abs=0.01)   # three bf16 passes
    assert r["floor_us"] == pytest.approx(3 * 2 * T * E * H / 2.5e15 * 1e6, abs=0.1)
    f = calls["moe_expert_ffn_gather"]                  # no grouped copy: the gather call
    assert f["bytes"] == 26837516288 + 13952614400
    assert f["floor_us"] == pytest.approx((26837516288 + 13952614400) / 8e12 * 1e6, abs=0.1)
    c = calls["moe_combine_identity"]
    assert c["bytes"] == S * H * 2 + 2 * T * H * 2 + T * K * 8
