"""Benchmark of the MoE layer forward pass on one MI355X.

One step = one forward pass over one batch of synthetic input already
resident in HBM, enqueued back to back on one stream: router scores, routing,
dispatch (indices), the expert FFNs (gathering their rows from x), and combine
with the identity experts' term folded in (--grouped-copy and
--separate-identity time the six-call composition's pieces instead).  Default
workload: the full-scale prefill-shaped layer (T = 8192 tokens, hidden 6144,
512 SwiGLU FFN experts of intermediate 2048 + 256 identity experts, K = 12,
38.65 GB of bf16 expert weights on the GPU).

Prints one JSON line: tokens/s, the roofline of the dominant kernel (the
gate/up expert GEMM, HBM-bound at these shapes) from per-kernel HIP events
recorded in the timed region, and the oracle's CPU throughput on a bounded
sample of the same workload.

    python bench.py [--steps 20] [--warmup 3] [--workload prefill_bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_moe_layer_02_amd as moe  # noqa: E402
import workload  # noqa: E402

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gateup_traffic.json")
FFN_SOURCE = os.path.join(ROOT, "sparse_moe_layer_02_amd", "csrc", "ffn.hip")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix, published
# The calls of one forward pass and the kernels each one launches.
CALLS = {
    "moe_router_logits": ("router_logits",),
    "moe_route": ("route_topk", "route_hist"),
    "moe_permute": ("permute", "permute_gather"),
    "moe_expert_ffn": ("ffn_tiles", "ffn_gateup_dense_bf16", "ffn_gateup_bf16",
                       "ffn_down_dense_bf16", "ffn_down_narrow_bf16", "ffn_down_bf16",
                       "ffn_gateup_f32", "ffn_down_f32"),
    "moe_zero_experts": ("zero_experts",),
    "moe_combine": ("combine",),
    "moe_combine_identity": ("combine_identity",),
}
METRIC = "MoE-layer tokens/sec at 1 GPU; grouped-GEMM MFMA util and HBM GB/s vs peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="prefill_bf16", choices=sorted(workload.CONFIGS))
    p.add_argument("--profile-steps", type=int, default=5,
                   help="steps of the separate pass, after the timed region, that times every "
                        "kernel with HIP events for the per-call table")
    p.add_argument("--cpu-tokens", type=int, default=96,
                   help="tokens of the oracle's CPU sample (0 = skip)")
    p.add_argument("--kernels", action="store_true", help="also print the per-kernel table")
    p.add_argument("--bias-controller", type=float, default=0.0, metavar="TARGET",
                   help="also run one bias-controller update per step (moe_bias_update, "
                        "FFN experts per token held at TARGET; gains 1.0/0.05/0.2)")
    p.add_argument("--flush-mib", type=int, default=0,
                   help="write a scratch buffer of this many MiB before every timed step "
                        "(outside the step's events) so that small layers do not run from the "
                        "256 MB Infinity Cache; ms_per_step is then the mean of per-step events")
    p.add_argument("--grouped-copy", action="store_true",
                   help="dispatch copies the grouped x rows (moe_permute into x_perm, then "
                        "moe_expert_ffn) instead of the expert GEMM gathering them from x")
    p.add_argument("--separate-identity", action="store_true",
                   help="run the identity experts as their own call (moe_zero_experts into "
                        "y_acc, on a second stream, then moe_combine) instead of inside combine "
                        "(moe_combine_identity)")
    p.add_argument("--router-split-per-call", action="store_true",
                   help="split the fp32 router weights into their bf16 planes inside every "
                        "router call instead of once before the run (moe_router_split_weights, "
                        "a weight-format preparation outside the timed steps)")
    p.add_argument("--companions", default="decode_bf16,skewed_bf16",
                   help="other full-scale workloads timed after the headline on the same "
                        "resident weights (comma-separated; 'none' to skip); each gets its own "
                        "sub-object with ms/step, tokens/s and the expert GEMMs' HBM and MFMA "
                        "fractions")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="first run one plain device-to-device copy of this many MiB (the "
                        "reference dispatch that scales HBM byte counters)")
    return p.parse_args()


def algorithmic(cfg, counts, S):
    """Bytes the method must move / FLOPs it must do, per kernel of interest.
    Expert weights count once per active expert; activations once per row."""
    es = 2 if cfg.dtype == "bf16" else 4
    active = int((counts[:cfg.N] > 0).sum())
    H, I = cfg.H, cfg.I
    w13 = active * 2 * I * H * es
    w2 = active * H * I * es
    gateup_bytes = w13 + S * H * es + S * I * es        # weights + grouped x rows + hh rows
    down_bytes = w2 + S * I * es + S * H * es           # weights + hh rows + y_perm rows
    gateup_flops = 2.0 * S * H * 2 * I
    down_flops = 2.0 * S * I * H
    return dict(active=active, gateup_bytes=gateup_bytes, down_bytes=down_bytes,
                gateup_flops=gateup_flops, down_flops=down_flops)


def call_floors(cfg, counts, S, kern, grouped_copy=False):
    """Per call of the forward pass: measured microseconds, algorithmic bytes
    (inputs read once, outputs written once, weights of active experts read
    once) and FLOPs, the floor max(bytes / HBM peak, FLOPs / matrix peak),
    and the call's fraction of its floor.  The router's FLOPs are counted as
    the three bf16 matrix passes it runs on bf16 layers (an fp32-exact
    product), against the bf16 peak; on fp32 layers as one pass against the
    fp32 peak.  Dispatch counts the grouped copy of the x rows only when
    it makes one; otherwise the expert GEMM reads them from x itself
    (moe_expert_ffn_gather) and dispatch moves indices only."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, H, E, N, I, K = cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K
    alg = algorithmic(cfg, counts, S)
    mm_peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    router_flops = 2.0 * T * E * H * (3 if cfg.dtype == "bf16" else 1)
    work = {
        "moe_router_logits": (T * H * es + E * H * 4 + T * E * 4, router_flops),
        "moe_route": (T * E * 4 + E * 4 + T * K * 8 + E * 8, 0.0),
        "moe_permute": (T * K * 4 * 2 + (N + 1) * 4 + S * 4 + T * K * 4
                        + ((T * H * es + S * H * es) if grouped_copy else 0), 0.0),
        "moe_expert_ffn": (alg["gateup_bytes"] + alg["down_bytes"],
                           alg["gateup_flops"] + alg["down_flops"]),
        "moe_zero_experts": (T * H * es + T * H * 4 + T * K * 8, 0.0),
        "moe_combine": (S * H * es + T * H * 4 + T * H * es + T * K * 8, 0.0),
        "moe_combine_identity": (S * H * es + T * H * es + T * H * es + T * K * 8, 0.0),
    }
    out = {}
    for call, names in CALLS.items():
        if not any(n in kern for n in names):
            continue      # not a call of this forward path
        us = sum(kern[n][1] / kern[n][0] * 1e3 for n in names if n in kern)
        nbytes, flops = work[call]
        floor_us = max(nbytes / (HBM_PEAK_GBS * 1e3), flops / (mm_peak * 1e6))
        if call == "moe_expert_ffn" and not grouped_copy:
            call = "moe_expert_ffn_gather"
        out[call] = dict(us=round(us, 1), bytes=int(nbytes), gflop=round(flops / 1e9, 2),
                         floor_us=round(floor_us, 1),
                         frac_of_floor=round(floor_us / us, 3) if us > 0 else None)
    return out


def routing_stats(cfg, counts, S):
    """Realised routing of the timed batch: FFN share of the T*K picks and
    rows per active FFN expert."""
    rows = counts[:cfg.N]
    act = rows[rows > 0]
    return dict(ffn_share=round(S / (cfg.T * cfg.K), 4), identity_picks=int(cfg.T * cfg.K - S),
                active_ffn_experts=int(act.size),
                rows_per_active_expert={"min": int(act.min()) if act.size else 0,
                                        "median": float(np.median(act)) if act.size else 0.0,
                                        "max": int(act.max()) if act.size else 0})


def code_sha256(path):
    """SHA-256 of a C++/HIP source with its // comments, trailing blanks and
    empty lines removed: the same for two versions that differ only in their
    comments (which compile to the same kernels)."""
    out = []
    with open(path, encoding="utf-8") as f:
        for line in f:
            i = line.find("//")
            if i >= 0:
                line = line[:i]
            line = line.rstrip()
            if line:
                out.append(line)
    return hashlib.sha256("\n".join(out).encode()).hexdigest()


def measured_traffic(workload_name):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain-copy calibration), or None
    if they were taken on another workload or another version of the kernel
    (compared by code_sha256 of the GEMM source)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        src = code_sha256(FFN_SOURCE)
    except (OSError, ValueError):
        return None
    if rec.get("code_sha256") != src or rec.get("workload") != workload_name:
        return None
    return int(rec["bytes_per_launch"])


def router_similarity(w_router, reps=20):
    """The router-stability diagnostic on the workload's router weights, timed
    apart from the forward pass (it is not part of a step): per-kernel mean
    microseconds and the Gram kernel's rate against the fp32 matrix peak.
    Algorithmic FLOPs: the E(E+1)/2 distinct dot products of length H."""
    E, H = w_router.shape
    dev = w_router.device
    sim = torch.empty((E, E), dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.moe_router_similarity_workspace_bytes(E, H), dtype=torch.uint8,
                     device=dev)
    for _ in range(3):
        moe.moe_router_similarity(w_router, sim, mean, ws)
    torch.cuda.synchronize(dev)
    moe.moe_profile_enable(True)
    for _ in range(reps):
        moe.moe_router_similarity(w_router, sim, mean, ws)
    torch.cuda.synchronize(dev)
    moe.moe_profile_enable(False)
    kern = moe.moe_profile_summary()
    us = {k: round(v[1] / v[0] * 1e3, 1) for k, v in kern.items()}
    flops = float(E) * (E + 1) * H
    gram_s = kern["sim_gram"][1] / kern["sim_gram"][0] * 1e-3
    return dict(rows=E, hidden=H, mean_cosine=float(mean.item()), kernels_us=us,
                total_us=round(sum(us.values()), 1),
                gram_tflops=round(flops / gram_s / 1e12, 2),
                gram_mfma_f32_frac=round(flops / gram_s / 1e12 / MFMA_F32_PEAK_TFLOPS, 4))


def _host_cpu():
    """CPU model, logical CPUs of the host and CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    allowed = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    return model, os.cpu_count(), allowed


def cpu_baseline(cfg, inp, n_tokens):
    """The oracle, single-threaded and pinned to one host core, on n_tokens
    sampled tokens through all six stages, each stage timed on its own
    (time.perf_counter, a steady clock).  Copies of expert weights to the host
    are not timed.  Every stage's cost is linear in the tokens (rows per
    token are fixed by the routing), so the full-batch time is extrapolated
    per stage and labelled as such."""
    import oracle
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(cfg.T, n_tokens, replace=False))
    dev = inp["x"].device
    x = inp["x"][torch.from_numpy(toks).to(dev)].float().cpu().numpy()
    wr = inp["w_router"].cpu().numpy()
    b = inp["bias"].cpu().numpy()
    K, N = cfg.K, cfg.N
    model, ncpu, allowed = _host_cpu()
    core = allowed[0] if allowed else None
    if core is not None:
        os.sched_setaffinity(0, {core})
    stages = dict.fromkeys(("router_logits", "route", "permute", "expert_ffn", "zero_experts",
                            "combine"), 0.0)
    try:
        t0 = time.perf_counter()
        l32 = oracle.router_logits(x, wr).astype(np.float32)
        t1 = time.perf_counter()
        idx, gate, _ = oracle.route(l32, b, K)
        t2 = time.perf_counter()
        off, rs, slot = oracle.permute(idx, N)
        t3 = time.perf_counter()
        stages["router_logits"], stages["route"], stages["permute"] = t1 - t0, t2 - t1, t3 - t2
        xp = x[rs // K]
        yp = np.empty((rs.size, cfg.H))
        for e in np.nonzero(np.diff(off))[0]:
            a, c = int(off[e]), int(off[e + 1])
            w13e = inp["w13"][e].float().cpu().numpy()
            w2e = inp["w2"][e].float().cpu().numpy()
            t0 = time.perf_counter()
            yp[a:c] = oracle.ffn_rows(xp[a:c], w13e, w2e)
            stages["expert_ffn"] += time.perf_counter() - t0
        t0 = time.perf_counter()
        yacc = oracle.zero_experts(x, idx, gate, N)
        t1 = time.perf_counter()
        oracle.combine(yp, slot, idx, gate, cfg.scale, yacc, N)
        t2 = time.perf_counter()
        stages["zero_experts"], stages["combine"] = t1 - t0, t2 - t1
    finally:
        if core is not None:
            os.sched_setaffinity(0, set(allowed))
    spent = sum(stages.values())
    scale = cfg.T / n_tokens
    return dict(value=round(n_tokens / spent, 3), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{n_tokens} of {cfg.T} tokens of {cfg.name}, all six stages, "
                       f"single-threaded fp64 oracle pinned to one core ({spent:.1f} s of CPU; "
                       f"weight copies to the host not timed)",
                host_cpu_model=model, host_nproc=ncpu, pinned_core=core,
                stage_seconds={k: round(v, 4) for k, v in stages.items()},
                extrapolated_full_batch_seconds={
                    "label": f"extrapolated: sample stage times x {cfg.T}/{n_tokens}",
                    **{k: round(v * scale, 1) for k, v in stages.items()},
                    "total": round(spent * scale, 1)})


def time_workload(cfg, inp, args, dev, x=None, bias=None, steps=None, warmup=None,
                  profile_steps=None, log=True):
    """Warm-up, then `steps` timed forward passes of one workload on resident
    inputs (x / bias override the inputs of inp), then a short pass with
    every kernel bracketed for the per-call table.  Returns a dict of the
    timings and the buffers of the last pass."""
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    profile_steps = args.profile_steps if profile_steps is None else profile_steps
    x = inp["x"] if x is None else x
    bias = (inp["bias"] if bias is None else bias).clone()
    buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev,
                            grouped_copy=args.grouped_copy,
                            separate_identity=args.separate_identity)
    if not args.router_split_per_call:
        moe.prepare_router(inp["w_router"], buf)   # once: the weights do not change
    stream = torch.cuda.current_stream(dev)
    if args.bias_controller > 0:
        integral = torch.zeros(cfg.N, dtype=torch.float32, device=dev)
        prev_err = torch.zeros(cfg.N, dtype=torch.float32, device=dev)

    def step():
        moe.forward(x, inp["w_router"], bias, inp["w13"], inp["w2"], cfg.K, cfg.scale, buf)
        if args.bias_controller > 0:
            moe.moe_bias_update(buf["counts"], cfg.T, cfg.N, args.bias_controller, 1.0, 0.05, 0.2,
                                bias, integral, prev_err)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    if log:
        print(f"[bench] {cfg.name}: warmup done ({warmup} steps); timing {steps} steps",
              file=sys.stderr, flush=True)

    # In the timed region only the two expert GEMM launches are bracketed by
    # HIP events (the roofline's kernel times): bracketing every launch costs
    # ~80 us of stream time per step (measured).  The per-call table comes
    # from a separate pass afterwards.
    # each expert GEMM is one launch for the partial m-tiles plus, on bf16
    # layers, one for the full 256-row m-tiles (the dense kernel), and for
    # down one more for the partial m-tiles of at most 128 rows
    gemm_names = ((("ffn_gateup_bf16", "ffn_gateup_dense_bf16"),
                   ("ffn_down_bf16", "ffn_down_dense_bf16", "ffn_down_narrow_bf16"))
                  if cfg.dtype == "bf16" else (("ffn_gateup_f32",), ("ffn_down_f32",)))
    moe.moe_profile_select(gemm_names[0] + gemm_names[1])
    moe.moe_profile_enable(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.flush_mib > 0:
        scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
    torch.cuda.synchronize(dev)
    start.record(stream)
    for i in range(steps):
        if args.flush_mib > 0:
            scratch.fill_(i & 0xFF)
            evs[i][0].record(stream)
        step()
        if args.flush_mib > 0:
            evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize(dev)
    moe.moe_profile_enable(False)
    if args.flush_mib > 0:
        ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    else:
        ms = start.elapsed_time(end) / steps
    kern_timed = moe.moe_profile_summary()
    moe.moe_profile_select(None)

    # the per-call table: every kernel bracketed, a few more steps
    prof_ms = None
    kern = kern_timed
    if profile_steps > 0:
        moe.moe_profile_enable(True)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for _ in range(profile_steps):
            step()
        p1.record(stream)
        torch.cuda.synchronize(dev)
        moe.moe_profile_enable(False)
        kern = moe.moe_profile_summary()
        prof_ms = p0.elapsed_time(p1) / profile_steps

    counts = buf["counts"].cpu().numpy()
    S = int(buf["offsets"][-1].item())
    alg = algorithmic(cfg, counts, S)
    def mean_ms(names):   # summed mean launch durations of one GEMM's kernels
        return sum(kern_timed[n][1] / kern_timed[n][0] for n in names if n in kern_timed)
    gu_ms = mean_ms(gemm_names[0])
    dn_ms = mean_ms(gemm_names[1])
    return dict(ms=ms, kern_timed=kern_timed, kern=kern, prof_ms=prof_ms, counts=counts, S=S,
                alg=alg, gemm_names=gemm_names, gu_ms=gu_ms, dn_ms=dn_ms, buf=buf,
                steps=steps, profile_steps=profile_steps)


def gemm_fracs(alg, gu_ms, dn_ms):
    """HBM and MFMA fractions of the two expert GEMMs from their algorithmic
    bytes and FLOPs and their mean launch durations."""
    def one(nbytes, flops, ms):
        return {"kernel_ms": round(ms, 4),
                "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "algorithmic_bytes": int(nbytes), "gflop": round(flops / 1e9, 2)}
    gu = one(alg["gateup_bytes"], alg["gateup_flops"], gu_ms)
    dn = one(alg["down_bytes"], alg["down_flops"], dn_ms)
    both_ms = gu_ms + dn_ms
    floor_ms = max((alg["gateup_bytes"] + alg["down_bytes"]) / (HBM_PEAK_GBS * 1e9),
                   (alg["gateup_flops"] + alg["down_flops"]) / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    return gu, dn, {"ms": round(both_ms, 4), "floor_ms": round(floor_ms, 4),
                    "frac_of_floor": round(floor_ms / both_ms, 4),
                    "binding_roof": "hbm" if (alg["gateup_bytes"] + alg["down_bytes"])
                    / (HBM_PEAK_GBS * 1e9) >= (alg["gateup_flops"] + alg["down_flops"])
                    / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"}


def companion(name, inp, args, dev):
    """Another full-scale layer on the same resident expert and router
    weights (only its tokens and bias differ): its own timed steps and the
    same per-GEMM fractions as the headline."""
    cfg = workload.CONFIGS[name]
    x = workload.make_x(cfg).to(dev)
    bias = workload.make_bias(cfg).to(dev)
    print(f"[bench] {name}: same weights, {cfg.T} tokens", file=sys.stderr, flush=True)
    r = time_workload(cfg, inp, args, dev, x=x, bias=bias)
    gu, dn, ffn = gemm_fracs(r["alg"], r["gu_ms"], r["dn_ms"])
    out = {"workload": name, "tokens": cfg.T, "ffn_scale": cfg.scale, "steps": r["steps"],
           "ms_per_step": round(r["ms"], 4), "tokens_per_s": round(cfg.T / (r["ms"] * 1e-3), 1),
           "gateup_gemm": gu, "down_gemm": dn, "expert_ffn": ffn,
           "calls": call_floors(cfg, r["counts"], r["S"], r["kern"], args.grouped_copy),
           "routing": routing_stats(cfg, r["counts"], r["S"])}
    del r["buf"]
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    cfg = workload.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] {cfg.name}: drawing inputs on {torch.cuda.get_device_name(dev)}",
          file=sys.stderr, flush=True)
    inp = workload.make_inputs(cfg, dev)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    r = time_workload(cfg, inp, args, dev)
    ms, kern, alg, S, counts = r["ms"], r["kern"], r["alg"], r["S"], r["counts"]
    gu, dn, ffn = gemm_fracs(alg, r["gu_ms"], r["dn_ms"])
    achieved = alg["gateup_bytes"] / (r["gu_ms"] * 1e-3) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(cfg.name),
                    kernel=" + ".join(n for n in r["gemm_names"][0] if n in r["kern_timed"]), kernel_ms=round(r["gu_ms"], 4),
                    algorithmic_bytes=alg["gateup_bytes"], mfma_frac=gu["mfma_frac"])
    prof_ms = r["prof_ms"]
    result = {
        "metric": METRIC,
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,sigma) weights; no checkpoint)",
        "config": {"workload": cfg.name + ("+bias_controller" if args.bias_controller > 0 else ""),
                   "tokens": cfg.T, "hidden": cfg.H, "ffn_experts": cfg.N,
                   "zero_experts": cfg.Z, "intermediate": cfg.I, "top_k": cfg.K,
                   "ffn_scale": cfg.scale, "ffn_rows": S, "active_ffn_experts": alg["active"],
                   "dispatch": "grouped_copy" if args.grouped_copy else "row_gather",
                   "identity_experts": "separate" if args.separate_identity else "in_combine",
                   "router_weights": "split_per_call" if args.router_split_per_call
                   else "presplit_planes"},
        "roofline": roofline,
        "down_gemm": {k: dn[k] for k in ("kernel_ms", "hbm_frac", "mfma_frac")},
        "expert_ffn": ffn,
        "kernels_us": {k: round(v[1] / v[0] * 1e3, 1) for k, v in kern.items()},
        "kernels_timing": (f"expert GEMMs: HIP events in the timed region; other kernels: a "
                           f"separate pass of {r['profile_steps']} steps with every launch "
                           f"bracketed ({prof_ms:.4f} ms per step there)"
                           if prof_ms is not None else "timed region (expert GEMMs only)"),
        "calls": call_floors(cfg, counts, S, kern, args.grouped_copy),
        "routing": routing_stats(cfg, counts, S),
    }
    del r
    if args.flush_mib > 0:
        result["cache_flush_mib_between_steps"] = args.flush_mib
    names = [] if args.companions in ("", "none") else args.companions.split(",")
    full_scale = all(workload.CONFIGS[n].replace(T=cfg.T, bias_mode=cfg.bias_mode,
                                                 bias_lo=cfg.bias_lo, bias_hi=cfg.bias_hi,
                                                 scale=cfg.scale, name=cfg.name) == cfg
                     for n in names)
    if names and not full_scale:
        print("[bench] companions skipped: they need the headline's expert weights",
              file=sys.stderr, flush=True)
    elif names:
        result["same_weights_workloads"] = {n: companion(n, inp, args, dev) for n in names}
    result["router_similarity"] = router_similarity(inp["w_router"])
    if args.cpu_tokens > 0:
        print(f"[bench] timing the oracle on {args.cpu_tokens} tokens", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_tokens, cfg.T))
    else:
        result["cpu_baseline"] = None
    if args.kernels:
        for k, (n, t) in kern.items():
            print(f"{k:28s} {n:5d} launches  {t / n * 1e3:10.1f} us", file=sys.stderr)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
