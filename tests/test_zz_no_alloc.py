"""The allocation-free expert-FFN entry point (moe_expert_ffn_gather_noalloc)
against moe_expert_ffn_gather, through the C ABI: bit for bit on two calls in
a row, the second with a smaller batch (the fixed scratch keeps the first
call's contents), a too-large batch rejected before any launch, and the call
captured into a HIP graph and replayed."""
import numpy as np
import pytest
import torch

import sparse_moe_layer_02_amd as moe
import workload
from _parity import device, host

pytestmark = pytest.mark.gpu

CFG = workload.MoEConfig("noalloc", T=300, H=1024, N=32, Z=8, I=512, K=6, dtype="bf16",
                         sigma_w=0.03, bias_lo=-0.1, bias_hi=0.1, scale=1.0)


def _routed(cfg, inp, dev):
    """Router, routing and dispatch through the library: the gather inputs."""
    buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev)
    moe.moe_router_logits(inp["x"], inp["w_router"], buf["logits"])
    moe.moe_route(buf["logits"], inp["bias"], cfg.K, buf["topk_idx"], buf["topk_gate"],
                  buf["counts"], buf["status"])
    moe.moe_permute(inp["x"], buf["topk_idx"], buf["counts"], cfg.N, buf["offsets"], None,
                    buf["row_src"], buf["slot_row"])
    return buf


def test_noalloc_matches_the_workspace_call_on_two_calls():
    dev = device()
    full = workload.make_inputs(CFG, dev)
    for T in (300, 77):                       # the second call is smaller
        cfg = CFG.replace(T=T)
        print(f"\n[case] noalloc T={T}", flush=True)
        inp = dict(full, x=full["x"][:T].contiguous())
        buf = _routed(cfg, inp, dev)
        rows = T * cfg.K
        y_ws = torch.full((rows, cfg.H), float("nan"), dtype=torch.bfloat16, device=dev)
        y_na = torch.full((rows, cfg.H), float("nan"), dtype=torch.bfloat16, device=dev)
        moe.moe_expert_ffn_gather(inp["x"], cfg.K, buf["row_src"], buf["offsets"], inp["w13"],
                                  inp["w2"], y_ws, buf["ws_ffn"])
        moe.moe_expert_ffn_gather_noalloc(inp["x"], cfg.K, buf["row_src"], buf["offsets"],
                                          inp["w13"], inp["w2"], y_na)
        torch.cuda.synchronize()
        S = int(host(buf["offsets"])[-1])
        assert S > 0
        assert torch.equal(y_na[:S], y_ws[:S])
        assert torch.isfinite(y_na[:S].float()).all()
        assert torch.isnan(y_na[S:].float()).all()     # rows past S untouched


def test_noalloc_rejects_sizes_beyond_the_scratch():
    dev = device()
    H, I, N = 6144, 2048, 512
    rows = 16384                                 # hh alone needs 64 MiB
    assert moe.moe_expert_ffn_workspace_bytes(rows, N, I, torch.bfloat16) > \
        moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((16, H), dtype=torch.bfloat16, device=dev)
    f = moe.lib().moe_expert_ffn_gather_noalloc
    p = x.data_ptr()
    st = f(p, 16, 1, p, p, rows, N, H, I, p, p, 1, p, None)
    assert st == 7, st                             # MOE_ERR_TOO_LARGE
    assert moe.lib().moe_status_string(7) == b"sizes exceed the fixed scratch"


def test_noalloc_call_captured_in_a_graph():
    """The entry point's purpose: captured into a HIP graph (its scratch
    address is looked up by the eager call before the capture) and replayed,
    it gives the eager result bit for bit on every replay."""
    dev = device()
    inp = workload.make_inputs(CFG, dev)
    buf = _routed(CFG, inp, dev)
    rows = CFG.T * CFG.K
    y = torch.empty((rows, CFG.H), dtype=torch.bfloat16, device=dev)

    def call():
        moe.moe_expert_ffn_gather_noalloc(inp["x"], CFG.K, buf["row_src"], buf["offsets"],
                                          inp["w13"], inp["w2"], y)

    call()
    torch.cuda.synchronize()
    S = int(host(buf["offsets"])[-1])
    ref = y[:S].clone()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y[:S], ref), rep
