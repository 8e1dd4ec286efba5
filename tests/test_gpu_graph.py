"""The layer forward captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library allocates nothing, sets no memory with hipMemset and
keeps no state between calls, so a captured forward must give, on every
replay, bit for bit what the eager calls give.  Each replay starts from
poisoned outputs, with eager work and host synchronisations in between."""
import pytest
import torch

import sparse_moe_layer_02_amd as moe
import workload
from _parity import device

pytestmark = pytest.mark.gpu

OUTS = ("logits", "topk_idx", "topk_gate", "counts", "offsets", "slot_row", "y")
ROWS = ("row_src", "y_perm")   # defined for the first S = offsets[-1] rows only


def _run(cfg, inp, buf):
    return moe.forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K,
                       cfg.scale, buf)


@pytest.mark.parametrize("path", ["fused", "six_calls_two_streams"])
def test_captured_forward_replays_match_eager(path):
    dev = device()
    # T = 1024 reaches the six-call path's second stream (identity experts
    # beside dispatch and the GEMMs), and the mid shape has experts of more
    # than 256 rows (full-tile and partial-tile GEMM launches)
    cfg = workload.CONFIGS["mid_bf16"].replace(T=1024)
    print(f"\n[case] graph capture {path} {cfg.name} T={cfg.T}", flush=True)
    inp = workload.make_inputs(cfg, dev)
    kw = {} if path == "fused" else {"separate_identity": True}
    buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev, **kw)
    _run(cfg, inp, buf)
    torch.cuda.synchronize(dev)
    ref = {k: buf[k].clone() for k in OUTS}
    S = int(ref["offsets"][-1].item())
    ref_rows = {k: buf[k][:S].clone() for k in ROWS}

    # warm up on a side stream, then capture
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        _run(cfg, inp, buf)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(cfg, inp, buf)
    torch.cuda.synchronize(dev)

    other = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for k in OUTS:
            if buf[k].dtype.is_floating_point:
                buf[k].fill_(float("nan"))
            else:
                buf[k].fill_(-7)
        buf["y_perm"].fill_(float("nan"))
        buf["row_src"].fill_(-7)
        other.mul_(1.0001)               # eager work between the replays
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        for k in OUTS:
            assert torch.equal(buf[k], ref[k]), (rep, k)
        for k in ROWS:
            assert torch.equal(buf[k][:S], ref_rows[k]), (rep, k)
    assert int(buf["status"].item()) == 0
