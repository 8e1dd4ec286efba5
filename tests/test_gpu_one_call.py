"""moe_forward, the whole layer in one C call, against the five calls of
forward()'s default path: the same y bit for bit and the same routing in its
workspace, and against the oracle end to end."""
import numpy as np
import pytest
import torch

import sparse_moe_layer_02_amd as moe
import workload
from _parity import TOL, check_end_to_end, device, forward, host, inputs_on_host

pytestmark = pytest.mark.gpu


def _al(b):
    return (b + 255) // 256 * 256


CASES = [
    ("tiny_fp32", {}, None, True),
    ("mid_bf16", {"T": 1500}, (3,), True),      # one expert takes nearly every token
    ("mid_bf16", {"T": 1}, None, False),
    ("tiny_fp32", {"N": 0, "Z": 16, "T": 200}, None, False),   # identity experts only
    ("mid_bf16", {"N": 24, "Z": 0, "T": 300}, None, True),     # FFN experts only
]


@pytest.mark.parametrize("name,over,heavy,planes", CASES,
                         ids=[f"{c[0]}-{'-'.join(f'{k}{v}' for k, v in c[1].items())}"
                              f"-heavy{bool(c[2])}-planes{c[3]}" for c in CASES])
def test_one_call_matches_the_five_calls(name, over, heavy, planes):
    cfg = workload.CONFIGS[name].replace(**over)
    dev = device()
    print(f"\n[case] {cfg} heavy={heavy} planes={planes}", flush=True)
    inp = workload.make_inputs(cfg, dev)
    if heavy:
        bias = host(inp["bias"]).copy()
        bias[list(heavy)] += 6.0 * cfg.sigma_w * np.sqrt(2.0 * cfg.H)
        inp["bias"] = torch.as_tensor(bias, dtype=torch.float32, device=dev)
    buf = moe.alloc_buffers(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K, cfg.torch_dtype, dev)
    if planes:
        moe.prepare_router(inp["w_router"], buf)
    y_ref = forward(cfg, inp, buf).clone()

    nbytes = moe.moe_forward_workspace_bytes(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K,
                                             cfg.torch_dtype)
    assert nbytes > 0
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=dev)
    y = torch.full_like(y_ref, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.moe_forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K,
                    cfg.scale, y, ws, w_planes=buf.get("w_planes"), dev_status=status)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert int(status[0]) == 0

    # the routing the call left in its workspace: logits, then topk_idx
    T, E, K = cfg.T, cfg.E, cfg.K
    off_idx = _al(T * E * 4)
    idx = ws[off_idx:off_idx + T * K * 4].view(torch.int32).view(T, K)
    assert torch.equal(idx, buf["topk_idx"])
    if heavy:
        counts = host(buf["counts"])[:cfg.N]
        assert counts[heavy[0]] >= 0.9 * T   # several 256-row m-tiles

    h = inputs_on_host(inp)
    err, flips = check_end_to_end(cfg, h["x"], h["w_router"], h["bias"], h["w13"], h["w2"],
                                  host(y), host(idx))
    print(f"end-to-end normwise {err:.3e}, flipped tokens {flips}", flush=True)
    assert err <= TOL[cfg.dtype]


def test_one_call_captured_replays_match_eager():
    # moe_forward allocates nothing and sets no memory with hipMemset: captured
    # into a HIP graph (torch.cuda.CUDAGraph) it must give on every replay,
    # from a poisoned workspace and output, bit for bit the eager y
    dev = device()
    cfg = workload.CONFIGS["mid_bf16"].replace(T=1024)
    print(f"\n[case] graph capture of moe_forward {cfg.name} T={cfg.T}", flush=True)
    inp = workload.make_inputs(cfg, dev)
    nbytes = moe.moe_forward_workspace_bytes(cfg.T, cfg.H, cfg.E, cfg.N, cfg.I, cfg.K,
                                             cfg.torch_dtype)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    y = torch.empty((cfg.T, cfg.H), dtype=cfg.torch_dtype, device=dev)

    def run():
        moe.moe_forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], cfg.K,
                        cfg.scale, y, ws)

    run()
    torch.cuda.synchronize(dev)
    ref = y.clone()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize(dev)
    other = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xAB)
        other.mul_(1.0001)
        torch.cuda.synchronize(dev)
        graph.replay()
        other.add_(1.0)
        torch.cuda.synchronize(dev)
        assert torch.equal(y, ref), f"replay {rep}"
