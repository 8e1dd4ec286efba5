"""The expert GEMMs alone, through moe_expert_ffn and moe_expert_ffn_gather,
against the oracle's FFN rows, with crafted rows per expert: every number of
32-row groups from 1 to 8, a partial tile of 225-255 rows, full 256-row
tiles and experts spanning several tiles.  Hidden sizes that are multiples of
192 select the down GEMM's 192-row weight tiles for tiles of up to 224 rows
(128-row ones for the rest); the others use 128-row tiles throughout.  At
2I = 512 the gate/up GEMM's partial tiles of 2-5 groups take 256-row weight
tiles; where H is a multiple of 512 (H = 1024, 1536) the down GEMM's last
m-tiles of up to 4 groups take 512-row weight tiles."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_02_amd as moe
from _parity import THREADS, TOL, device, host, normwise

pytestmark = pytest.mark.gpu

ROWS = [1, 40, 70, 100, 150, 180, 200, 224, 230, 256, 300, 513, 17]


@pytest.mark.parametrize("H,I", [(384, 128), (768, 256), (640, 192), (1024, 256), (1536, 256)])
def test_expert_rows_match_oracle(H, I):
    dev = device()
    print(f"\n[case] expert FFN H={H} I={I} rows {ROWS}", flush=True)
    N = len(ROWS)
    S = sum(ROWS)
    K = 3
    T = (S + K - 1) // K
    g = torch.Generator(device="cpu").manual_seed(H + I)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w13 = (torch.randn(N, 2 * I, H, generator=g) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(N, H, I, generator=g) * 0.05).to(torch.bfloat16)
    # row r reads token (r * 7919) % T (a scattered gather), slot 0
    rs = ((torch.arange(S) * 7919) % T * K).to(torch.int32)
    offsets = torch.tensor(np.r_[0, np.cumsum(ROWS)], dtype=torch.int32)
    xd, w13d, w2d = x.to(dev), w13.to(dev), w2.to(dev)
    x_perm = xd[(rs // K).long().to(dev)].contiguous()
    ws = torch.empty(moe.moe_expert_ffn_workspace_bytes(S, N, I, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    y_copy = torch.empty(S, H, dtype=torch.bfloat16, device=dev)
    y_gath = torch.empty(S, H, dtype=torch.bfloat16, device=dev)
    moe.moe_expert_ffn(x_perm, offsets.to(dev), w13d, w2d, y_copy, ws)
    moe.moe_expert_ffn_gather(xd, K, rs.to(dev), offsets.to(dev), w13d, w2d, y_gath, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_copy, y_gath)
    xp = x.float().numpy()[(rs // K).numpy()]
    yp = host(y_gath)
    off = offsets.numpy()
    for e in range(N):
        a, b = int(off[e]), int(off[e + 1])
        ref = oracle.ffn_rows(xp[a:b], w13[e].float().numpy(), w2[e].float().numpy(),
                              threads=THREADS)
        err = normwise(yp[a:b], ref)
        assert err <= TOL["bf16"], (e, ROWS[e], err)
