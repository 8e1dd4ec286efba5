"""Output integrity checks of the whole forward pass through the C ABI.

Silent-data-corruption analogue: the LongCat-Flash Technical Report notes
(Key claims [§1, §3.1.3]) rely on deterministic computation so that two runs
of the same step can be compared bit for bit.  Here a layer's outputs are
digested, a second run must reproduce the digest exactly, a single flipped
bit in one expert weight (a host write, as a memory error would leave it)
must change it, and restoring the bit must bring it back.

Canary bands: every buffer the forward pass writes is a view into a larger
allocation whose bands before and after it hold a known byte pattern; after
the pass the bands must be untouched.
"""
import hashlib

import numpy as np
import pytest
import torch

import sparse_moe_layer_02_amd as moe
import workload
from _parity import device, host

pytestmark = pytest.mark.gpu

CFG = workload.CONFIGS["mid_bf16"].replace(T=1024)
GUARD = 4096            # bytes of canary before and after each buffer
PATTERN = 0xA5


def _digest(buf):
    h = hashlib.sha256()
    for k in ("logits", "topk_idx", "topk_gate", "counts", "offsets", "y"):
        h.update(buf[k].detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    S = int(host(buf["offsets"])[-1])
    h.update(buf["y_perm"][:S].detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def _run(inp, buf):
    moe.forward(inp["x"], inp["w_router"], inp["bias"], inp["w13"], inp["w2"], CFG.K, CFG.scale,
                buf)
    torch.cuda.synchronize()


def test_deterministic_digest_catches_a_flipped_weight_bit():
    dev = device()
    inp = workload.make_inputs(CFG, dev)
    buf = moe.alloc_buffers(CFG.T, CFG.H, CFG.E, CFG.N, CFG.I, CFG.K, CFG.torch_dtype, dev)
    _run(inp, buf)
    d0 = _digest(buf)
    _run(inp, buf)
    assert _digest(buf) == d0, "two runs of the same layer differ"
    # flip one mantissa bit of a gate weight of the busiest expert
    e = int(np.argmax(host(buf["counts"])[:CFG.N]))
    w = inp["w13"][e].view(torch.int16)
    old = w[0, 0].clone()
    w[0, 0] = old ^ 0x0004
    torch.cuda.synchronize()
    _run(inp, buf)
    d1 = _digest(buf)
    assert d1 != d0, "a flipped weight bit left the outputs unchanged"
    w[0, 0] = old
    torch.cuda.synchronize()
    _run(inp, buf)
    assert _digest(buf) == d0, "restoring the bit did not restore the outputs"


def _guarded(shape, dtype, dev):
    """A tensor of `shape` inside an allocation with GUARD canary bytes on
    both sides (16-byte aligned); returns (tensor, whole uint8 buffer)."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    n16 = (n + 15) // 16 * 16
    raw = torch.full((GUARD + n16 + GUARD,), PATTERN, dtype=torch.uint8, device=dev)
    t = raw[GUARD:GUARD + n].view(dtype).view(shape)
    return t, raw, n


def _bands_intact(raw, n):
    h = host(raw)
    return bool((h[:GUARD] == PATTERN).all() and (h[GUARD + n:] == PATTERN).all())


@pytest.mark.parametrize("path", ["fast", "stages"])
def test_canary_bands_around_every_output_are_untouched(path):
    dev = device()
    inp = workload.make_inputs(CFG, dev)
    kw = {} if path == "fast" else {"grouped_copy": True, "separate_identity": True}
    buf = moe.alloc_buffers(CFG.T, CFG.H, CFG.E, CFG.N, CFG.I, CFG.K, CFG.torch_dtype, dev, **kw)
    raws = {}
    for k in ("logits", "topk_idx", "topk_gate", "counts", "offsets", "row_src", "slot_row",
              "y_perm", "ws_ffn", "y", "x_perm", "y_acc"):
        if buf.get(k) is None:
            continue
        t, raw, n = _guarded(tuple(buf[k].shape), buf[k].dtype, dev)
        buf[k] = t
        raws[k] = (raw, n)
    _run(inp, buf)
    bad = [k for k, (raw, n) in raws.items() if not _bands_intact(raw, n)]
    assert not bad, f"canary bands overwritten around {bad}"
    # the pass itself was complete: every token's output is finite
    assert torch.isfinite(buf["y"].float()).all()
