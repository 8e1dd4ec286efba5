"""The C-ABI boundary on the host: the library loads, exports every function
include/moe_mi355x.h declares, and rejects bad arguments with status codes
before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest
import torch

import sparse_moe_layer_02_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")
OK, NULL, SHAPE, DTYPE, ALIGN, WS = 0, 1, 2, 3, 4, 5
P = ctypes.c_void_p
FAKE = P(0x10000)        # never dereferenced: validation fails first or only sizes are read


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    names = declared_functions()
    assert len(names) == 21, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe._SIGS)


def test_status_strings():
    lib = moe.lib()
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(WS) == b"workspace too small"
    assert lib.moe_status_string(99) == b"unknown status"


def test_workspace_queries():
    lib = moe.lib()
    # the FFN workspace holds the intermediate activations: rows x I elements
    b16 = lib.moe_expert_ffn_workspace_bytes(98304, 512, 2048, 1)
    f32 = lib.moe_expert_ffn_workspace_bytes(98304, 512, 2048, 0)
    assert b16 >= 98304 * 2048 * 2 and f32 >= 98304 * 2048 * 4
    assert lib.moe_expert_ffn_workspace_bytes(10, 4, 64, 7) == 0


def test_router_logits_validation():
    f = moe.lib().moe_router_logits
    assert f(None, 1, FAKE, 4, 64, 8, FAKE, None) == NULL
    assert f(FAKE, 5, FAKE, 4, 64, 8, FAKE, None) == DTYPE
    assert f(FAKE, 1, FAKE, 0, 64, 8, FAKE, None) == SHAPE
    assert f(FAKE, 1, FAKE, 4, 64, 0, FAKE, None) == SHAPE
    assert f(P(0x10001), 1, FAKE, 4, 64, 8, FAKE, None) == ALIGN


def test_router_planes_validation():
    split = moe.lib().moe_router_split_weights
    assert split(None, 8, 64, FAKE, None) == NULL
    assert split(FAKE, 8, 64, None, None) == NULL
    assert split(FAKE, 0, 64, FAKE, None) == SHAPE
    assert split(FAKE, 8, 60, FAKE, None) == SHAPE          # H % 8
    assert split(P(0x10004), 8, 64, FAKE, None) == ALIGN    # 16-byte vectors
    assert split(FAKE, 8, 64, P(0x10008), None) == ALIGN
    f = moe.lib().moe_router_logits_planes
    assert f(None, 1, FAKE, FAKE, 4, 64, 8, FAKE, None) == NULL
    assert f(FAKE, 1, None, FAKE, 4, 64, 8, FAKE, None) == NULL   # w_router stays required
    assert f(FAKE, 5, FAKE, FAKE, 4, 64, 8, FAKE, None) == DTYPE
    assert f(FAKE, 1, FAKE, FAKE, 0, 64, 8, FAKE, None) == SHAPE
    assert f(FAKE, 1, FAKE, FAKE, 4, 60, 8, FAKE, None) == SHAPE  # planes need H % 8
    assert f(FAKE, 1, FAKE, P(0x10008), 4, 64, 8, FAKE, None) == ALIGN


def test_route_validation():
    f = moe.lib().moe_route
    args = [FAKE, FAKE, 16, 24, 4, FAKE, FAKE, FAKE, None, None]
    a = list(args); a[0] = None
    assert f(*a) == NULL
    a = list(args); a[4] = 0
    assert f(*a) == SHAPE
    a = list(args); a[4] = 25                     # K > E
    assert f(*a) == SHAPE
    a = list(args); a[3] = 1025; a[4] = 4         # E beyond one wave's 16 keys per lane
    assert f(*a) == SHAPE
    a = list(args); a[2] = 1 << 28; a[4] = 16     # T*K >= 2^31
    assert f(*a) == SHAPE
    a = list(args); a[8] = P(0x10002)
    assert f(*a) == ALIGN


def test_permute_validation():
    f = moe.lib().moe_permute
    args = [FAKE, 1, FAKE, FAKE, 64, 256, 4, 16, FAKE, FAKE, FAKE, FAKE, None]
    a = list(args); a[3] = None                   # counts are required
    assert f(*a) == NULL
    a = list(args); a[5] = 250                    # H not a multiple of 8
    assert f(*a) == SHAPE
    a = list(args); a[7] = 5000                   # too many FFN experts
    assert f(*a) == SHAPE
    a = list(args); a[9] = P(0x10008)             # x_perm not 16-byte aligned
    assert f(*a) == ALIGN
    a = list(args); a[3] = P(0x10002)             # counts not 4-byte aligned
    assert f(*a) == ALIGN
    a = list(args); a[0] = None                   # x without x_perm to copy into
    assert f(*a) == NULL
    a = list(args); a[0] = None; a[9] = None      # indices only (no copy): x unused
    a[7] = 5000
    assert f(*a) == SHAPE                         # still validated past the NULL check
    a = list(args); a[10] = None                  # row_src is always written
    assert f(*a) == NULL
    a = list(args); a[4] = 1 << 28; a[6] = 16     # T*K >= 2^31
    assert f(*a) == SHAPE


def test_expert_ffn_validation():
    f = moe.lib().moe_expert_ffn
    need = moe.lib().moe_expert_ffn_workspace_bytes(256, 16, 1024, 1)
    args = [FAKE, FAKE, 256, 16, 2048, 1024, FAKE, FAKE, 1, FAKE, FAKE, need, None]
    a = list(args); a[6] = None
    assert f(*a) == NULL
    a = list(args); a[4] = 2000                   # bf16 path needs H % 128 == 0
    assert f(*a) == SHAPE
    a = list(args); a[5] = 1000                   # and I % 64 == 0
    assert f(*a) == SHAPE
    a = list(args); a[11] = need - 1
    assert f(*a) == WS
    a = list(args); a[8] = 9
    assert f(*a) == DTYPE
    a = list(args); a[3] = 0                      # no FFN experts: nothing to do
    assert f(*a) == OK
    a[6] = a[7] = None                            # ... and no weights needed
    assert f(*a) == OK


def test_expert_ffn_gather_validation():
    f = moe.lib().moe_expert_ffn_gather
    need = moe.lib().moe_expert_ffn_workspace_bytes(256, 16, 1024, 1)
    args = [FAKE, 64, 4, FAKE, FAKE, 256, 16, 2048, 1024, FAKE, FAKE, 1, FAKE, FAKE, need, None]
    a = list(args); a[3] = None                   # row_src
    assert f(*a) == NULL
    a = list(args); a[0] = None                   # x
    assert f(*a) == NULL
    a = list(args); a[1] = 0                      # T
    assert f(*a) == SHAPE
    a = list(args); a[2] = 0                      # K
    assert f(*a) == SHAPE
    a = list(args); a[1] = 1 << 28; a[2] = 8      # T*K >= 2^31
    assert f(*a) == SHAPE
    a = list(args); a[7] = 2000                   # bf16 path needs H % 128 == 0
    assert f(*a) == SHAPE
    a = list(args); a[0] = P(0x10008)             # x rows not 16-byte aligned
    assert f(*a) == ALIGN
    a = list(args); a[3] = P(0x10002)             # row_src not int-aligned
    assert f(*a) == ALIGN
    a = list(args); a[14] = need - 1
    assert f(*a) == WS
    a = list(args); a[6] = 0                      # no FFN experts: nothing to do
    assert f(*a) == OK
    a[9] = a[10] = None                           # ... and no weights needed
    assert f(*a) == OK


def test_zero_and_combine_validation():
    z = moe.lib().moe_zero_experts
    assert z(FAKE, 1, FAKE, FAKE, 8, 100, 4, 2, FAKE, None) == SHAPE
    assert z(FAKE, 1, FAKE, None, 8, 128, 4, 2, FAKE, None) == NULL
    c = moe.lib().moe_combine
    assert c(FAKE, 1, FAKE, FAKE, ctypes.c_float(1.0), FAKE, 8, 128, 2000, FAKE, None) == SHAPE
    assert c(FAKE, 1, FAKE, FAKE, ctypes.c_float(1.0), FAKE, 8, 128, 4, P(0x10004), None) == ALIGN


def test_combine_identity_validation():
    f = moe.lib().moe_combine_identity
    one = ctypes.c_float(1.0)
    args = [FAKE, FAKE, 1, FAKE, FAKE, one, 8, 128, 4, FAKE, None]
    a = list(args); a[1] = None                   # x
    assert f(*a) == NULL
    a = list(args); a[3] = None                   # slot_row
    assert f(*a) == NULL
    a = list(args); a[2] = 3
    assert f(*a) == DTYPE
    a = list(args); a[7] = 100                    # H % 8
    assert f(*a) == SHAPE
    a = list(args); a[8] = 2000                   # K beyond the slot list
    assert f(*a) == SHAPE
    a = list(args); a[6] = 0
    assert f(*a) == SHAPE
    a = list(args); a[1] = P(0x10008)             # x rows not 16-byte aligned
    assert f(*a) == ALIGN
    a = list(args); a[9] = P(0x10004)             # y
    assert f(*a) == ALIGN


def test_forward_validation():
    # the one-call forward runs every check of its five calls before any of
    # them, so a bad argument enqueues nothing (here: no HIP call at all)
    lib = moe.lib()
    q = lib.moe_forward_workspace_bytes
    assert q(8, 128, 24, 16, 64, 4, 1) > 0
    assert q(0, 128, 24, 16, 64, 4, 1) == 0 and q(8, 128, 24, 30, 64, 4, 1) == 0
    assert q(8, 128, 24, 16, 64, 4, 7) == 0
    ws_bytes = q(8, 128, 24, 16, 64, 4, 1)
    f = lib.moe_forward
    one = ctypes.c_float(1.0)
    # x, dtype, w_router, w_planes, bias, w13, w2, T, H, E, n_ffn, I, K, s, y, status, ws, bytes
    args = [FAKE, 1, FAKE, None, FAKE, FAKE, FAKE, 8, 128, 24, 16, 64, 4, one, FAKE, None, FAKE,
            ws_bytes, None]
    for i in (0, 2, 4, 14, 16):                   # x, w_router, bias, y, ws
        a = list(args); a[i] = None
        assert f(*a) == NULL, i
    a = list(args); a[5] = None                   # FFN weights, with FFN experts
    assert f(*a) == NULL
    a = list(args); a[10] = 0; a[5] = a[6] = None   # no FFN experts: no weights needed,
    a[17] = 1                                     # so the workspace is the failing check
    assert f(*a) == WS
    a = list(args); a[1] = 4
    assert f(*a) == DTYPE
    for i, v in ((7, 0), (8, 100), (8, 64), (9, 2000), (12, 0), (12, 25), (10, 25), (11, 32)):
        a = list(args); a[i] = v                  # T, H % 8, bf16 H % 128, E, K, K > E, n_ffn > E, I % 64
        assert f(*a) == SHAPE, (i, v)
    for i in (0, 3, 14):                          # x, w_planes, y: 16 bytes
        a = list(args); a[i] = P(0x10008)
        assert f(*a) == ALIGN, i
    a = list(args); a[16] = P(0x10080)            # ws: 256 bytes
    assert f(*a) == ALIGN
    a = list(args); a[17] = ws_bytes - 1
    assert f(*a) == WS


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_router_logits(x, torch.zeros((8, 64)), torch.zeros((4, 8)))


def test_bias_update_validation():
    f = moe.lib().moe_bias_update
    F = ctypes.c_float
    args = [FAKE, 64, 16, F(2.0), F(1.0), F(0.05), F(0.2), FAKE, FAKE, FAKE, None]
    a = list(args); a[7] = None
    assert f(*a) == NULL
    a = list(args); a[1] = 0                      # no tokens
    assert f(*a) == SHAPE
    a = list(args); a[2] = 0                      # no FFN experts
    assert f(*a) == SHAPE
    a = list(args); a[2] = 5000                   # beyond 4096
    assert f(*a) == SHAPE
    a = list(args); a[3] = F(float("nan"))        # non-finite target
    assert f(*a) == SHAPE
    a = list(args); a[6] = F(float("inf"))        # non-finite gain
    assert f(*a) == SHAPE
    a = list(args); a[8] = P(0x10002)
    assert f(*a) == ALIGN


def test_router_similarity_validation():
    lib = moe.lib()
    f = lib.moe_router_similarity
    need = lib.moe_router_similarity_workspace_bytes(768, 6144)
    # partial 64 x 64 Gram tiles of 78 triangle tiles, at least one K split
    assert need >= 78 * 64 * 64 * 4
    assert lib.moe_router_similarity_workspace_bytes(768, 6) == 0        # H % 4
    assert lib.moe_router_similarity_workspace_bytes(0, 64) == 0
    assert lib.moe_router_similarity_workspace_bytes(50000, 64) == 0     # E * E >= 2^31
    args = [FAKE, 768, 6144, FAKE, FAKE, FAKE, need, None]
    a = list(args); a[4] = None
    assert f(*a) == NULL
    a = list(args); a[2] = 6142
    assert f(*a) == SHAPE
    a = list(args); a[1] = 0
    assert f(*a) == SHAPE
    a = list(args); a[0] = P(0x10004)                  # w_router needs 16 bytes
    assert f(*a) == ALIGN
    a = list(args); a[5] = P(0x10080)                  # workspace needs 256 bytes
    assert f(*a) == ALIGN
    a = list(args); a[6] = need - 1
    assert f(*a) == WS


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no fallback: without the shared library every call raises
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()
    with pytest.raises(RuntimeError, match="missing"):
        moe.moe_expert_ffn_workspace_bytes(64, 12, 512, torch.bfloat16)
