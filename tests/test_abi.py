"""C-ABI library checks that need no GPU: it loads, exports every declared
symbol, sizes workspaces from the shape alone and rejects bad arguments on the
host before anything is enqueued."""
import ctypes
import os
import re

import pytest

from dropless_moe_dispatch_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dispatch.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared()
    assert {"moe_route_topk", "moe_build_index", "moe_expert_fwd", "moe_combine", "moe_expert_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert B.status_string(0) == "ok"
    assert "workspace" in B.status_string(B.MOE_ERR_WORKSPACE)
    assert B.status_string(99) == "unknown status"


def test_workspace_sizes_depend_on_shape_only():
    s = B.shape(16384, 2048, 128, 8, 768)
    sizes = [B.workspace_bytes(s, w) for w in range(8)]
    assert all(n > 0 for n in sizes)
    assert B.workspace_bytes(s, 8) == 0 and B.workspace_bytes(s, -1) == 0
    # the lean backward workspace is the full one without the [T*K, 2h] dH buffer
    assert sizes[B.MOE_WS_EXPERT_BWD] - sizes[B.MOE_WS_EXPERT_BWD_LEAN] == 16384 * 8 * 2 * 768 * 2
    # the H-only backward workspace adds exactly the [T*K, h] A' buffer (256-byte aligned)
    extra = sizes[B.MOE_WS_EXPERT_BWD_H] - sizes[B.MOE_WS_EXPERT_BWD]
    assert 16384 * 8 * 768 * 2 <= extra < 16384 * 8 * 768 * 2 + 256
    # the staged-Y ablation's workspace is the one that holds a T*K*d buffer
    assert sizes[B.MOE_WS_COMBINE_STAGED] >= 16384 * 8 * 2048 * 2
    # the dense-map index backend holds two [E][T] int32 maps
    assert 2 * 128 * 16384 * 4 <= sizes[B.MOE_WS_INDEX_DENSE] < 2 * 128 * 16384 * 4 + 1024
    # combine workspace holds the fp32 [T,d] fold accumulator, not a [T*K,d] buffer
    comb = sizes[B.MOE_WS_COMBINE]
    assert 16384 * 2048 * 4 <= comb < 16384 * 8 * 2048 * 2
    bad = B.shape(16, 100, 8, 2, 128)           # d not a multiple of 128
    assert B.workspace_bytes(bad, 0) == 0


FAKE = 0x10000  # 16-byte aligned fake device address: never dereferenced


@pytest.mark.parametrize("T,d,E,K,h,dt,code", [
    (0, 128, 8, 2, 128, "bf16", B.MOE_ERR_INVALID_ARG),
    (16, 128, 4, 5, 128, "bf16", B.MOE_ERR_INVALID_ARG),      # K > E
    (16, 128, 2000, 2, 128, "bf16", B.MOE_ERR_UNSUPPORTED),   # E > 1024
    (16, 128, 64, 40, 128, "bf16", B.MOE_ERR_UNSUPPORTED),    # K > 32
    (16, 96, 8, 2, 128, "bf16", B.MOE_ERR_UNSUPPORTED),       # d % 128
    (16, 128, 8, 2, 200, "f32", B.MOE_ERR_UNSUPPORTED),       # h % 128
    (1 << 29, 128, 8, 8, 128, "bf16", B.MOE_ERR_INVALID_ARG),  # T*K >= 2^31
    (1 << 20, 1024, 8, 2, 128, "bf16", B.MOE_ERR_UNSUPPORTED),   # x [T,d] of 2 GiB: past 32-bit offsets
    (1 << 19, 1024, 8, 2, 128, "f32", B.MOE_ERR_UNSUPPORTED),    # the same in fp32
    (64, 8192, 8, 2, 131072, "bf16", B.MOE_ERR_UNSUPPORTED),     # one expert's [h,d] of 2 GiB
    (1 << 18, 128, 8, 2, 2048, "bf16", B.MOE_ERR_UNSUPPORTED),   # T rows of [a|b]: 2^18 * 4096 * 2 B
])
def test_shape_validation_happens_on_host(T, d, E, K, h, dt, code):
    s = B.shape(T, d, E, K, h, dt)
    assert B.moe_route_topk(s, FAKE, FAKE, None, FAKE, FAKE, FAKE, stream=0, check=False) == code
    assert B.moe_build_index(s, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0, check=False, ws_bytes=1 << 40) == code


def test_pointer_and_workspace_validation():
    s = B.shape(64, 128, 8, 2, 128)
    L = B.lib()
    sp = ctypes.byref(s)
    # null required pointer
    assert L.moe_route_topk(sp, FAKE, FAKE, None, None, FAKE, FAKE, 0) == B.MOE_ERR_INVALID_ARG
    # misaligned pointer
    assert L.moe_build_index(sp, FAKE + 4, FAKE, FAKE, FAKE, FAKE, 1 << 30, 0) == B.MOE_ERR_INVALID_ARG
    # workspace too small
    need = B.workspace_bytes(s, B.MOE_WS_INDEX)
    assert L.moe_build_index(sp, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0) == B.MOE_ERR_WORKSPACE
    need = B.workspace_bytes(s, B.MOE_WS_COMBINE)
    assert L.moe_combine(sp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0) == B.MOE_ERR_WORKSPACE
    need = B.workspace_bytes(s, B.MOE_WS_EXPERT_FWD)
    assert L.moe_expert_fwd(sp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0) == B.MOE_ERR_WORKSPACE
    need = B.workspace_bytes(s, B.MOE_WS_EXPERT_BWD)

    def bwd_args():
        a = [FAKE] * 20          # dout .. dw_down
        a[13] = None             # a_prime: only with H-only saving
        a[14] = None             # dh: optional (the workspace holds it)
        return a
    req = bwd_args()
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need - 1, 0) == B.MOE_ERR_WORKSPACE   # ds is optional
    req[16] = None               # dwg missing
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need, 0) == B.MOE_ERR_INVALID_ARG
    # y_swi == NULL (H-only saving) needs the larger MOE_WS_EXPERT_BWD_H workspace ...
    req = bwd_args()
    req[12] = None               # y_swi
    need_h = B.workspace_bytes(s, B.MOE_WS_EXPERT_BWD_H)
    assert need_h > need
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need, 0) == B.MOE_ERR_WORKSPACE
    req[11] = None               # h_ab is still required
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need_h, 0) == B.MOE_ERR_INVALID_ARG
    # ... unless the caller gives A' a buffer of its own (the forward's dead y_swi)
    req = bwd_args()
    req[12], req[13] = None, FAKE + 0x100
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need - 1, 0) == B.MOE_ERR_WORKSPACE
    req[13] = FAKE + 0x104       # misaligned
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need, 0) == B.MOE_ERR_INVALID_ARG
    req[13] = req[11]            # A' over the saved a|b
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need, 0) == B.MOE_ERR_INVALID_ARG
    req = bwd_args()
    req[13] = FAKE + 0x100       # a saved y and an A' buffer: ambiguous
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need, 0) == B.MOE_ERR_INVALID_ARG
    # dH in a caller buffer: the lean workspace, dH's [T*K, 2h] smaller, suffices
    lean = B.workspace_bytes(s, B.MOE_WS_EXPERT_BWD_LEAN)
    assert lean == need - (64 * 2 * 2 * 128 * 2)

    def distinct_args():         # every buffer at an address of its own
        a = [FAKE + 0x1000 * i for i in range(20)]
        a[13] = a[14] = None
        return a
    req = distinct_args()
    req[14] = FAKE + 0x100000
    assert L.moe_expert_bwd(sp, *req, None, FAKE, lean - 1, 0) == B.MOE_ERR_WORKSPACE
    req[14] = req[11]            # dH over the saved a|b: allowed
    assert L.moe_expert_bwd(sp, *req, None, FAKE, lean - 1, 0) == B.MOE_ERR_WORKSPACE
    for bad in (req[12], req[0], req[1], req[15], FAKE + 0x100004):   # y_swi, dout, x, dx, misaligned
        req[14] = bad
        assert L.moe_expert_bwd(sp, *req, None, FAKE, need, 0) == B.MOE_ERR_INVALID_ARG
    req = distinct_args()
    req[12], req[14] = None, req[11]          # H-only with dH given needs an A' buffer too
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need_h, 0) == B.MOE_ERR_INVALID_ARG
    req[13] = FAKE + 0x200000
    assert L.moe_expert_bwd(sp, *req, None, FAKE, lean - 1, 0) == B.MOE_ERR_WORKSPACE
    req[14] = req[13]            # dH over A'
    assert L.moe_expert_bwd(sp, *req, None, FAKE, need_h, 0) == B.MOE_ERR_INVALID_ARG


def test_activation_kind_validation():
    L = B.lib()
    s = B.shape(64, 128, 8, 2, 128, act="relu")
    assert B.workspace_bytes(s, B.MOE_WS_EXPERT_FWD) > 0
    # a plain expert's backward workspace holds dH of width h, not 2h (256 rows
    # per expert: no dW row split, whose partials would differ too)
    g = B.shape(1024, 128, 8, 2, 1024)
    p = B.shape(1024, 128, 8, 2, 1024, act="silu")
    diff = B.workspace_bytes(g, B.MOE_WS_EXPERT_BWD) - B.workspace_bytes(p, B.MOE_WS_EXPERT_BWD)
    assert 1024 * 2 * 1024 * 2 <= diff < 1024 * 2 * 1024 * 2 + 512
    bad = B.shape(64, 128, 8, 2, 128)
    bad.act = 7
    assert B.workspace_bytes(bad, B.MOE_WS_INDEX) == 0
    assert L.moe_build_index(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 0) == B.MOE_ERR_INVALID_ARG
    # w_up is optional for a plain expert and required for SwiGLU
    need = B.workspace_bytes(s, B.MOE_WS_EXPERT_FWD)
    assert L.moe_expert_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need - 1, 0) \
        == B.MOE_ERR_WORKSPACE
    sg = B.shape(64, 128, 8, 2, 128)
    need = B.workspace_bytes(sg, B.MOE_WS_EXPERT_FWD)
    assert L.moe_expert_fwd(ctypes.byref(sg), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, 0) \
        == B.MOE_ERR_INVALID_ARG


def test_spin_limit_setter_roundtrip():
    prev = B.set_spin_limit(1000)
    assert B.set_spin_limit(0) == 1000          # polls <= 0 only reads
    assert B.set_spin_limit(prev) == 1000


def test_one_workspace_serves_forward_combine_and_backward():
    """The shared-workspace rule: every expert call's layout starts with the
    same carving, so the largest kind serves all three."""
    s = B.shape(16384, 2048, 128, 8, 768)
    fwd, comb, bwd = (B.workspace_bytes(s, k) for k in (B.MOE_WS_EXPERT_FWD, B.MOE_WS_COMBINE, B.MOE_WS_EXPERT_BWD))
    assert fwd < comb < bwd
    # the backward adds dH [T*K, 2h] and small buffers to the combine's carving;
    # it does not repeat the fp32 [T, d] accumulator
    dh = 16384 * 8 * 2 * 768 * 2
    assert dh <= bwd - comb < dh + 16384 * 2048 * 4
    # with dH in a caller buffer the backward needs the same carving without it
    lean = B.workspace_bytes(s, B.MOE_WS_EXPERT_BWD_LEAN)
    assert lean == bwd - dh and comb < lean
