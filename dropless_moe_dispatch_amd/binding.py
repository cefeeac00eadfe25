"""Thin ctypes binding over libmoe_dispatch.so.

Argument marshalling only: torch tensors are passed as device pointers plus
the current HIP stream; every step of the layer runs in the library's HIP
kernels.  There is no fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libmoe_dispatch.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_F32, MOE_BF16 = 0, 1
MOE_WS_INDEX, MOE_WS_EXPERT_FWD, MOE_WS_COMBINE, MOE_WS_EXPERT_BWD, MOE_WS_EXPERT_BWD_H = 0, 1, 2, 3, 4
MOE_WS_COMBINE_STAGED = 5
MOE_WS_INDEX_DENSE = 6
MOE_WS_EXPERT_BWD_LEAN = 7


MOE_ACT_SWIGLU, MOE_ACT_SILU, MOE_ACT_RELU = 0, 1, 2
ACTS = {"swiglu": MOE_ACT_SWIGLU, "silu": MOE_ACT_SILU, "relu": MOE_ACT_RELU}


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
                ("h", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


class MoeDeviceError(RuntimeError):
    """A bounded wait of an ordered fold ran out on the device: the call
    returned MOE_OK when it enqueued, but its output (out or dx) is invalid."""


_lib = None
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                              "(run dropless_moe_dispatch_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        sp = ctypes.POINTER(MoeShape)
        L.moe_workspace_bytes.argtypes = [sp, ctypes.c_int]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_route_topk.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P]
        L.moe_build_index.argtypes = [sp, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_build_index_dense.argtypes = [sp, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_build_index_noalloc.argtypes = [sp, _P, _P, _P, _P, _P]
        L.moe_build_index_noalloc.restype = ctypes.c_int
        L.moe_expert_fwd.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_combine.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_combine_staged.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_expert_bwd.argtypes = [sp] + [_P] * 22 + [ctypes.c_size_t, _P]
        for f in ("moe_route_topk", "moe_build_index", "moe_build_index_dense", "moe_expert_fwd", "moe_combine", "moe_combine_staged", "moe_expert_bwd"):
            getattr(L, f).restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_set_spin_limit.argtypes = [ctypes.c_int]
        L.moe_set_spin_limit.restype = ctypes.c_int
        L.moe_timing_enable.argtypes = [ctypes.c_int]
        L.moe_timing_enable.restype = ctypes.c_int
        L.moe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.moe_timing_read.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().moe_status_string(code).decode()


def shape(T, d, E, K, h, dtype="bf16", act="swiglu") -> MoeShape:
    """act: "swiglu" (gated expert), "silu" or "relu" (plain two-layer expert)."""
    return MoeShape(T, d, E, K, h, MOE_BF16 if dtype == "bf16" else MOE_F32, ACTS[act])


def workspace_bytes(s: MoeShape, which: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(s), which))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def _nbytes(t):
    return t.numel() * t.element_size()


def moe_route_topk(s, x, wg, bias, logits, topk_ids, topk_w, stream=None, check=True):
    rc = lib().moe_route_topk(ctypes.byref(s), _ptr(x), _ptr(wg), _ptr(bias), _ptr(logits), _ptr(topk_ids),
                              _ptr(topk_w), _stream(stream))
    if check:
        _check("moe_route_topk", rc)
    return rc


def moe_build_index(s, topk_ids, offsets, eti, tim, ws, stream=None, check=True, ws_bytes=None):
    rc = lib().moe_build_index(ctypes.byref(s), _ptr(topk_ids), _ptr(offsets), _ptr(eti), _ptr(tim), _ptr(ws),
                               _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    if check:
        _check("moe_build_index", rc)
    return rc


def moe_build_index_noalloc(s, topk_ids, offsets, eti, tim, stream=None, check=True):
    """moe_build_index with the library's static per-GPU scratch instead of a workspace."""
    rc = lib().moe_build_index_noalloc(ctypes.byref(s), _ptr(topk_ids), _ptr(offsets), _ptr(eti), _ptr(tim),
                                       _stream(stream))
    if check:
        _check("moe_build_index_noalloc", rc)
    return rc


def moe_build_index_dense(s, topk_ids, offsets, eti, tim, ws, stream=None, check=True, ws_bytes=None):
    """The same index through MoEBlaze's literal three steps (dense [E][T] map)."""
    rc = lib().moe_build_index_dense(ctypes.byref(s), _ptr(topk_ids), _ptr(offsets), _ptr(eti), _ptr(tim), _ptr(ws),
                                     _nbytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    if check:
        _check("moe_build_index_dense", rc)
    return rc


def moe_expert_fwd(s, x, offsets, eti, w_gate, w_up, h_ab, y_swi, ws, stream=None, check=True):
    rc = lib().moe_expert_fwd(ctypes.byref(s), _ptr(x), _ptr(offsets), _ptr(eti), _ptr(w_gate), _ptr(w_up),
                              _ptr(h_ab), _ptr(y_swi), _ptr(ws), _nbytes(ws), _stream(stream))
    if check:
        _check("moe_expert_fwd", rc)
    return rc


def moe_combine(s, y_swi, w_down, offsets, eti, tim, topk_ids, topk_w, out, ws, stream=None, check=True):
    rc = lib().moe_combine(ctypes.byref(s), _ptr(y_swi), _ptr(w_down), _ptr(offsets), _ptr(eti), _ptr(tim),
                           _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))
    if check:
        _check("moe_combine", rc)
    return rc


def moe_combine_staged(s, y_swi, w_down, offsets, eti, tim, topk_ids, topk_w, out, ws, stream=None, check=True):
    """Staged-Y combine (ablation of moe_combine; materialises a [T*K, d] buffer)."""
    rc = lib().moe_combine_staged(ctypes.byref(s), _ptr(y_swi), _ptr(w_down), _ptr(offsets), _ptr(eti), _ptr(tim),
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))
    if check:
        _check("moe_combine_staged", rc)
    return rc


def moe_expert_bwd(s, dout, x, wg, w_gate, w_up, w_down, topk_ids, topk_w, offsets, eti, tim, h_ab, y_swi,
                   a_prime, dh, dx, dwg, dw_gate, dw_up, dw_down, ds, ws, stream=None, check=True):
    rc = lib().moe_expert_bwd(ctypes.byref(s), _ptr(dout), _ptr(x), _ptr(wg), _ptr(w_gate), _ptr(w_up),
                              _ptr(w_down), _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(eti), _ptr(tim),
                              _ptr(h_ab), _ptr(y_swi), _ptr(a_prime), _ptr(dh), _ptr(dx), _ptr(dwg),
                              _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(ds), _ptr(ws), _nbytes(ws),
                              _stream(stream))
    if check:
        _check("moe_expert_bwd", rc)
    return rc


def set_spin_limit(polls: int) -> int:
    return int(lib().moe_set_spin_limit(polls))


def timing_enable(on: bool) -> bool:
    return bool(lib().moe_timing_enable(1 if on else 0))


def timing_read(cap: int = 4096):
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = lib().moe_timing_read(names, ms, cap)
    return [(names[i].decode(), float(ms[i])) for i in range(n)]
