"""Python binding of libmoe_decode.so, the MI355X routed-expert MoE decode layer.

The functions carry the names of the C ABI in include/moe_decode.h and only marshal arguments:
torch device tensors become raw device pointers, the stream defaults to torch's current stream,
and a negative status raises MoeError.  Every step of the layer runs in the HIP kernels; there is
no other implementation to fall back to, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_decode.so")

MOE_FMT_F32, MOE_FMT_BF16, MOE_FMT_MXFP4, MOE_FMT_FP8 = 0, 1, 2, 3
MOE_OK = 0
MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_FORMAT, MOE_ERR_WORKSPACE = -1, -2, -3, -4
MOE_ERR_OFFSETS, MOE_ERR_HIP, MOE_ERR_ALIGN, MOE_ERR_TIMEOUT = -5, -6, -7, -8
MOE_ERR_SCRATCH = -9
MOE_NOALLOC_SCRATCH_BYTES = 2138112
MOE_MAX_TOKENS, MOE_MAX_EXPERTS, MOE_MAX_TOPK = 16, 512, 16

EXPORTED = ("moe_workspace_bytes", "moe_route", "moe_decode_forward", "moe_decode_forward_noalloc",
            "moe_lm_head", "moe_read_status", "moe_status_string")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, moe_status_string(status), status))
        self.status = status


MOE_ROUTER_NORM, MOE_ROUTER_BIAS = 1, 2


class moe_desc_t(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("act_format", ctypes.c_int32), ("weight_format", ctypes.c_int32),
                ("router_flags", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("norm_weight", ctypes.c_void_p), ("router_bias", ctypes.c_void_p)]


class moe_lm_head_desc_t(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32), ("weight_format", ctypes.c_int32)]


class moe_weights_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate", "up", "down", "gate_s", "up_s", "down_s",
                 "sh_gate", "sh_up", "sh_down", "sh_gate_s", "sh_up_s", "sh_down_s")]


class moe_dispatch_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("unit_count", "unit_expert", "unit_off", "row_token", "row_slot", "row_weight", "req_unique")]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmoe_decode.so is not built (%s); run __graft_entry__.build() or "
                              "python moe_speculative_decode_amd/build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(moe_desc_t)]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [ctypes.POINTER(moe_desc_t), i32, vp, vp, vp, vp, ctypes.POINTER(moe_dispatch_t),
                                vp, sz, vp]
        L.moe_decode_forward.restype = ctypes.c_int
        L.moe_decode_forward.argtypes = [ctypes.POINTER(moe_desc_t), i32, vp, vp, ctypes.POINTER(moe_weights_t),
                                         vp, i32, vp, vp, vp, ctypes.POINTER(moe_dispatch_t), vp, sz, vp]
        L.moe_decode_forward_noalloc.restype = ctypes.c_int
        L.moe_decode_forward_noalloc.argtypes = [ctypes.POINTER(moe_desc_t), i32, vp, vp, ctypes.POINTER(moe_weights_t),
                                                 vp, i32, vp, vp, vp, ctypes.POINTER(moe_dispatch_t), vp]
        L.moe_lm_head.restype = ctypes.c_int
        L.moe_lm_head.argtypes = [ctypes.POINTER(moe_lm_head_desc_t), i32, vp, vp, vp, vp, vp]
        L.moe_read_status.restype = ctypes.c_int
        L.moe_read_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_workspace_bytes(desc: moe_desc_t) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc)))


def moe_route(desc, M, x, w_router, topk_ids, topk_w, ws, disp: Optional[moe_dispatch_t] = None, stream=None):
    st = lib().moe_route(ctypes.byref(desc), M, _ptr(x), _ptr(w_router), _ptr(topk_ids), _ptr(topk_w),
                         ctypes.byref(disp) if disp is not None else None, _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream))
    _check(st, "moe_route")


def moe_decode_forward(desc, M, x, w_router, weights: moe_weights_t, y, ws, req_offsets=None, R: int = 0,
                       topk_ids=None, topk_w=None, disp: Optional[moe_dispatch_t] = None, stream=None):
    st = lib().moe_decode_forward(ctypes.byref(desc), M, _ptr(x), _ptr(w_router), ctypes.byref(weights),
                                  _ptr(req_offsets), R, _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                  ctypes.byref(disp) if disp is not None else None, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "moe_decode_forward")


def moe_decode_forward_noalloc(desc, M, x, w_router, weights: moe_weights_t, y, req_offsets=None, R: int = 0,
                               topk_ids=None, topk_w=None, disp: Optional[moe_dispatch_t] = None, stream=None):
    st = lib().moe_decode_forward_noalloc(ctypes.byref(desc), M, _ptr(x), _ptr(w_router), ctypes.byref(weights),
                                          _ptr(req_offsets), R, _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                          ctypes.byref(disp) if disp is not None else None, _stream(stream))
    _check(st, "moe_decode_forward_noalloc")


def moe_lm_head(desc: moe_lm_head_desc_t, M, x, w, logits, w_scale=None, stream=None):
    st = lib().moe_lm_head(ctypes.byref(desc), M, _ptr(x), _ptr(w), _ptr(w_scale), _ptr(logits), _stream(stream))
    _check(st, "moe_lm_head")


def moe_read_status(ws, stream=None) -> int:
    out = ctypes.c_int32(0)
    _check(lib().moe_read_status(_ptr(ws), _stream(stream), ctypes.byref(out)), "moe_read_status")
    return int(out.value)
