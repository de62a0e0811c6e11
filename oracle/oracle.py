"""ctypes wrapper of the fp64 CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the checker of the HIP library, never part of its product path.  Only
the test suite, the package smoke check and the benchmark's CPU-baseline leg may import it.  It
imports nothing from the HIP package; inputs reach it as the storage bytes of the seeded generator.

Every function here marshals arguments; all arithmetic is in moe_oracle.c, which documents the
definition it follows step by step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

F32, BF16, MXFP4, FP8 = 0, 1, 2, 3


def build(force: bool = True, src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction, OpenMP over tokens)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


NORM, BIAS = 1, 2  # router flags: RMSNorm prologue, bias-corrected selection


class _Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("act_fmt", ctypes.c_int32), ("weight_fmt", ctypes.c_int32),
                ("router_flags", ctypes.c_int32), ("norm_eps", ctypes.c_double)]


class _Aux(ctypes.Structure):
    _fields_ = [("norm_w", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("gate", "up", "down", "gate_s", "up_s", "down_s",
                 "sh_gate", "sh_up", "sh_down", "sh_gate_s", "sh_up_s", "sh_down_s")]


def load(path: str):
    """Loads an oracle build (the default one, or a test build of the same source)."""
    L = ctypes.CDLL(path)
    L.oracle_bf16_to_f64.restype = ctypes.c_double
    L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_e2m1_to_f64.restype = ctypes.c_double
    L.oracle_e2m1_to_f64.argtypes = [ctypes.c_uint8]
    L.oracle_e8m0_to_f64.restype = ctypes.c_double
    L.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_to_f64.restype = ctypes.c_double
    L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    L.oracle_round_bf16.restype = ctypes.c_double
    L.oracle_round_bf16.argtypes = [ctypes.c_double]
    L.oracle_route.restype = None
    L.oracle_route.argtypes = [ctypes.POINTER(_Desc), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.POINTER(_Aux), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p]
    L.oracle_moe_forward.restype = None
    L.oracle_moe_forward.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Weights), ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Aux), ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    L.oracle_compact.restype = ctypes.c_int32
    L.oracle_compact.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    L.oracle_decode_matrix.restype = None
    L.oracle_decode_matrix.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p]
    L.oracle_max_threads.restype = ctypes.c_int32
    L.oracle_lm_head.restype = None
    L.oracle_lm_head.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
    return L


_lib = None
_override = None


def lib():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        _lib = load(LIB)
    return _lib


class use:
    """Context manager: route every call of this module to another build of the oracle."""

    def __init__(self, path: str):
        self.L = load(path)

    def __enter__(self):
        global _override
        self.prev, _override = _override, self.L
        return self

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def desc(H, E, k, I, Is, act_fmt, weight_fmt, router_flags=0, norm_eps=1e-6) -> _Desc:
    return _Desc(H, E, k, I, Is, act_fmt, weight_fmt, router_flags, norm_eps)


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(v)


def _aux(norm_w, bias):
    if norm_w is None and bias is None:
        return None
    return ctypes.byref(_Aux(_ptr(norm_w), _ptr(bias)))


def bf16_to_f64(b: int) -> float:
    return lib().oracle_bf16_to_f64(b)


def e2m1_to_f64(code: int) -> float:
    return lib().oracle_e2m1_to_f64(code)


def e8m0_to_f64(s: int) -> float:
    return lib().oracle_e8m0_to_f64(s)


def e4m3_to_f64(code: int) -> float:
    return lib().oracle_e4m3_to_f64(code)


def route(d: _Desc, x: np.ndarray, wr: np.ndarray, norm_w=None, bias=None
          ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """-> (logits [M,E] f64, ids [M,k] i32, w [M,k] f64, gap [M] f64).  norm_w ([H], activation
    format) and bias ([E] float32) are the router's prologue tensors, used when d's flags say so."""
    M = x.shape[0]
    logits = np.zeros((M, d.num_experts))
    ids = np.zeros((M, d.top_k), np.int32)
    w = np.zeros((M, d.top_k))
    gap = np.zeros(M)
    lib().oracle_route(ctypes.byref(d), M, _ptr(x), _ptr(wr), _aux(norm_w, bias), _ptr(logits), _ptr(ids), _ptr(w),
                       _ptr(gap))
    return logits, ids, w, gap


def forward(d: _Desc, weights: dict, x: np.ndarray, wr: np.ndarray, threads: int = 0, norm_w=None, bias=None):
    """Whole layer.  weights: dict with keys gate, up, down (+ _s scales for MXFP4) and sh_*.
    -> (y [M,H] f64, ids [M,k], w [M,k], gap [M])."""
    M = x.shape[0]
    W = _Weights(*[_ptr(weights.get(n)) for n in
                   ("gate", "up", "down", "gate_s", "up_s", "down_s",
                    "sh_gate", "sh_up", "sh_down", "sh_gate_s", "sh_up_s", "sh_down_s")])
    y = np.zeros((M, d.hidden))
    ids = np.zeros((M, d.top_k), np.int32)
    w = np.zeros((M, d.top_k))
    gap = np.zeros(M)
    lib().oracle_moe_forward(ctypes.byref(d), ctypes.byref(W), M, _ptr(x), _ptr(wr), _aux(norm_w, bias), _ptr(y),
                             _ptr(ids), _ptr(w), _ptr(gap), threads)
    return y, ids, w, gap


def compact(ids: np.ndarray, w: Optional[np.ndarray], E: int):
    """-> dict(U, unit_expert [U+1], unit_off [U+2], row_token, row_slot, row_w [M*k+M])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, k = ids.shape
    n = M * k + M
    ue = np.zeros(min(M * k, E) + 1, np.int32)
    uo = np.zeros(min(M * k, E) + 2, np.int32)
    rt = np.zeros(n, np.int32)
    rs = np.zeros(n, np.int32)
    rw = np.zeros(n)
    wv = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    U = lib().oracle_compact(M, k, E, _ptr(ids), _ptr(wv), _ptr(ue), _ptr(uo), _ptr(rt), _ptr(rs), _ptr(rw))
    return {"U": int(U), "unit_expert": ue[:U + 1].copy(), "unit_off": uo[:U + 2].copy(),
            "row_token": rt, "row_slot": rs, "row_w": rw}


def decode_matrix(fmt: int, data: np.ndarray, scales: Optional[np.ndarray], rows: int, cols: int) -> np.ndarray:
    out = np.zeros((rows, cols))
    lib().oracle_decode_matrix(fmt, _ptr(np.ascontiguousarray(data)),
                               _ptr(None if scales is None else np.ascontiguousarray(scales)), rows, cols, _ptr(out))
    return out


def lm_head(fmt: int, x: np.ndarray, w: np.ndarray, scales: Optional[np.ndarray] = None, threads: int = 0):
    """logits [M, V] fp64 of the LM head: x [M, H] bf16 storage, w [V, H] bf16 or FP8 codes with
    per-row float32 scales [V]."""
    M, H = x.shape
    V = w.shape[0]
    out = np.zeros((M, V))
    lib().oracle_lm_head(fmt, H, V, M, _ptr(np.ascontiguousarray(x)), _ptr(np.ascontiguousarray(w)),
                         _ptr(None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)),
                         _ptr(out), threads)
    return out


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def layer_weights(layer) -> dict:
    """Storage arrays of a synth.Layer in the oracle's weights dict."""
    W = {}
    for name in ("gate", "up", "down"):
        data, sc = layer.stacks[name]
        W[name] = data
        if sc is not None:
            W[name + "_s"] = sc
    if layer.shared is not None:
        for name in ("gate", "up", "down"):
            data, sc = layer.shared[name]
            W["sh_" + name] = data
            if sc is not None:
                W["sh_" + name + "_s"] = sc
    return W


def layer_desc(cfg) -> _Desc:
    flags = (NORM if getattr(cfg, "router_norm", False) else 0) | (BIAS if getattr(cfg, "router_bias", False) else 0)
    return desc(cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter, cfg.shared_inter, cfg.act_fmt,
                cfg.weight_fmt, flags, getattr(cfg, "norm_eps", 1e-6))


def router_aux(layer) -> dict:
    """The router prologue tensors of a synth.Layer as keyword arguments of route / forward."""
    return {"norm_w": getattr(layer, "norm_w", None), "bias": getattr(layer, "router_bias", None)}
