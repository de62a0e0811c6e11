"""Seeded synthetic inputs for the routed-expert MoE decode layer.

This module only draws random numbers and encodes them into storage formats (binary32, bfloat16,
MXFP4).  It holds none of the layer's arithmetic: no routing, no matrix products, no activation.
Both the HIP path and the CPU oracle consume exactly the bytes it produces, so the encoders'
own rounding never affects parity.

Recipe (one layer shared by every Ling-shaped workload, as in a real model):
  * every tensor is drawn from its own numpy PCG64 stream keyed by
    SeedSequence(layer_seed, spawn_key=(tag, index)); expert e of a stack uses index e, so any
    single expert can be regenerated without materialising the 6 GB stack;
  * weights: standard normal in float64, times 0.02, then encoded;
  * hidden states: tag HIDDEN_NOISE per token (plain N(0,1)), or, for speculative-verify windows,
    x_t = b_r + 0.5 * n_t with one base vector b_r per request (tag HIDDEN_BASE) so that tokens of
    one window pick overlapping experts;
  * float64 -> binary32 is IEEE round-to-nearest-even; binary32 -> bfloat16 is round-to-nearest-even
    on the bit pattern;
  * MXFP4 follows the OCP Microscaling v1.0 conversion: per block of 32 consecutive K elements the
    shared exponent is floor(log2(amax)) - 2 (2 = largest E2M1 exponent), each element is
    rounded to the nearest E2M1 value (ties to even mantissa) after division by the scale and
    saturates at +-6.

The shapes are those of Ling-3.0-flash ("3 ways to boost MoE inference on NVIDIA DGX Spark",
"Model and baseline configuration": hidden 2,560, eight of 512 routed experts plus one shared
expert; moe_intermediate_size 768 per "Chasing the Batch-1 Floor", "Where the time goes now").
"""
from __future__ import annotations

import dataclasses
import json
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

F32, BF16, MXFP4, FP8 = 0, 1, 2, 3
FORMAT_NAMES = {F32: "f32", BF16: "bf16", MXFP4: "mxfp4", FP8: "fp8"}
FP8_BLOCK = 128      # FP8 weights: one binary32 scale per block of 128 rows x 128 columns
FP8_MAX = 448.0      # largest finite E4M3 magnitude

# stream tags
T_ROUTER, T_GATE, T_UP, T_DOWN, T_SH_GATE, T_SH_UP, T_SH_DOWN, T_HIDDEN_BASE, T_HIDDEN_NOISE = range(9)
T_NORM, T_BIAS = 9, 10

NORM_GAIN_STD = 0.1   # RMSNorm gain g = 1 + 0.1 N(0,1), in the activation format
BIAS_STD = 0.5        # selection bias b ~ N(0, 0.5^2), binary32: half the spread of the logits

WEIGHT_STD = 0.02
MX_BLOCK = 32


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    hidden: int          # H
    num_experts: int     # E
    top_k: int           # k
    inter: int           # I (routed)
    shared_inter: int    # Is (0: no shared expert)
    act_fmt: int         # x, router, y
    weight_fmt: int      # routed + shared expert weights
    request_lens: tuple  # verify-window lengths of the packed batch; M = sum
    hidden_recipe: str   # "iid" or "shared_base"
    layer_seed: int = 0
    description: str = ""
    router_norm: bool = False   # RMSNorm prologue before the router (and the experts)
    router_bias: bool = False   # bias-corrected top-k selection
    norm_eps: float = 1e-6
    hidden_scale: float = 1.0   # hidden states drawn times this (a residual stream before its norm)

    @property
    def M(self) -> int:
        return int(sum(self.request_lens))

    @property
    def offsets(self) -> List[int]:
        out = [0]
        for n in self.request_lens:
            out.append(out[-1] + n)
        return out


def _ling(name, fmt, lens, recipe, desc, router=False):
    if router:  # the router chain's RMSNorm prologue and bias-corrected selection, on un-normed states
        return LayerConfig(name, 2560, 512, 8, 768, 768, BF16, fmt, tuple(lens), recipe, 0, desc,
                           router_norm=True, router_bias=True, norm_eps=1e-6, hidden_scale=4.0)
    return LayerConfig(name, 2560, 512, 8, 768, 768, BF16, fmt, tuple(lens), recipe, 0, desc)


CONFIGS: Dict[str, LayerConfig] = {
    "tiny_f32": LayerConfig("tiny_f32", 128, 8, 2, 64, 64, F32, F32, (1,), "iid", 0,
                            "tiny MoE layer, fp32, M=1, H=128, E=8, top-2, I=Is=64"),
    "ling_bf16_m1": _ling("ling_bf16_m1", BF16, (1,), "iid",
                          "Ling shapes, bf16, M=1 (batch-1 decode)"),
    "ling_bf16_m6": _ling("ling_bf16_m6", BF16, (6,), "shared_base",
                          "Ling shapes, bf16, M=6 (one NEXTN verify window of 6 draft tokens)"),
    "ling_bf16_m16_ragged": _ling("ling_bf16_m16_ragged", BF16, (2, 6, 3, 5), "shared_base",
                                  "Ling shapes, bf16, M=16 ragged verify, requests {2,6,3,5}"),
    "ling_mxfp4_m6": _ling("ling_mxfp4_m6", MXFP4, (6,), "shared_base",
                           "Ling shapes, MXFP4 expert weights, bf16 router/activations, M=6"),
    "ling_mxfp4_m1": _ling("ling_mxfp4_m1", MXFP4, (1,), "iid",
                           "Ling shapes, MXFP4 expert weights, bf16 router/activations, M=1"),
    "ling_mxfp4_m16_ragged": _ling("ling_mxfp4_m16_ragged", MXFP4, (2, 6, 3, 5), "shared_base",
                                   "Ling shapes, MXFP4 expert weights, M=16 ragged verify, requests {2,6,3,5}"),
    # FP8 (E4M3) expert weights with one binary32 scale per 128 x 128 block, bf16 router/activations
    "ling_fp8_m1": _ling("ling_fp8_m1", FP8, (1,), "iid", "Ling shapes, FP8 block-128 expert weights, M=1"),
    "ling_fp8_m6": _ling("ling_fp8_m6", FP8, (6,), "shared_base", "Ling shapes, FP8 block-128 expert weights, M=6"),
    "ling_fp8_m16_ragged": _ling("ling_fp8_m16_ragged", FP8, (2, 6, 3, 5), "shared_base",
                                 "Ling shapes, FP8 block-128 expert weights, M=16 ragged verify"),
    # the router chain with its RMSNorm prologue and bias-corrected top-k (hidden states x4)
    "ling_bf16_m1_router": _ling("ling_bf16_m1_router", BF16, (1,), "iid",
                                 "Ling shapes, bf16, M=1, RMSNorm prologue + bias-corrected top-k", True),
    "ling_bf16_m6_router": _ling("ling_bf16_m6_router", BF16, (6,), "shared_base",
                                 "Ling shapes, bf16, M=6, RMSNorm prologue + bias-corrected top-k", True),
    "ling_bf16_m16_ragged_router": _ling("ling_bf16_m16_ragged_router", BF16, (2, 6, 3, 5), "shared_base",
                                         "Ling shapes, bf16, M=16 ragged, RMSNorm prologue + bias-corrected top-k",
                                         True),
    "ling_mxfp4_m6_router": _ling("ling_mxfp4_m6_router", MXFP4, (6,), "shared_base",
                                  "Ling shapes, MXFP4, M=6, RMSNorm prologue + bias-corrected top-k", True),
}


# ----------------------------------------------------------------------------------------------
# random streams and encoders
# ----------------------------------------------------------------------------------------------

def normal(seed: int, tag: int, index: int, n: int) -> np.ndarray:
    """n float64 N(0,1) draws from the stream (seed, tag, index)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag, index))))
    return g.standard_normal(n)


def f32_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> binary32 (IEEE round-to-nearest-even)."""
    return np.ascontiguousarray(a, dtype=np.float64).astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> binary32 -> bfloat16 bits (uint16), round-to-nearest-even at each step."""
    u = f32_bits(a).view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


# E2M1 magnitudes of codes 0..7 (OCP MX v1.0): 0, 0.5, 1, 1.5, 2, 3, 4, 6
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_round(q: np.ndarray) -> np.ndarray:
    """|q| -> E2M1 magnitude code (0..7), nearest grid value, ties to the even code, saturating."""
    q = np.minimum(np.abs(q), 6.0)
    # midpoints between consecutive grid values; at an exact midpoint pick the even code
    mids = 0.5 * (_E2M1_GRID[1:] + _E2M1_GRID[:-1])
    code = np.searchsorted(mids, q, side="left").astype(np.uint8)  # q <= mid -> lower code
    at_mid = np.zeros(q.shape, dtype=bool)
    lower = code.astype(np.int64)
    valid = lower < 7
    at_mid[valid] = q[valid] == mids[lower[valid]]
    # at a midpoint searchsorted(side=left) gave the lower code; move to the even one
    odd_low = at_mid & ((code & 1) == 1)
    code[odd_low] += 1
    return code


def mxfp4_encode(w: np.ndarray):
    """float64 [N, K] -> (codes uint8 [N, K/2], scales uint8 [N, K/32]).

    Element 2i of a row goes to the low nibble of byte i, element 2i+1 to the high nibble.
    """
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % MX_BLOCK == 0
    blk = w.reshape(N, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blk).max(axis=2)
    # floor(log2(amax)) exactly: amax = f * 2^e with f in [0.5, 1) gives e - 1
    _, e = np.frexp(amax)
    xexp = np.where(amax > 0, e.astype(np.int64) - 1 - 2, -127)
    xexp = np.clip(xexp, -127, 127).astype(np.int64)
    scales = (xexp + 127).astype(np.uint8)
    q = blk / np.ldexp(1.0, xexp)[:, :, None]
    mag = _e2m1_round(q)
    sign = ((q < 0) & (mag > 0)).astype(np.uint8)
    code = (mag | (sign << 3)).reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(scales)


def _e4m3_round(q: np.ndarray) -> np.ndarray:
    """float64 -> E4M3 code bytes (OCP 8-bit floating point): nearest value, ties to the even
    mantissa, saturating at +-448.  Spacing 2^(e-3) in the binade [2^e, 2^(e+1)), e >= -6; below
    2^-6 the subnormal spacing 2^-9."""
    sign = (q < 0) | ((q == 0) & np.signbit(q))
    a = np.minimum(np.abs(q), FP8_MAX)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1): binade 2^(ex-1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    ulp = np.ldexp(1.0, e - 3)
    n = np.rint(a / ulp)                      # numpy rint: ties to even
    v = np.minimum(n * ulp, FP8_MAX)          # a carry into the next binade stays representable
    _, ex2 = np.frexp(v)
    e2 = np.maximum(ex2.astype(np.int64) - 1, -6)
    normal = v >= 2.0 ** -6
    field = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, np.rint(v / np.ldexp(1.0, e2 - 3)) - 8, np.rint(v / 2.0 ** -9))
    code = (field << 3) | mant.astype(np.int64)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def fp8_block_encode(w: np.ndarray):
    """float64 [N, K] -> (E4M3 codes uint8 [N, K], binary32 scales [N/128, K/128]).  Per block of
    128 x 128 the scale is amax / 448 (rounded to binary32; 1 for an all-zero block) and each
    element is encoded as w / scale."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert N % FP8_BLOCK == 0 and K % FP8_BLOCK == 0
    blk = w.reshape(N // FP8_BLOCK, FP8_BLOCK, K // FP8_BLOCK, FP8_BLOCK)
    amax = np.abs(blk).max(axis=(1, 3))
    scales = np.where(amax > 0, amax / FP8_MAX, 1.0).astype(np.float32)
    q = blk / scales.astype(np.float64)[:, None, :, None]
    codes = _e4m3_round(q).reshape(N, K)
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


def encode_weight(w: np.ndarray, fmt: int):
    """float64 [N, K] -> storage of format fmt: (data, scales or None)."""
    if fmt == F32:
        return f32_bits(w), None
    if fmt == BF16:
        return bf16_bits(w), None
    if fmt == FP8:
        return fp8_block_encode(w)
    return mxfp4_encode(w)


def encode_act(a: np.ndarray, fmt: int) -> np.ndarray:
    return f32_bits(a) if fmt == F32 else bf16_bits(a)


# ----------------------------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------------------------

class Layer:
    """Host copies of one MoE layer's weights in storage format.

    Stacks are expert-major: gate/up [E][I][H], down [E][H][I]; MXFP4 stacks have codes with K/2
    bytes per row and scales [..][K/32].  Experts are generated on demand (see materialise)."""

    def __init__(self, cfg: LayerConfig, experts: Optional[Sequence[int]] = None, threads: int = 0):
        self.cfg = cfg
        H, E, I, Is = cfg.hidden, cfg.num_experts, cfg.inter, cfg.shared_inter
        s, wf = cfg.layer_seed, cfg.weight_fmt
        self.router = encode_act(normal(s, T_ROUTER, 0, E * H).reshape(E, H) * WEIGHT_STD, cfg.act_fmt)
        self.norm_w = None    # [H] activation format
        self.router_bias = None  # [E] float32
        if cfg.router_norm:
            self.norm_w = encode_act(1.0 + NORM_GAIN_STD * normal(s, T_NORM, 0, H), cfg.act_fmt)
        if cfg.router_bias:
            self.router_bias = f32_bits(BIAS_STD * normal(s, T_BIAS, 0, E))
        self.shared = None
        if Is > 0:
            self.shared = {
                "gate": encode_weight(normal(s, T_SH_GATE, 0, Is * H).reshape(Is, H) * WEIGHT_STD, wf),
                "up": encode_weight(normal(s, T_SH_UP, 0, Is * H).reshape(Is, H) * WEIGHT_STD, wf),
                "down": encode_weight(normal(s, T_SH_DOWN, 0, H * Is).reshape(H, Is) * WEIGHT_STD, wf),
            }
        self.stacks = {}
        for name, rows, cols in (("gate", I, H), ("up", I, H), ("down", H, I)):
            if wf == MXFP4:
                self.stacks[name] = (np.zeros((E, rows, cols // 2), np.uint8),
                                     np.zeros((E, rows, cols // MX_BLOCK), np.uint8))
            elif wf == FP8:
                self.stacks[name] = (np.zeros((E, rows, cols), np.uint8),
                                     np.zeros((E, rows // FP8_BLOCK, cols // FP8_BLOCK), np.float32))
            else:
                dt = np.float32 if wf == F32 else np.uint16
                self.stacks[name] = (np.zeros((E, rows, cols), dt), None)
        self.present = np.zeros(E, dtype=bool)
        self.materialise(range(E) if experts is None else experts, threads)

    def _gen_expert(self, e: int):
        cfg = self.cfg
        H, I, s, wf = cfg.hidden, cfg.inter, cfg.layer_seed, cfg.weight_fmt
        for name, tag, rows, cols in (("gate", T_GATE, I, H), ("up", T_UP, I, H), ("down", T_DOWN, H, I)):
            data, sc = encode_weight(normal(s, tag, e, rows * cols).reshape(rows, cols) * WEIGHT_STD, wf)
            self.stacks[name][0][e] = data
            if sc is not None:
                self.stacks[name][1][e] = sc

    def materialise(self, experts, threads: int = 0):
        todo = [int(e) for e in experts if not self.present[int(e)]]
        if not todo:
            return
        threads = threads or min(16, len(os.sched_getaffinity(0)))
        if threads > 1 and len(todo) > 1:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(self._gen_expert, todo))
        else:
            for e in todo:
                self._gen_expert(e)
        self.present[todo] = True


def make_hidden(cfg: LayerConfig, hidden_seed: int) -> np.ndarray:
    """Hidden states [M][H] in the activation storage format."""
    H = cfg.hidden
    rows = []
    t = 0
    for r, n in enumerate(cfg.request_lens):
        base = normal(hidden_seed, T_HIDDEN_BASE, r, H) if cfg.hidden_recipe == "shared_base" else None
        for _ in range(n):
            noise = normal(hidden_seed, T_HIDDEN_NOISE, t, H)
            rows.append(noise if base is None else base + 0.5 * noise)
            t += 1
    return encode_act(np.stack(rows) * cfg.hidden_scale, cfg.act_fmt)


# ----------------------------------------------------------------------------------------------
# the LM head (vocabulary projection)
# ----------------------------------------------------------------------------------------------

T_LM_HEAD, T_LM_HIDDEN = 11, 12
LM_ROWS_PER_STREAM = 4096  # rows drawn per random stream, so the 157,184 rows generate in parallel


@dataclasses.dataclass(frozen=True)
class LMHeadConfig:
    name: str
    hidden: int       # H
    vocab: int        # V
    weight_fmt: int   # BF16, or FP8 (E4M3 codes + one binary32 scale per row)
    M: int            # tokens
    seed: int = 0
    description: str = ""


LM_HEADS: Dict[str, LMHeadConfig] = {
    # Ling-3.0-flash's vocabulary projection ("3 ways to boost MoE inference on NVIDIA DGX Spark",
    # "Model and baseline configuration" and "Optimization 2": 157,184 x 2,560)
    "lm_head_bf16_m1": LMHeadConfig("lm_head_bf16_m1", 2560, 157184, BF16, 1, 0, "LM head, bf16 weights, M=1"),
    "lm_head_fp8_m1": LMHeadConfig("lm_head_fp8_m1", 2560, 157184, FP8, 1, 0,
                                   "LM head, FP8 weights (per-row scale), M=1"),
    "lm_head_bf16_m6": LMHeadConfig("lm_head_bf16_m6", 2560, 157184, BF16, 6, 0, "LM head, bf16 weights, M=6"),
    "lm_head_fp8_m6": LMHeadConfig("lm_head_fp8_m6", 2560, 157184, FP8, 6, 0,
                                   "LM head, FP8 weights (per-row scale), M=6"),
}


def fp8_row_encode(w: np.ndarray):
    """float64 [V, H] -> (E4M3 codes uint8 [V, H], binary32 scales [V]): per row the scale is
    amax / 448 (1 for an all-zero row) and each element is encoded as w / scale."""
    w = np.asarray(w, dtype=np.float64)
    amax = np.abs(w).max(axis=1)
    scales = np.where(amax > 0, amax / FP8_MAX, 1.0).astype(np.float32)
    codes = _e4m3_round(w / scales.astype(np.float64)[:, None])
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


def lm_head_weights(cfg: LMHeadConfig, threads: int = 0):
    """The LM head's weight [V, H] (bf16 storage, or FP8 codes) and its per-row scales (FP8) or None.
    Rows are drawn N(0, 0.02^2) in streams of LM_ROWS_PER_STREAM rows."""
    V, H = cfg.vocab, cfg.hidden
    data = np.zeros((V, H), np.uint16 if cfg.weight_fmt == BF16 else np.uint8)
    scales = np.zeros(V, np.float32) if cfg.weight_fmt == FP8 else None

    def gen(i):
        r0 = i * LM_ROWS_PER_STREAM
        r1 = min(V, r0 + LM_ROWS_PER_STREAM)
        w = normal(cfg.seed, T_LM_HEAD, i, (r1 - r0) * H).reshape(r1 - r0, H) * WEIGHT_STD
        if cfg.weight_fmt == FP8:
            data[r0:r1], scales[r0:r1] = fp8_row_encode(w)
        else:
            data[r0:r1] = bf16_bits(w)

    n = (V + LM_ROWS_PER_STREAM - 1) // LM_ROWS_PER_STREAM
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(gen, range(n)))
    return data, scales


def lm_head_hidden(cfg: LMHeadConfig, seed: int = 0) -> np.ndarray:
    """Token rows [M, H] bf16, N(0, 1)."""
    return bf16_bits(normal(seed, T_LM_HIDDEN, 0, cfg.M * cfg.hidden).reshape(cfg.M, cfg.hidden))


_SEEDS_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "tests", "golden", "seeds.json")


def accepted_hidden_seed(name: str) -> int:
    """The first hidden-state seed (0, 1, ...) of a named workload whose every token has a
    top-k / top-(k+1) router-logit gap of at least 1e-3, as recorded by the oracle script that
    writes tests/golden/seeds.json."""
    with open(_SEEDS_FILE) as f:
        return int(json.load(f)[name]["hidden_seed"])
