"""Dense brute force of the MoE layer in numpy, written independently of the oracle.

It decodes the storage formats itself (numpy bit views and the E2M1 value table of the OCP
Microscaling v1.0 specification), routes with a full sort of the float64 logits, and runs EVERY
expert on every token, masking the unselected ones with weight zero.  It is only feasible on tiny
shapes and exists to pin the oracle from outside.
"""
import numpy as np

# OCP MX v1.0, FP4 (E2M1) value table, codes 0..15
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _e4m3_table():
    """The 256 E4M3 values, from torch's float8_e4m3fn type (a library independent of the oracle)."""
    import torch
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def dec(fmt, data, scales=None):
    """storage -> float64 (same shape as the logical matrix)."""
    if fmt == 0:
        return np.asarray(data, dtype=np.float32).astype(np.float64)
    if fmt == 1:
        return (np.asarray(data, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if fmt == 3:  # E4M3 codes times one binary32 scale per 128 x 128 block (last two axes)
        vals = _e4m3_table()[np.asarray(data, dtype=np.uint8)]
        sc = np.asarray(scales, dtype=np.float32).astype(np.float64)
        return vals * np.repeat(np.repeat(sc, 128, axis=-2), 128, axis=-1)
    codes = np.asarray(data, dtype=np.uint8)
    lo = codes & 15
    hi = codes >> 4
    el = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    vals = E2M1_TABLE[el]
    sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


def _bf16_table():
    """Every finite bfloat16 value (one per value: -0 dropped) in ascending order, with its bits."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).view(np.float32).astype(np.float64)
    keep = np.isfinite(vals) & ~((vals == 0) & np.signbit(vals))
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], bits[keep][order].astype(np.uint16)


_BF16_VALS, _BF16_BITS = _bf16_table()


def round_bf16(v):
    """Nearest bfloat16 value of each float64 (ties: the candidate with an even bit pattern), by
    comparing the distances to the two bracketing finite bfloat16 values.  Finite inputs inside the
    finite range only."""
    v = np.asarray(v, dtype=np.float64)
    hi = np.clip(np.searchsorted(_BF16_VALS, v, side="left"), 1, len(_BF16_VALS) - 1)
    lo = hi - 1
    a, b = _BF16_VALS[lo], _BF16_VALS[hi]
    da, db = np.abs(v - a), np.abs(b - v)
    even_lo = (_BF16_BITS[lo] & 1) == 0
    pick_lo = (da < db) | ((da == db) & even_lo)
    out = np.where(pick_lo, a, b)
    return np.where(v == _BF16_VALS[hi], _BF16_VALS[hi], out)


def rms_norm(x, g, eps):
    """RMSNorm rows of x with gain g, rounded once to bfloat16."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return round_bf16(g[None, :] * (x * r))


def route(logits, k, bias=None):
    """ids [M,k]: the k largest keys (logit, or logit + bias) by (key desc, id asc); weights =
    softmax of the logits restricted to the selected experts; reported by (weight desc, id asc)."""
    M, E = logits.shape
    keys = logits if bias is None else logits + np.asarray(bias, dtype=np.float64)[None, :]
    ids = np.zeros((M, k), np.int64)
    w = np.zeros((M, k))
    for m in range(M):
        sel = np.lexsort((np.arange(E), -keys[m]))[:k]
        z = np.exp(logits[m, sel] - logits[m, sel].max())
        ww = z / z.sum()
        o = np.lexsort((sel, -ww))
        ids[m] = sel[o]
        w[m] = ww[o]
    return ids, w


def silu(z):
    return z / (1.0 + np.exp(-z))


def forward(cfg_tuple, x, wr, W, norm_w=None, bias=None, eps=1e-6):
    """cfg_tuple = (H, E, k, I, Is, act_fmt, weight_fmt); W = oracle-style storage dict; norm_w
    (activation format) turns on the RMSNorm prologue, bias the biased selection.
    Returns (y [M,H], ids, w)."""
    H, E, k, I, Is, af, wf = cfg_tuple
    xd = dec(af, x)
    if norm_w is not None:
        xd = rms_norm(xd, dec(af, norm_w), eps)
    logits = xd @ dec(af, wr).T
    ids, w = route(logits, k, bias)
    M = xd.shape[0]
    y = np.zeros((M, H))
    gate = dec(wf, W["gate"], W.get("gate_s"))
    up = dec(wf, W["up"], W.get("up_s"))
    down = dec(wf, W["down"], W.get("down_s"))
    for e in range(E):
        mask = np.zeros(M)
        for m in range(M):
            hit = np.nonzero(ids[m] == e)[0]
            if hit.size:
                mask[m] = w[m, hit[0]]
        a = silu(xd @ gate[e].T) * (xd @ up[e].T)
        y += mask[:, None] * (a @ down[e].T)
    if Is > 0:
        sg = dec(wf, W["sh_gate"], W.get("sh_gate_s"))
        su = dec(wf, W["sh_up"], W.get("sh_up_s"))
        sd = dec(wf, W["sh_down"], W.get("sh_down_s"))
        y += (silu(xd @ sg.T) * (xd @ su.T)) @ sd.T
    return y, ids, w
