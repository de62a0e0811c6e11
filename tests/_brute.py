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


def dec(fmt, data, scales=None):
    """storage -> float64 (same shape as the logical matrix)."""
    if fmt == 0:
        return np.asarray(data, dtype=np.float32).astype(np.float64)
    if fmt == 1:
        return (np.asarray(data, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes = np.asarray(data, dtype=np.uint8)
    lo = codes & 15
    hi = codes >> 4
    el = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    vals = E2M1_TABLE[el]
    sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


def route(logits, k):
    """ids [M,k] by (logit desc, id asc); weights = softmax restricted to the selected logits."""
    M, E = logits.shape
    ids = np.zeros((M, k), np.int64)
    w = np.zeros((M, k))
    for m in range(M):
        order = np.lexsort((np.arange(E), -logits[m]))
        sel = order[:k]
        ids[m] = sel
        z = np.exp(logits[m, sel] - logits[m, sel].max())
        w[m] = z / z.sum()
    return ids, w


def silu(z):
    return z / (1.0 + np.exp(-z))


def forward(cfg_tuple, x, wr, W):
    """cfg_tuple = (H, E, k, I, Is, act_fmt, weight_fmt); W = oracle-style storage dict.
    Returns (y [M,H], ids, w)."""
    H, E, k, I, Is, af, wf = cfg_tuple
    xd = dec(af, x)
    logits = xd @ dec(af, wr).T
    ids, w = route(logits, k)
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
