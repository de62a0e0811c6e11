"""The C ABI library loads, exports every entry point the header declares, and rejects invalid
arguments on the host before anything is launched (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import moe_speculative_decode_amd as mdl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")
FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails validation first


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:size_t|int|const char\*)\s+(moe_\w+)\(", text, flags=re.M)


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(mdl.EXPORTED)
    L = mdl.lib()
    for n in names:
        assert hasattr(L, n), n
    # the exports are plain C symbols (no C++ mangling)
    nm = os.popen("nm -D --defined-only %s" % mdl.LIB_PATH).read()
    for n in names:
        assert re.search(r"\bT %s$" % n, nm, flags=re.M), n


def ling(**kw):
    d = dict(hidden=2560, num_experts=512, top_k=8, inter=768, shared_inter=768, max_tokens=16,
             act_format=mdl.MOE_FMT_BF16, weight_format=mdl.MOE_FMT_BF16)
    d.update(kw)
    return mdl.moe_desc_t(**d)


def test_workspace_bytes():
    n = mdl.moe_workspace_bytes(ling())
    # at least logits + SwiGLU rows + partial rows for 16 tokens
    assert n >= 4 * (16 * 512 + 16 * 9 * 768 + 16 * 9 * 2560)
    assert mdl.moe_workspace_bytes(ling(max_tokens=1)) < n
    for bad in (ling(top_k=0), ling(top_k=600), ling(num_experts=513), ling(hidden=2564), ling(max_tokens=17),
                ling(act_format=mdl.MOE_FMT_F32), ling(weight_format=7), ling(inter=0),
                ling(weight_format=mdl.MOE_FMT_MXFP4, hidden=2560 + 8), ling(hidden=8192),
                # beyond the kernel instances: no accepted shape reaches untested code
                ling(hidden=2560 + 32), ling(inter=768 + 32), ling(shared_inter=1024),
                ling(weight_format=mdl.MOE_FMT_MXFP4, hidden=3072),
                ling(act_format=mdl.MOE_FMT_F32, weight_format=mdl.MOE_FMT_F32, hidden=264, inter=64,
                     shared_inter=64),
                ling(act_format=mdl.MOE_FMT_F32, weight_format=mdl.MOE_FMT_F32, hidden=128, inter=264,
                     shared_inter=64)):
        assert mdl.moe_workspace_bytes(bad) == 0
    assert mdl.moe_workspace_bytes(ling(act_format=mdl.MOE_FMT_F32, weight_format=mdl.MOE_FMT_F32, hidden=256,
                                        inter=256, shared_inter=256)) > 0


def call_route(desc, M=1, x=FAKE, wr=FAKE, ids=FAKE, w=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return mdl.lib().moe_route(ctypes.byref(desc), M, x, wr, ids, w, None, ws, ws_bytes, None)


def call_fwd(desc, M=1, weights=None, y=FAKE, off=None, R=0, ws_bytes=1 << 30, x=FAKE):
    W = weights if weights is not None else mdl.moe_weights_t(*([FAKE] * 12))
    return mdl.lib().moe_decode_forward(ctypes.byref(desc), M, x, FAKE, ctypes.byref(W), off, R, y, None, None,
                                        None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,M,status", [
    (dict(), 0, mdl.MOE_ERR_SHAPE),
    (dict(), 17, mdl.MOE_ERR_SHAPE),
    (dict(max_tokens=4), 5, mdl.MOE_ERR_SHAPE),
    (dict(top_k=513), 1, mdl.MOE_ERR_SHAPE),
    (dict(act_format=mdl.MOE_FMT_F32), 1, mdl.MOE_ERR_FORMAT),
    (dict(weight_format=mdl.MOE_FMT_MXFP4, inter=776), 1, mdl.MOE_ERR_SHAPE),
])
def test_route_rejects(kw, M, status):
    assert call_route(ling(**kw), M=M) == status


def test_router_prologue_checks():
    assert call_route(ling(router_flags=4)) == mdl.MOE_ERR_FORMAT
    assert call_route(ling(router_flags=mdl.MOE_ROUTER_NORM, norm_eps=1e-6)) == mdl.MOE_ERR_NULL
    assert call_route(ling(router_flags=mdl.MOE_ROUTER_BIAS)) == mdl.MOE_ERR_NULL
    assert call_route(ling(router_flags=mdl.MOE_ROUTER_BIAS, router_bias=FAKE + 4)) == mdl.MOE_ERR_ALIGN
    assert call_route(ling(router_flags=mdl.MOE_ROUTER_NORM, norm_eps=-1.0, norm_weight=FAKE)) == mdl.MOE_ERR_SHAPE
    assert call_route(ling(act_format=mdl.MOE_FMT_F32, weight_format=mdl.MOE_FMT_F32, hidden=128, inter=64,
                           shared_inter=64, router_flags=mdl.MOE_ROUTER_NORM, norm_weight=FAKE)) == mdl.MOE_ERR_FORMAT


def test_route_null_align_workspace():
    d = ling()
    assert call_route(d, x=None) == mdl.MOE_ERR_NULL
    assert call_route(d, ids=None) == mdl.MOE_ERR_NULL
    assert call_route(d, x=FAKE + 4) == mdl.MOE_ERR_ALIGN
    assert call_route(d, ws_bytes=mdl.moe_workspace_bytes(d) - 1) == mdl.MOE_ERR_WORKSPACE
    assert mdl.lib().moe_route(None, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == mdl.MOE_ERR_NULL


def test_forward_rejects():
    d = ling()
    assert call_fwd(d, y=None) == mdl.MOE_ERR_NULL
    assert call_fwd(d, y=FAKE + 8) == mdl.MOE_ERR_ALIGN
    W = mdl.moe_weights_t(*([FAKE] * 12))
    W.down = None
    assert call_fwd(d, weights=W) == mdl.MOE_ERR_NULL
    W = mdl.moe_weights_t(*([FAKE] * 12))
    W.sh_up = None
    assert call_fwd(d, weights=W) == mdl.MOE_ERR_NULL
    assert call_fwd(ling(shared_inter=0), weights=W) != mdl.MOE_ERR_NULL  # no shared expert: not needed
    W = mdl.moe_weights_t(*([FAKE] * 12))
    W.gate_s = None
    assert call_fwd(ling(weight_format=mdl.MOE_FMT_MXFP4), weights=W) == mdl.MOE_ERR_NULL
    W = mdl.moe_weights_t(*([FAKE] * 12))
    W.up = FAKE + 2
    assert call_fwd(d, weights=W) == mdl.MOE_ERR_ALIGN
    assert call_fwd(d, off=FAKE, R=0) == mdl.MOE_ERR_OFFSETS
    assert call_fwd(d, off=FAKE, R=17) == mdl.MOE_ERR_OFFSETS
    assert call_fwd(d, ws_bytes=100) == mdl.MOE_ERR_WORKSPACE


def test_noalloc_rejects_on_host():
    """The fixed scratch serves max_tokens * (top_k + 1) <= 144 pair rows; larger descriptions are
    rejected before any HIP call (so this runs without a GPU), as are invalid descriptions."""
    W = mdl.moe_weights_t(*([FAKE] * 12))
    L = mdl.lib()

    def call(desc):
        return L.moe_decode_forward_noalloc(ctypes.byref(desc), 1, FAKE, FAKE, ctypes.byref(W), None, 0, FAKE, None,
                                            None, None, None)
    assert call(ling(top_k=16, max_tokens=16)) == mdl.MOE_ERR_SCRATCH
    assert call(ling(top_k=8, max_tokens=16 + 1)) == mdl.MOE_ERR_SHAPE
    assert call(ling(top_k=9, max_tokens=15)) == mdl.MOE_ERR_SCRATCH  # 150 rows
    assert call(ling(hidden=4096)) == mdl.MOE_ERR_SHAPE
    assert L.moe_decode_forward_noalloc(None, 1, FAKE, FAKE, ctypes.byref(W), None, 0, FAKE, None, None, None,
                                        None) == mdl.MOE_ERR_NULL


def test_lm_head_rejects_on_host():
    L = mdl.lib()

    def call(H=2560, V=157184, fmt=mdl.MOE_FMT_BF16, M=1, x=FAKE, w=FAKE, sc=None, out=FAKE):
        d = mdl.moe_lm_head_desc_t(H, V, fmt)
        return L.moe_lm_head(ctypes.byref(d), M, x, w, sc, out, None)
    assert call(M=0) == mdl.MOE_ERR_SHAPE
    assert call(M=17) == mdl.MOE_ERR_SHAPE
    assert call(H=2568) == mdl.MOE_ERR_SHAPE
    assert call(H=520, fmt=mdl.MOE_FMT_FP8, sc=FAKE) == mdl.MOE_ERR_SHAPE  # FP8 rows of whole 16-code chunks
    assert call(V=0) == mdl.MOE_ERR_SHAPE
    assert call(fmt=mdl.MOE_FMT_MXFP4) == mdl.MOE_ERR_FORMAT
    assert call(fmt=mdl.MOE_FMT_FP8) == mdl.MOE_ERR_NULL  # no scales
    assert call(x=None) == mdl.MOE_ERR_NULL
    assert call(out=FAKE + 4) == mdl.MOE_ERR_ALIGN
    assert L.moe_lm_head(None, 1, FAKE, FAKE, None, FAKE, None) == mdl.MOE_ERR_NULL


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert mdl.moe_status_string(s) and mdl.moe_status_string(s) != "unknown status"
    assert mdl.moe_status_string(-99) == "unknown status"
    with pytest.raises(mdl.MoeError):
        mdl._check(mdl.MOE_ERR_SHAPE, "x")
