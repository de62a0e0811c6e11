"""moe_decode_forward_noalloc (no workspace argument; the library's per-device static scratch)
against moe_decode_forward with a caller workspace, through the C ABI: two calls in a row per
pair, the second with a smaller input, each bit-identical to the workspace entry point (the same
kernels) and within the oracle bar."""
import numpy as np
import pytest
import torch

import moe_speculative_decode_amd as mdl
from moe_speculative_decode_amd import device as dev
from moe_speculative_decode_amd import synth
from tests import _gpu_common as G

pytestmark = pytest.mark.gpu


def _noalloc(case, x=None):
    M, H, k = case.M, case.cfg.hidden, case.cfg.top_k
    y = torch.empty((M, H), dtype=dev.act_dtype(case.cfg), device="cuda")
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((M, k), -1.0, dtype=torch.float32, device="cuda")
    disp = dev.DispatchOut(M, k, case.cfg.num_experts)
    mdl.moe_decode_forward_noalloc(case.desc, M, case.x if x is None else x, case.dl.router, case.dl.weights(), y,
                                   topk_ids=ids, topk_w=w, disp=disp.struct())
    return y, ids, w, disp


def _pair(first, second):
    for case in (first, second):
        y_ws, ids_ws, w_ws = case.run()
        y, ids, w, disp = _noalloc(case)
        torch.cuda.synchronize()
        err, _ = G.y_error(y, case.y_ref)
        G.log("noalloc", case.cfg.name, "M=%d err/rms=%.3e" % (case.M, err))
        assert torch.equal(y, y_ws) and torch.equal(ids, ids_ws) and torch.equal(w, w_ws)
        G.check_routing(ids, w, case.ids_ref, case.w_ref)
        G.check_dispatch(disp, case.comp_ref, ids, case.ids_ref, case.w_ref, case.M, case.cfg.top_k,
                         has_shared=case.cfg.shared_inter > 0)
        assert err <= G.TOL[case.cfg.weight_fmt], err


def _small(name, fmt, lens):
    act = synth.F32 if fmt == synth.F32 else synth.BF16
    inter = 256 if fmt == synth.FP8 else 192  # FP8: whole 128 x 128 scale blocks
    return synth.LayerConfig(name, 512, 64, 4, inter, 128, act, fmt, tuple(lens), "shared_base", 7)


@pytest.mark.parametrize("fmt", [synth.BF16, synth.MXFP4, synth.FP8], ids=["bf16", "mxfp4", "fp8"])
def test_noalloc_small_two_calls(fmt):
    big = G.Case(_small("na16", fmt, (3, 1, 7, 5)))
    small = G.Case(_small("na3", fmt, (3,)), layer_cfg=big.cfg)
    _pair(big, small)


def test_noalloc_ling_bf16_two_calls():
    cfg6 = synth.CONFIGS["ling_bf16_m6"]
    cfg1 = synth.CONFIGS["ling_bf16_m1"]
    a = G.Case(cfg6, hidden_seed=G.seeds()["ling_bf16_m6"]["hidden_seed"])
    b = G.Case(cfg1, hidden_seed=G.seeds()["ling_bf16_m1"]["hidden_seed"])
    _pair(a, b)


def test_noalloc_ling_fp8_two_calls():
    """Sixteen ragged FP8 tokens (unit-major, the largest pair-row count the scratch holds), then one."""
    cfg16 = synth.CONFIGS["ling_fp8_m16_ragged"]
    cfg1 = synth.CONFIGS["ling_fp8_m1"]
    a = G.Case(cfg16, hidden_seed=G.seeds()["ling_fp8_m16_ragged"]["hidden_seed"])
    b = G.Case(cfg1, hidden_seed=G.seeds()["ling_fp8_m1"]["hidden_seed"])
    _pair(a, b)


def test_noalloc_graph_replay():
    """Captured calls replay correctly from the same scratch, with eager calls in between."""
    case = G.Case(_small("na_graph", synth.BF16, (6,)))
    y_e, _, _, _ = _noalloc(case)
    torch.cuda.synchronize()
    M, H = case.M, case.cfg.hidden
    y = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mdl.moe_decode_forward_noalloc(case.desc, M, case.x, case.dl.router, case.dl.weights(), y, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), rep
        y2, _, _, _ = _noalloc(case)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_e)
