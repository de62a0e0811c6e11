"""GPU parity of the HIP layer against the fp64 oracle, through the C ABI.

Bars: per-token expert-id sets equal; routing weights within 1e-5; y within the format's
max-abs / rms(y_oracle) bar (bf16 2e-2, MXFP4 5e-2, fp32 1e-4); dispatch tables exact.
Shapes: the named Ling workloads at full size, plus small layers that still span several
row tiles of every kernel with ragged tails, and the degenerate cases of the method."""
import numpy as np
import pytest
import torch

import moe_speculative_decode_amd as mdl
from moe_speculative_decode_amd import device as dev
from moe_speculative_decode_amd import synth
from tests import _gpu_common as G

pytestmark = pytest.mark.gpu

BF16, MXFP4, F32, FP8 = synth.BF16, synth.MXFP4, synth.F32, synth.FP8


def small(name, fmt=BF16, H=512, E=64, k=4, I=192, Is=128, lens=(5,), recipe="shared_base", norm=False, bias=False):
    act = F32 if fmt == F32 else BF16
    return synth.LayerConfig(name, H, E, k, I, Is, act, fmt, tuple(lens), recipe, 7, router_norm=norm,
                             router_bias=bias, hidden_scale=4.0 if norm else 1.0)


SMALL = [
    small("bf16_m1", lens=(1,), recipe="iid"),
    small("bf16_m5", lens=(5,)),
    small("bf16_m16_ragged", lens=(3, 1, 7, 5)),
    small("bf16_tail", H=520, I=200, Is=72, lens=(6,)),
    # bf16 slice mode with 54 pair and token rows of 768 (84 KB of LDS), two requests; 63 rows
    # (seven tokens) would not fit and run unit-major
    small("bf16_slice_i768_m6", E=64, k=8, I=768, lens=(2, 4)),
    small("bf16_unit_major_i768_m7", E=64, k=8, I=768, lens=(7,)),
    small("mxfp4_m1", MXFP4, lens=(1,), recipe="iid"),
    small("mxfp4_m2", MXFP4, lens=(2,)),  # slice mode, line-form matrix-core gate/up (below three tokens)
    small("mxfp4_m6", MXFP4, lens=(6,)),
    small("mxfp4_m16", MXFP4, H=544, I=224, Is=96, lens=(9, 7)),
    # all pair rows do not fit in LDS as bf16 -> unit-major down rows for MXFP4 (vector path)
    small("mxfp4_m16_unit_major", MXFP4, H=512, E=256, k=8, I=768, Is=128, lens=(16,)),
    # MXFP4 slice mode with the shared expert's scale bytes in LDS (Is / 32 a multiple of 4) and two requests
    small("mxfp4_m6_scale_window", MXFP4, H=512, E=128, k=8, I=256, Is=128, lens=(2, 4)),
    small("f32_m3", F32, H=256, E=32, k=3, I=96, Is=64, lens=(3,)),
    small("bf16_no_shared", Is=0, lens=(4,)),
    small("bf16_k1", k=1, lens=(6,)),
    small("bf16_k_eq_E", E=8, k=8, lens=(3,)),
    small("bf16_k16", E=128, k=16, lens=(16,)),
    small("bf16_E512", E=512, k=8, lens=(8,)),
    # many experts per top-k wave (one wave per token, eight logits per lane), every workgroup
    # redoing the top-k below three tokens and the delegated top-k from three tokens on
    small("bf16_E512_m2", E=512, k=8, lens=(2,)),
    small("bf16_E384_m3", E=384, k=6, lens=(3,)),
    small("bf16_E512_k16_m1", E=512, k=16, lens=(1,), recipe="iid"),
    small("bf16_E200_m1", E=200, k=8, lens=(1,), recipe="iid"),
    # the router chain's RMSNorm prologue and bias-corrected selection, alone and together, below
    # and above the delegated top-k, with vector and matrix-core gate/up
    small("router_nb_m1", lens=(1,), recipe="iid", norm=True, bias=True),
    small("router_nb_m6", lens=(6,), norm=True, bias=True),
    small("router_nb_m16", E=128, k=8, lens=(4, 5, 7), norm=True, bias=True),
    small("router_norm_m3", lens=(3,), norm=True),
    small("router_bias_m2", E=512, k=8, lens=(2,), bias=True),
    small("router_bias_k16", E=128, k=16, lens=(5,), bias=True),
    small("router_nb_mxfp4_m6", MXFP4, lens=(6,), norm=True, bias=True),
    small("router_nb_tail", H=520, I=200, Is=72, lens=(7,), norm=True, bias=True),
    # FP8 (E4M3, one scale per 128 x 128 block): slice mode, unit-major, ragged chunk tails (H = 640:
    # 40 chunks a row), down rows of several 128-row blocks per unit, and the router prologue
    small("fp8_m1", FP8, I=256, lens=(1,), recipe="iid"),
    small("fp8_m6", FP8, I=256, lens=(6,)),
    small("fp8_m16", FP8, H=640, I=384, Is=256, lens=(9, 7)),
    small("fp8_k8_m16", FP8, E=256, k=8, I=768, Is=128, lens=(16,)),
    small("fp8_router_nb_m6", FP8, I=256, lens=(6,), norm=True, bias=True),
    # router rows span twice the chunks of FP8 gate/up rows (bf16 activations)
    small("fp8_h1024", FP8, H=1024, I=256, lens=(3,)),
    small("fp8_h2560", FP8, H=2560, E=64, k=4, I=256, Is=128, lens=(2,), norm=True),
    # matrix-core gate/up in slice mode (FP8 from three tokens, M * k <= 16)
    small("fp8_slice_mfma_m4", FP8, I=256, lens=(4,)),
    # the line-form matrix-core gate/up for MXFP4 (unit-major): scale rows not a multiple of 16
    # bytes (H = 544: 17 blocks, a last stage of one block) and the shared expert's tiles from 8 tokens
    small("mxfp4_um_tail", MXFP4, H=544, E=64, k=4, I=768, Is=96, lens=(16,)),
]


def _check_case(case, disp=None):
    y, ids, w = case.run(disp=disp)
    torch.cuda.synchronize()
    assert mdl.moe_read_status(case.ws) == mdl.MOE_OK
    err, rms = G.y_error(y, case.y_ref)
    G.log(case.cfg.name, "M=%d U=%d err/rms=%.3e rms=%.3e" % (case.M, case.comp_ref["U"], err, rms))
    G.check_routing(ids, w, case.ids_ref, case.w_ref)
    assert err <= G.TOL[case.cfg.weight_fmt], err
    if disp is not None:
        G.check_dispatch(disp, case.comp_ref, ids, case.ids_ref, case.w_ref, case.M, case.cfg.top_k,
                         has_shared=case.cfg.shared_inter > 0)
    return y


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_layers(cfg):
    G.log("small", cfg)
    case = G.Case(cfg)
    disp = dev.DispatchOut(case.M, cfg.top_k, cfg.num_experts)
    _check_case(case, disp)


def test_tiny_f32_config():
    cfg = synth.CONFIGS["tiny_f32"]
    case = G.Case(cfg, hidden_seed=G.seeds()["tiny_f32"]["hidden_seed"])
    disp = dev.DispatchOut(case.M, cfg.top_k, cfg.num_experts)
    _check_case(case, disp)


@pytest.mark.parametrize("name", ["ling_bf16_m1", "ling_bf16_m6", "ling_bf16_m16_ragged", "ling_mxfp4_m1",
                                  "ling_mxfp4_m6", "ling_mxfp4_m16_ragged", "ling_bf16_m1_router",
                                  "ling_bf16_m6_router", "ling_bf16_m16_ragged_router", "ling_mxfp4_m6_router",
                                  "ling_fp8_m1", "ling_fp8_m6", "ling_fp8_m16_ragged"])
def test_ling_configs(name):
    cfg = synth.CONFIGS[name]
    G.log("ling", name, "generating layer")
    case = G.Case(cfg, hidden_seed=G.seeds()[name]["hidden_seed"])
    disp = dev.DispatchOut(case.M, cfg.top_k, cfg.num_experts, R=len(cfg.request_lens))
    y, ids, w = case.run(disp=disp, req_offsets=cfg.offsets)
    torch.cuda.synchronize()
    err, rms = G.y_error(y, case.y_ref)
    G.log(name, "U=%d err/rms=%.3e" % (case.comp_ref["U"], err))
    assert case.comp_ref["U"] == G.seeds()[name]["U"]
    G.check_routing(ids, w, case.ids_ref, case.w_ref)
    G.check_dispatch(disp, case.comp_ref, ids, case.ids_ref, case.w_ref, case.M, cfg.top_k)
    assert err <= G.TOL[cfg.weight_fmt], err
    # distinct routed experts per packed request
    off = cfg.offsets
    want = [len(set(case.ids_ref[off[r]:off[r + 1]].ravel().tolist())) for r in range(len(off) - 1)]
    assert disp.req_unique.cpu().tolist() == want
    assert mdl.moe_read_status(case.ws) == mdl.MOE_OK


@pytest.mark.parametrize("fmt", [BF16, MXFP4, FP8], ids=["bf16", "mxfp4", "fp8"])
def test_deterministic_and_permutation_equivariant(fmt):
    """Unit-major down rows (and the matrix-core gate/up with its per-wave step ranges for MXFP4
    and FP8): bit-identical across runs and token orders.  99 pair and token rows of 768 do not
    fit the slice mode's 96 KB of bf16 SwiGLU rows, so bf16 and MXFP4 run unit-major too."""
    cfg = small("perm", fmt, k=8, I=768, lens=(11,))
    case = G.Case(cfg)
    y1, ids1, w1 = case.run()
    y2, ids2, w2 = case.run()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(ids1, ids2) and torch.equal(w1, w2)
    perm = torch.tensor(np.random.default_rng(3).permutation(case.M), device="cuda")
    yp, idsp, wp = case.run(x=case.x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(yp, y1[perm])
    for m in range(case.M):
        assert set(idsp[m].tolist()) == set(ids1[perm[m]].tolist())


@pytest.mark.parametrize("fmt", [BF16, MXFP4, FP8], ids=["bf16", "mxfp4", "fp8"])
def test_permutation_equivariant_slice_mode(fmt):
    """Few pair rows: every workgroup computes its own columns of every unit (bf16 and MXFP4 on the
    matrix cores, FP8 on the vector path after a matrix-core gate/up).  The result is
    bit-identical across token orders (fixed operand order per token column)."""
    cfg = small("perm_slice", fmt, k=4, I=256 if fmt == FP8 else 192, lens=(4,))
    case = G.Case(cfg)
    y1, ids1, _ = case.run()
    perm = torch.tensor([2, 0, 3, 1], device="cuda")
    yp, idsp, _ = case.run(x=case.x[perm].contiguous())
    torch.cuda.synchronize()
    err, _ = G.y_error(y1, case.y_ref)
    G.log("perm_slice", synth.FORMAT_NAMES[fmt], "err/rms=%.3e" % err)
    assert err <= G.TOL[fmt]
    assert torch.equal(yp, y1[perm])
    for m in range(case.M):
        assert set(idsp[m].tolist()) == set(ids1[perm[m]].tolist())


def test_router_prologue_deterministic_and_permutation_equivariant():
    cfg = small("perm_nb", lens=(11,), norm=True, bias=True)
    case = G.Case(cfg)
    y1, ids1, w1 = case.run()
    y2, ids2, w2 = case.run()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(ids1, ids2) and torch.equal(w1, w2)
    err, _ = G.y_error(y1, case.y_ref)
    G.log("perm_nb", "err/rms=%.3e" % err)
    assert err <= G.TOL[BF16]
    perm = torch.tensor(np.random.default_rng(4).permutation(case.M), device="cuda")
    yp, _, _ = case.run(x=case.x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(yp, y1[perm])


# (tokens, I): slice mode at one and six tokens; sixteen tokens of I = 768 do not fit the slice
# mode's LDS rows and run unit-major
MODES = [((1,), 192), ((6,), 192), ((16,), 768)]
MODE_IDS = ["m1_slice", "m6_slice", "m16_unit_major"]


@pytest.mark.parametrize("lens,inter", MODES, ids=MODE_IDS)
def test_repeated_calls_fewer_experts_than_cus(lens, inter):
    """E = 64 routed experts on 256 compute units: most workgroups own no router row.  Ten calls in
    a row on one workspace, alternating two token batches, each against the oracle."""
    cfg = small("rep", I=inter, lens=lens, recipe="iid" if lens == (1,) else "shared_base")
    a = G.Case(cfg)
    b = G.Case(cfg, x_host=G.accepted_hidden(cfg, a.layer, start=50)[0])
    b.ws = a.ws
    for i in range(10):
        c = a if i % 2 == 0 else b
        y, ids, w = c.run()
        torch.cuda.synchronize()
        G.check_routing(ids, w, c.ids_ref, c.w_ref)
        err, _ = G.y_error(y, c.y_ref)
        assert err <= G.TOL[BF16], (i, err)
    assert mdl.moe_read_status(a.ws) == mdl.MOE_OK


@pytest.mark.parametrize("lens,inter", MODES, ids=MODE_IDS)
def test_wait_timeout_writes_nan(lens, inter):
    """A wait that gives up leaves no output that looks valid.  Forced from the host: the workspace
    header's spin-limit word is set to 16 polls and the call counters of every eighth workgroup are
    advanced, so those workgroups take another call index than the rest and their tags and counter
    sets never meet.  Every wait is bounded, so every workgroup exits; y and the routing weights
    come out NaN and the status word reads MOE_ERR_TIMEOUT.  A fresh workspace then works."""
    cfg = small("timeout", I=inter, lens=lens, recipe="iid" if lens == (1,) else "shared_base")
    case = G.Case(cfg)
    cus = min(torch.cuda.get_device_properties(0).multi_processor_count, 1024)
    words = case.ws.view(torch.int32)
    words[1] = 16  # spin-limit test hook
    for b in range(0, cus, 8):  # workgroup b's call counter: word 64 + 4 b
        words[64 + 4 * b] = 3
    torch.cuda.synchronize()
    y, ids, w = case.run()
    torch.cuda.synchronize()
    G.log("timeout", lens, "nan y: %d of %d" % (int(torch.isnan(y.float()).sum()), y.numel()))
    assert mdl.moe_read_status(case.ws) == mdl.MOE_ERR_TIMEOUT
    assert torch.isnan(y.float()).all()
    assert torch.isnan(w).all()
    assert int(ids.min()) >= 0 and int(ids.max()) < cfg.num_experts
    case.ws = dev.workspace(case.desc)
    y, ids, w = case.run()
    torch.cuda.synchronize()
    assert mdl.moe_read_status(case.ws) == mdl.MOE_OK
    G.check_routing(ids, w, case.ids_ref, case.w_ref)
    assert G.y_error(y, case.y_ref)[0] <= G.TOL[BF16]


def test_identical_tokens_share_experts():
    cfg = small("same", lens=(1,), recipe="iid")
    base = G.Case(cfg)
    x = np.repeat(base.x_host, 7, axis=0)
    cfg7 = small("same7", lens=(7,))
    case = G.Case(cfg7, x_host=x, layer_cfg=cfg)
    disp = dev.DispatchOut(7, cfg.top_k, cfg.num_experts)
    y = _check_case(case, disp)
    assert int(disp.unit_count.item()) == cfg.top_k
    assert all(torch.equal(y[0], y[m]) for m in range(7))


def test_fewer_tokens_than_workspace():
    cfg = small("ws16", lens=(16,))
    case = G.Case(cfg)
    # reuse the 16-token workspace for a 3-token call
    sub = G.Case(small("ws3", lens=(3,)), x_host=case.x_host[:3], layer_cfg=cfg)
    sub.desc = case.desc
    sub.ws = case.ws
    _check_case(sub)
    _check_case(case)


def test_bad_offsets_set_status_and_keep_output():
    cfg = small("offs", lens=(2, 4))
    case = G.Case(cfg)
    y, ids, w = case.run(req_offsets=[0, 4, 3])
    torch.cuda.synchronize()
    assert mdl.moe_read_status(case.ws) == mdl.MOE_ERR_OFFSETS
    assert mdl.moe_read_status(case.ws) == mdl.MOE_OK  # cleared by the read
    assert G.y_error(y, case.y_ref)[0] <= G.TOL[BF16]


def test_hip_graph_replay_matches_eager():
    cfg = small("graph", lens=(6,))
    case = G.Case(cfg)
    y_e, ids_e, w_e = case.run()
    torch.cuda.synchronize()
    M, H, k = case.M, cfg.hidden, cfg.top_k
    y = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((M, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((M, k), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mdl.moe_decode_forward(case.desc, M, case.x, case.dl.router, case.dl.weights(), y, case.ws,
                                   topk_ids=ids, topk_w=w, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), rep
        assert torch.equal(ids, ids_e) and torch.equal(w, w_e)
        ye2, _, _ = case.run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(ye2, y_e)


@pytest.mark.parametrize("norm,bias", [(False, False), (True, True)], ids=["plain", "norm_bias"])
def test_route_only_matches_forward_routing(norm, bias):
    cfg = small("route", lens=(9,), norm=norm, bias=bias)
    case = G.Case(cfg)
    ids = torch.full((case.M, cfg.top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((case.M, cfg.top_k), dtype=torch.float32, device="cuda")
    disp = dev.DispatchOut(case.M, cfg.top_k, cfg.num_experts)
    mdl.moe_route(case.desc, case.M, case.x, case.dl.router, ids, w, case.ws, disp=disp.struct())
    torch.cuda.synchronize()
    G.check_routing(ids, w, case.ids_ref, case.w_ref)
    G.check_dispatch(disp, case.comp_ref, ids, case.ids_ref, case.w_ref, case.M, cfg.top_k)
    _, ids_f, w_f = case.run()
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_f) and torch.equal(w, w_f)
