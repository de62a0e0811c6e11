"""GPU parity of the LM head (moe_lm_head) against the fp64 oracle, through the C ABI.

Bar: max |logit_gpu - logit_oracle| <= 1e-4 * rms(logits_oracle).  Derivation: every product of
a bf16 activation and a bf16 weight (or an E4M3 code, 4 significant bits) is exact in fp32.  One
token (the vector form): a lane sums its 40 products in four chains of 10, the chains are added
pairwise and the lanes of a row by a 6-level tree, so the rounding error is at most about
20 * 2^-24 * sum_h |x_h w_h| (one more rounding for the FP8 row scale).  Verify windows on the
matrix cores: one fixed chain of H / 32 products of 32 elements per logit in fp32; at most
log2(32) + 1 = 6 roundings per product, each at most 2^-24 times a partial sum of the logit
(|partial| <= 5 rms for these inputs), so about 480 roundings at H = 2,560.  With w ~ N(0, 0.02^2),
x ~ N(0, 1) and H = 2,560, sum_h |x_h w_h| is about 33 and rms(logits) about 1: the one-token bound
is near 4e-5 * rms; the matrix-core roundings are independent and of either sign, so they add like
a random walk, sqrt(480) * 2^-24 * 5 rms ~ 7e-6 rms, with a worst case of 1.4e-4 only if every
rounding took one sign at the largest partial.  1e-4 * rms holds both with a wide margin.  Results
are also bit-identical run to run."""
import numpy as np
import pytest
import torch

import moe_speculative_decode_amd as mdl
from moe_speculative_decode_amd import device as dev
from moe_speculative_decode_amd import synth
from oracle import oracle as O
from tests import _gpu_common as G

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _run(cfg, w, sc, x):
    desc = mdl.moe_lm_head_desc_t(cfg.hidden, cfg.vocab, cfg.weight_fmt)
    out = torch.full((cfg.M, cfg.vocab), float("nan"), dtype=torch.float32, device="cuda")
    mdl.moe_lm_head(desc, cfg.M, x, w, out, w_scale=sc)
    return out


def _check(cfg, seed=1):
    w, sc = synth.lm_head_weights(cfg)
    x = synth.lm_head_hidden(cfg, seed)
    ref = O.lm_head(cfg.weight_fmt, x, w, sc)
    wd, xd = dev.to_device(w), dev.to_device(x)
    scd = None if sc is None else dev.to_device(sc)
    a = _run(cfg, wd, scd, xd)
    b = _run(cfg, wd, scd, xd)
    torch.cuda.synchronize()
    got = a.cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    err = float(np.max(np.abs(got - ref)) / rms)
    G.log("lm_head", cfg.name, "M=%d V=%d H=%d err/rms=%.3e" % (cfg.M, cfg.vocab, cfg.hidden, err))
    assert np.all(np.isfinite(got))
    assert err <= TOL, err
    assert torch.equal(a, b)


SMALL = [
    synth.LMHeadConfig("bf16_v1000_m1", 512, 1000, synth.BF16, 1),
    synth.LMHeadConfig("bf16_v1000_m3", 512, 1000, synth.BF16, 3),
    synth.LMHeadConfig("bf16_tail_m16", 520, 4099, synth.BF16, 16),
    synth.LMHeadConfig("bf16_h2560_m5", 2560, 5000, synth.BF16, 5),
    synth.LMHeadConfig("fp8_v1000_m1", 512, 1000, synth.FP8, 1),
    synth.LMHeadConfig("fp8_tail_m7", 528, 3001, synth.FP8, 7),
    synth.LMHeadConfig("fp8_h2560_m16", 2560, 4096, synth.FP8, 16),
    synth.LMHeadConfig("bf16_v7_m2", 64, 7, synth.BF16, 2),   # fewer rows than waves
    synth.LMHeadConfig("fp8_v3_m1", 128, 3, synth.FP8, 1),
    # matrix-core form (2..16 tokens, whole 256-byte stages): ragged row ranges, partial tiles,
    # waves without rows, one stage per row, columns past M
    synth.LMHeadConfig("bf16_mf_v5003_m2", 256, 5003, synth.BF16, 2),
    synth.LMHeadConfig("bf16_mf_v33_m4", 128, 33, synth.BF16, 4),
    synth.LMHeadConfig("bf16_mf_h2560_m16", 2560, 20011, synth.BF16, 16),
    synth.LMHeadConfig("fp8_mf_v4099_m9", 512, 4099, synth.FP8, 9),
    synth.LMHeadConfig("fp8_mf_v17_m2", 256, 17, synth.FP8, 2),
    synth.LMHeadConfig("fp8_mf_h2560_m6", 2560, 30001, synth.FP8, 6),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_lm_head_small(cfg):
    _check(cfg)


@pytest.mark.parametrize("name", ["lm_head_bf16_m1", "lm_head_fp8_m1", "lm_head_bf16_m6", "lm_head_fp8_m6"])
def test_lm_head_full_size(name):
    G.log("lm_head", name, "generating")
    _check(synth.LM_HEADS[name])
