"""Plants plausible mistakes in a private copy of the oracle source, on the CPU, and checks that
the pins in test_oracle_pins.py catch every one of them.  The oracle under test/oracle is never
modified; each mutant is compiled into a temporary directory and swapped in with oracle.use()."""
import os
import shutil

import pytest

from oracle import oracle as O
from moe_speculative_decode_amd import synth
from tests import test_oracle_pins as P

MUTANTS = {
    "silu_sign": ("a[r] = g[r] / (1.0 + exp(-g[r])) * v[r];", "a[r] = g[r] / (1.0 + exp(g[r])) * v[r];"),
    "no_shared": ("            for (int h = 0; h < H; ++h) ym[h] += osh[h];\n", "\n"),
    "no_renorm": ("kept[j].v = p[key[j].id] / sum;", "kept[j].v = p[key[j].id];"),
    "tie_order": ("return (x->id > y->id) - (x->id < y->id);", "return (x->id < y->id) - (x->id > y->id);"),
    "nibble_swap": ("(c & 1) ? (byte >> 4) : (byte & 15)", "(c & 1) ? (byte & 15) : (byte >> 4)"),
    "scale_index": ("A->scales[r * (A->cols / 32) + c / 32]", "A->scales[r * (A->cols / 32) + c / 64]"),
    "gate_up_swapped": ("omat Wg = expert_mat(wf, W->gate, W->gate_s, e, I, H);",
                        "omat Wg = expert_mat(wf, W->up, W->up_s, e, I, H);"),
    "no_route_weight": ("ym[h] += wj * oj[h];", "ym[h] += oj[h];"),
    "wrong_expert": ("omat Wd = expert_mat(wf, W->down, W->down_s, e, H, I);",
                     "omat Wd = expert_mat(wf, W->down, W->down_s, ids[(int64_t)m * k], H, I);"),
    "bf16_shift": ("return dec_f32((uint32_t)b << 16);", "return dec_f32((uint32_t)b << 15);"),
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e - 2)"),
    "compact_slot": ("row_slot[row] = p % k;", "row_slot[row] = p / k;"),
    "gap_index": ("key[k - 1].v - key[k].v", "key[k - 2].v - key[k].v"),
    "softmax_sign": ("p[e] = exp(l[e] - lmax) / z;", "p[e] = exp(lmax - l[e]) / z;"),
    # router prologue
    "bias_ignored": ("key[e].v = biased ? l[e] + (double)bias[e] : l[e];", "key[e].v = l[e];"),
    "bias_in_weights": ("kept[j].v = p[key[j].id] / sum;", "kept[j].v = key[j].v / sum;"),
    "bias_sign": ("l[e] + (double)bias[e]", "l[e] - (double)bias[e]"),
    "order_by_key": ("qsort(kept, k, sizeof(keyed), cmp_desc);", ";"),
    "norm_no_gain": ("xn[h] = oracle_round_bf16(g[h] * (x[h] * r));", "xn[h] = oracle_round_bf16(x[h] * r);"),
    "norm_no_round": ("xn[h] = oracle_round_bf16(g[h] * (x[h] * r));", "xn[h] = g[h] * (x[h] * r);"),
    "norm_no_eps": ("sqrt(ss / H + eps)", "sqrt(ss / H)"),
    "norm_mean": ("sqrt(ss / H + eps)", "sqrt(ss / (H - 1) + eps)"),
    "norm_skipped": ("    if (d->router_flags & ORACLE_NORM) {", "    if (0) {"),
    "round_ties_up": ("(r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0))", "(r >= 0.5)"),
    # FP8 block-quantised weights
    "e4m3_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_subnormal": ("ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    "fp8_scale_col": ("4 * ((r / FP8_BLOCK) * (A->cols / FP8_BLOCK) + c / FP8_BLOCK)",
                      "4 * ((r / FP8_BLOCK) * (A->cols / FP8_BLOCK) + c / 64)"),
    "fp8_scale_row": ("4 * ((r / FP8_BLOCK) * (A->cols / FP8_BLOCK) + c / FP8_BLOCK)",
                      "4 * ((r / 64) * (A->cols / FP8_BLOCK) + c / FP8_BLOCK)"),
    "fp8_scale_transposed": ("4 * ((r / FP8_BLOCK) * (A->cols / FP8_BLOCK) + c / FP8_BLOCK)",
                             "4 * ((c / FP8_BLOCK) * (A->rows / FP8_BLOCK) + r / FP8_BLOCK)"),
    "fp8_expert_scales": ("A.scales = scales + 4 * e * (rows / FP8_BLOCK) * (cols / FP8_BLOCK);",
                          "A.scales = scales;"),
    # LM head
    "lm_head_row_scale": ("const double sc = (double)scales[v];", "const double sc = (double)scales[0];"),
    "lm_head_transposed": ("const uint8_t* codes = (const uint8_t*)w + (int64_t)v * H;",
                           "const uint8_t* codes = (const uint8_t*)w + (int64_t)v;"),
    "lm_head_token": ("const double* xrow = xs + (int64_t)m * H;", "const double* xrow = xs;"),
}

# pins that run quickly; together they must catch each mutant
PINS = [
    P.test_e2m1_table,
    P.test_mxfp4_nibble_and_scale_layout,
    lambda: P.test_bf16_decoder_all_patterns(),
    lambda: P.test_routing_vs_full_sort(synth.BF16),
    P.test_tie_break_lower_id_first,
    lambda: P.test_dense_brute_force(synth.BF16, 64, 16, 4, 32, 32, (2, 3)),
    lambda: P.test_dense_brute_force(synth.MXFP4, 64, 16, 4, 32, 64, (3, 3)),
    lambda: P.test_closed_form_swiglu(synth.BF16, 2.0, 0.5),
    lambda: P.test_compaction_vs_sets(6, 8, 512),
    P.test_round_bf16_nearest_with_ties_to_even,
    P.test_rmsnorm_of_constant_vector_is_the_gain,
    P.test_rmsnorm_eps_closed_form,
    P.test_rmsnorm_vs_brute_force,
    P.test_biased_selection_vs_full_sort,
    P.test_biased_selection_constructed,
    lambda: P.test_dense_brute_force_with_router_prologue(synth.BF16, (2, 3)),
    P.test_e4m3_all_codes,
    P.test_fp8_block_scale_layout,
    lambda: P.test_dense_brute_force(synth.FP8, 256, 8, 2, 128, 128, (3,)),
    lambda: P.test_lm_head_vs_numpy(synth.FP8),
    lambda: P.test_lm_head_identity_rows(synth.FP8),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(O.SRC).read()
    assert src.count(old) == 1, "mutation site vanished: " + name
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = O.build(force=True, src=str(path), out=str(tmp_path / "libmutant.so"))
    caught = []
    with O.use(lib):
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, "mutant %s passed every pin" % name
    shutil.rmtree(tmp_path, ignore_errors=True)
