"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a temporary copy of ``oracle/lit_oracle.c``
(on the CPU; nothing here touches a GPU), compiles it, and runs the pins that should
notice it.  At least one of them has to fail; a mutant that passes every pin means the
pins are too weak.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_attention as TA
from tests import test_oracle_candidates as TC
from tests import test_oracle_formats as TF
from tests import test_oracle_indexer as TI
from tests import test_oracle_producer as TP
from tests import test_oracle_topk as TT
from tests import test_oracle_window as TW

SRC = os.path.join(os.path.dirname(oracle.__file__), "lit_oracle.c")


def _window_derived(orc):
    for case in TW.DERIVED:
        TW.test_derived_cases(orc, *case)


def _one_hot(orc):
    TI.test_one_hot_weights_reduce_to_library_matmul(orc, 64)
    TI.test_one_hot_weights_reduce_to_library_matmul(orc, 128)


def _one_hot_fp4(orc):
    TI.test_fp4_one_hot_weights_reduce_to_library_matmul(orc, 64)
    TI.test_fp4_one_hot_weights_reduce_to_library_matmul(orc, 128)


MUTANTS = [
    # (name, original text, mutated text, pins expected to notice)
    ("relu dropped", "s += wh * (dot > 0.0 ? dot : 0.0);", "s += wh * dot;",
     [TI.test_closed_form_constant_blocks, TI.test_relu_identity_gives_linear_form]),
    ("relu sign flipped", "s += wh * (dot > 0.0 ? dot : 0.0);", "s += wh * (dot < 0.0 ? -dot : 0.0);",
     [TI.test_closed_form_constant_blocks, TI.test_relu_identity_gives_linear_form]),
    ("key scale dropped", "double kv = orc_code_at(krow, fmt, d) * orc_e8m0(k_sc[ks]);",
     "double kv = orc_code_at(krow, fmt, d);", [TI.test_closed_form_constant_blocks, _one_hot]),
    ("key scale block reversed", "size_t ks = ((size_t)b * T_cap + t) * nb + d / 32;",
     "size_t ks = ((size_t)b * T_cap + t) * nb + (nb - 1 - d / 32);",
     [TI.test_closed_form_constant_blocks, _one_hot]),
    ("query scale block off", "size_t si = (qi * Hi + h) * nb + d / 32;",
     "size_t si = (qi * Hi + h) * nb;",
     [TI.test_closed_form_constant_blocks, _one_hot]),
    ("head weight index", "double wh = (double)w[((size_t)b * S + i) * Hi + h];",
     "double wh = (double)w[((size_t)b * S + i) * Hi + (Hi - 1 - h)];",
     [TI.test_closed_form_constant_blocks, TI.test_relu_identity_gives_linear_form]),
    ("visibility off by one", "return (start_pos + i + 1) / ratio;", "return (start_pos + i) / ratio;",
     [TI.test_visibility_prefill_decode_and_chunk]),
    ("e4m3 bias", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);",
     [TF.test_e4m3_all_codes_match_torch, TF.test_e4m3_closed_forms]),
    ("e4m3 subnormal exponent", "v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);",
     [TF.test_e4m3_all_codes_match_torch, TF.test_e4m3_closed_forms]),
    ("e2m1 bias", "v = ldexp(1.0 + (double)m / 2.0, e - 1);", "v = ldexp(1.0 + (double)m / 2.0, e - 2);",
     [TF.test_e2m1_all_codes_match_table, _one_hot_fp4]),
    ("e2m1 subnormal", "v = (double)m / 2.0;", "v = (double)m;", [TF.test_e2m1_all_codes_match_table]),
    ("fp4 row stride", "const size_t E = fmt == ORC_FMT_E2M1 ? (size_t)Di / 2 : (size_t)Di;",
     "const size_t E = (size_t)Di;", [_one_hot_fp4, TI.test_fp4_closed_form_constant_blocks]),
    ("fp4 nibble from the wrong byte", "uint8_t byte = row[d / 2];", "uint8_t byte = row[d / 4];",
     [_one_hot_fp4, TI.test_fp4_equals_e4m3_on_shared_values]),
    ("candidate pin off by one", "p[(nvis - 1) / block_size].s = INFINITY;", "p[nvis / block_size].s = INFINITY;",
     [TC.test_hand_ranked_blocks, TC.test_prefill_visibility_and_empty_query]),
    ("candidate -inf blocks not dropped", "if (p[j].s > -INFINITY) sel[take++] = p[j].t;", "sel[take++] = p[j].t;",
     [TC.test_prefill_visibility_and_empty_query]),
    ("candidate block min instead of max", "if (srow[t] > m) m = srow[t];", "if (srow[t] < m || m == -INFINITY) m = srow[t];",
     [TC.test_hand_ranked_blocks, TC.test_monotone_map_and_block_permutation]),
    ("candidate block overlaps the next", "for (int t = j * block_size; t < (j + 1) * block_size && t < T; ++t) {",
     "for (int t = j * block_size; t <= (j + 1) * block_size && t < T; ++t) {",
     [TC.test_hand_ranked_blocks, TC.test_monotone_map_and_block_permutation]),
    ("KV fp4 scale per 32", "v[d] = orc_e2m1(nib) * orc_e4m3(s[d / 16]);", "v[d] = orc_e2m1(nib) * orc_e4m3(s[d / 32]);",
     [lambda o: TA.test_quantised_kv_equals_library_decoded_rows(o, 64)]),
    ("KV fp4 nibbles swapped", "uint8_t nib = (d % 2 == 0) ? (c[d / 2] & 15) : (c[d / 2] >> 4);",
     "uint8_t nib = (d % 2 == 1) ? (c[d / 2] & 15) : (c[d / 2] >> 4);",
     [lambda o: TA.test_quantised_kv_equals_library_decoded_rows(o, 64)]),
    ("KV e4m3 scale dropped", "for (int d = 0; d < D; ++d) v[d] = orc_e4m3(c[d]) * orc_e8m0(s[d / 32]);",
     "for (int d = 0; d < D; ++d) v[d] = orc_e4m3(c[d]);",
     [lambda o: TA.test_quantised_kv_equals_library_decoded_rows(o, 64)]),
    ("rotation sign", "const float re = ac - bs, im = as + bc;",
     "const float re = ac + bs, im = as + bc;", [TP.test_rmsnorm_closed_form_and_rotation]),
    ("compressed rotation at the last token", "const int pos = start_pos + 1 - ratio; /* the group's first token */",
     "const int pos = start_pos;", [TP.test_compressor_group_timing_and_pooling]),
    ("fp4 quantiser tie rule", "int c = (a > 0.25 * s) + (a >= 0.75 * s)", "int c = (a > 0.25 * s) + (a > 0.75 * s)",
     [TP.test_quant_e2m1_brute_force]),
    ("rms over D-1", "double r = 1.0 / sqrt(ss / D + eps);", "double r = 1.0 / sqrt(ss / (D - 1) + eps);",
     [TP.test_rmsnorm_closed_form_and_rotation, TP.test_compressor_group_timing_and_pooling]),
    ("pooling reads slot 0 only", "acc += e * (double)ks[(size_t)r * D + d];", "acc += e * (double)ks[d];",
     [TP.test_compressor_group_timing_and_pooling]),
    ("e4m3 encoder truncates", "int q = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);", "int q = (int)floor((ldexp(a, -e) - 1.0) * 8.0);",
     [TP.test_e4m3_encoder_matches_torch, TP.test_quant_e4m3_brute_force]),
    ("topk tie rule reversed", "return (x->t > y->t) - (x->t < y->t);",
     "return (x->t < y->t) - (x->t > y->t);", [TT.test_property_checker_with_ties_and_prefill]),
    ("topk ascending sort dropped", "qsort(sel, (size_t)take, sizeof(int), orc_int_cmp);", "",
     [TT.test_matches_torch_topk_on_distinct_scores, TT.test_property_checker_with_ties_and_prefill]),
    ("topk ignores visibility", "if (nvis > T) nvis = T;", "nvis = T;",
     [TT.test_property_checker_with_ties_and_prefill, TT.test_k_at_least_visible_selects_everything]),
    ("window shifted", "p = P - W + 1 + j;", "p = P - W + j;", [_window_derived]),
    ("window slot not wrapped", "row[j] = valid ? (int32_t)(p % R) : -1;", "row[j] = valid ? (int32_t)p : -1;",
     [_window_derived, lambda o: TW.test_brute_force_sets(o, 128, 1, 1023, 128)]),
    ("softmax scale dropped", "l[j] = scale * dot;", "l[j] = dot;",
     [TA.test_all_rows_equals_library_sdpa, TA.test_dense_masked_softmax_two_sources]),
    ("logit over dv dims only", "for (int d = 0; d < D; ++d) dot += orc_bf16(qh[d]) * kv[(size_t)j * D + d];",
     "for (int d = 0; d < dv; ++d) dot += orc_bf16(qh[d]) * kv[(size_t)j * D + d];",
     [TA.test_dense_masked_softmax_two_sources]),
    ("sink left out of normaliser", "double Z = sink ? exp(sk - m) : 0.0;", "double Z = 0.0;",
     [TA.test_sink_closed_forms]),
    ("window rows dropped", "orc_kv_row(win_fmt, win_kv, win_sc, (size_t)b * R + s, D, kv + (size_t)nj++ * D);", "(void)s;",
     [TA.test_dense_masked_softmax_two_sources, TA.test_order_permutation_and_duplication_invariance]),
]


@pytest.mark.parametrize("name,orig,mut,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(orc, name, orig, mut, pins):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation anchor not found once: {orig!r}"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mut.c")
        lib = os.path.join(d, "libmut.so")
        with open(path, "w") as f:
            f.write(src.replace(orig, mut))
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-w",
                        "-o", lib, path, "-lm"], check=True)
        caught = []
        with oracle.using_library(lib):
            for pin in pins:
                try:
                    pin(oracle)
                except (AssertionError, oracle.OracleError):
                    caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"mutant '{name}' passed every pin"
