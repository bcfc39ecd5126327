"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle source, plants one mistake (a dropped term, a
wrong sign, index or operand, a reversed tie-break ...), builds it on the
CPU and checks that at least one pin test fails against that build.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle
from tests import test_oracle_pins as pins

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "lsa_oracle.c")).read()

MUTATIONS = {
    "score_drops_last_dim": ("for (int32_t i = 0; i < b->d; i++)\n                acc = fmaf(qbar[i]",
                             "for (int32_t i = 0; i < b->d - 1; i++)\n                acc = fmaf(qbar[i]"),
    "fuse_weight_of_request0": ("acc = fmaf(w[(int64_t)r * b->H + h],", "acc = fmaf(w[h],"),
    "bias_sign": ("z[row] = fmaf(s, acc, bias[r]);", "z[row] = fmaf(s, acc, -bias[r]);"),
    "score_scale_dropped": ("z[row] = fmaf(s, acc, bias[r]);", "z[row] = acc + bias[r];"),
    "select_ge": ("if (z[row] > theta)", "if (z[row] >= theta)"),
    "refine_no_relu": ("rh[h] = (a > 0.0f) ? a : 0.0f;", "rh[h] = a;"),
    "refine_q_transposed": ("a = fmaf(qf[(int64_t)h * b->d + i]",
                            "a = fmaf(qf[((int64_t)i * b->H + h) % ((int64_t)b->H * b->d)]"),
    "refine_scale_dropped": ("if (b->idx_dt == O_FP8) I = I * sc;", ""),
    "topk_tie_high_first": ("return (a->tok > c->tok) - (a->tok < c->tok);",
                            "return (a->tok < c->tok) - (a->tok > c->tok);"),
    "topk_unsorted_emit": ("if (kk > 0) qsort(topk, (size_t)kk, sizeof(int32_t), o_int_cmp);", ""),
    "attn_v_offset": ("(double)o_elem(b->kv_dt, rows[i], b->v_off + e)",
                      "(double)o_elem(b->kv_dt, rows[i], e)"),
    "attn_wrong_last_recent": ("rows[kcnt + (s - rs)] = o_kv_row(b, chunk0, rec0, rs, s);",
                               "rows[kcnt + (s - rs)] = o_kv_row(b, chunk0, rec0, rs, "
                               "s == L - 1 ? rs : s);"),
    "attn_lse_no_max": ("lse[h] = m + log(l);", "lse[h] = log(l);"),
    "geometry_floor_off": ("int64_t rs = (int64_t)C * (h / C);",
                           "int64_t rs = (int64_t)C * ((h + C - 1) / C);"),
    "fp8_bias_8": ("ldexpf(1.0f + (float)m / 8.0f, e - 7)", "ldexpf(1.0f + (float)m / 8.0f, e - 8)"),
    "fp8_subnormal": ("ldexpf((float)m / 8.0f, -6)", "ldexpf((float)m / 8.0f, -7)"),
    "union_and_mode": ("any |= (z > theta);", "any = (l == 0) ? (z > theta) : (any & (z > theta));"),
    "union_last_layer_skipped": ("for (int32_t l = 0; l < n_layers; l++) {\n                float acc",
                                 "for (int32_t l = 0; l < n_layers - 1; l++) {\n                float acc"),
    "union_keys_of_layer0": ("o_elem(b->idx_dt, kic[l], row * b->d + i)", "o_elem(b->idx_dt, kic[0], row * b->d + i)"),
    "union_query_of_layer0": ("acc = fmaf(qbar[(int64_t)l * b->d + i],", "acc = fmaf(qbar[i],"),
    "sigmoid_sign": ("float t = -x * O_LOG2E;", "float t = x * O_LOG2E;"),
    "sigmoid_poly_short": ("for (int k = 6; k >= 0; k--) p = fmaf(p, f, O_EXP2C[k]);",
                           "for (int k = 6; k >= 1; k--) p = fmaf(p, f, O_EXP2C[k]);"),
    "sigscore_no_bias": ("const float x = fmaf(s, a, bias[r]);", "const float x = s * a;"),
    "sigscore_weight_of_request0": ("acc_s = fmaf(w[(int64_t)r * b->H + h],", "acc_s = fmaf(w[h],"),
    "sigscore_relu": ("acc_s = fmaf(w[(int64_t)r * b->H + h], lsao_sigmoid(x), acc_s);",
                      "acc_s = fmaf(w[(int64_t)r * b->H + h], x > 0.0f ? x : 0.0f, acc_s);"),
    "mass_chunk_index_shift": ("if (t < rs) pu[t / b->C] += p;", "if (t < rs) pu[(t + 1) / b->C] += p;"),
    "mass_recent_left_out": ("for (int64_t t = 0; t < L; t++) l += exp(x[t] - m);",
                             "for (int64_t t = 0; t < rs; t++) l += exp(x[t] - m);"),
    "mass_scale_dropped": ("x[t] = sm * acc;", "x[t] = acc;"),
    "mass_first_step_only": ("const int32_t nU = n_steps * b->Hq;", "const int32_t nU = b->Hq;"),
}

PIN_CALLS = [
    "p.test_fp8_decode_all_codes_match_torch()",
    "p.test_geometry_closed_form(16384, 64, 2048, (14336, 224, 2048))",
    "p.test_geometry_closed_form(5000, 64, 1024, (3968, 62, 1032))",
    "p.test_score_brute_force_exact(0)",
    "p.test_score_brute_force_exact(2)",
    "p.test_select_zero_logit_not_selected()",
    "p.test_refine_brute_force_exact(0)",
    "p.test_refine_brute_force_exact(2)",
    "p.test_topk_matches_textbook_sort_and_ties()",
    "p.test_full_selection_equals_dense_attention('f32_sep')",
    "p.test_no_selection_equals_sliding_window_attention()",
    "p.test_attention_closed_forms()",
    "p.test_union_is_union_of_single_layers(1)",
    "p.test_union_special_cases()",
    "p.test_sigmoid_against_double_and_closed_forms()",
    "p.test_sigmoid_score_brute_force(0)",
    "p.test_sigmoid_score_special_cases()",
    "p.test_chunk_mass_brute_force('f32_sep')",
    "p.test_chunk_mass_total_and_closed_forms()",
]

RUNNER = """
import sys
sys.path.insert(0, {root!r})
from oracle import oracle
oracle.load({so!r})
from tests import test_oracle_pins as p
for call in {calls!r}:
    try:
        eval(call)
    except AssertionError:
        print("CAUGHT", call)
        sys.exit(0)
sys.exit(3)
"""


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, name
    src = tmp_path / "mut.c"
    src.write_text(SRC.replace(old, new))
    so = tmp_path / "mut.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(so), "-lm"])
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = RUNNER.format(root=root, so=str(so), calls=PIN_CALLS)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0 and "CAUGHT" in res.stdout, (
        f"no pin caught mutation {name}: rc={res.returncode}\n{res.stdout[-2000:]}"
        f"\n{res.stderr[-2000:]}")
