"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is the oracle's own C source with one plausible mistake written in
(a dropped term, a wrong rounding, a swapped index, a wrong constant).  It is
compiled with the oracle's flags into a temporary library and the pins of
``oracle_pins`` run against it; a mutant that passes every pin would mean the
pins cannot see that kind of mistake.  Nothing here touches a GPU.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from tests import oracle_pins

MUTANTS = [
    ("round_half_away", "float r = rintf(t);", "float r = roundf(t);"),
    ("params_inv_from_scale", "            v = 15.0f / r;\n", "            v = 1.0f / s;\n"),
    ("params_scale_times_reciprocal", "            s = r / 15.0f;\n", "            s = r * (1.0f / 15.0f);\n"),
    ("params_m16_scale_not_rounded", "            s = oracle_f16_to_f32(oracle_f32_to_f16(r / 15.0f));\n",
     "            s = r / 15.0f;\n"),
    ("params_m16_inv_of_range", "            v = s != 0.0f ? 1.0f / s : 0.0f;\n", "            v = s != 0.0f ? 15.0f / r : 0.0f;\n"),
    ("m16_codes_against_binary32_scale", "        float inv = 1.0f / scale;\n",
     "        float inv = 15.0f / rng;\n"),
    ("m16_scale_truncated", "s16 = oracle_f32_to_f16(rng / 15.0f);",
     "s16 = oracle_f32_to_f16(rng / 15.0f);\n    if (oracle_f16_to_f32(s16) > rng / 15.0f)\n        s16 -= 1;"),
    ("m16_no_underflow_case", "    if (scale == 0.0f) {\n        for", "    if (rng == 0.0f) {\n        for"),
    ("m16_min_rounded", "    *out_min = oracle_f32_to_f16(mn);", "    *out_min = oracle_f32_to_f16(mn * 1.0005f);"),
    ("m16_codes_truncated", "            float r = rintf(t);\n            if (r < 0.0f)\n                r = 0.0f;\n            if (r > 15.0f)\n                r = 15.0f;\n            c[i] = (int)r;\n        }\n    }\n    pack_codes(c, codes);\n    *out_min = oracle_f32_to_f16(mn);",
     "            float r = floorf(t);\n            if (r < 0.0f)\n                r = 0.0f;\n            if (r > 15.0f)\n                r = 15.0f;\n            c[i] = (int)r;\n        }\n    }\n    pack_codes(c, codes);\n    *out_min = oracle_f32_to_f16(mn);"),
    ("w_dequant_drops_min", "int64_t units = (int64_t)llround(ldexp(mn, 24)) + (int64_t)code",
     "int64_t units = (int64_t)code"),
    ("w_dequant_rounds_down", "if (rem * 2 > q || (rem * 2 == q && ((lo / q) & 1)))", "if (0)"),
    ("w_dequant_ties_up", "if (rem * 2 > q || (rem * 2 == q && ((lo / q) & 1)))", "if (rem * 2 >= q)"),
    ("w_gemm_neighbour_group", "            int g = k / ORACLE_GROUP;\n            int c = oracle_code_at",
     "            int g = (k / ORACLE_GROUP + 1) % G;\n            int c = oracle_code_at"),
    ("w_gemm_x_reversed", "(double)oracle_f16_to_f32(x[(size_t)m * K + k])",
     "(double)oracle_f16_to_f32(x[(size_t)m * K + (K - 1 - k)])"),
    ("truncate_codes", "float r = rintf(t);", "float r = floorf(t);"),
    ("scale_over_16", "scale = rng / 15.0f;", "scale = rng / 16.0f;"),
    ("inv_over_16", "float inv = 15.0f / rng;", "float inv = 16.0f / rng;"),
    ("no_signed_zero_fix", "    *out_mn = mn + 0.0f;\n", "    *out_mn = mn;\n"),
    ("nibbles_swapped", "codes[j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));",
     "codes[j] = (uint8_t)((c[2 * j] << 4) | c[2 * j + 1]);"),
    ("dequant_drops_min", "* (double)row_scales[g] + (double)row_mins[g];", "* (double)row_scales[g];"),
    ("dequant_uses_next_group_scale", "(double)row_scales[g] + (double)row_mins[g]",
     "(double)row_scales[g ? g - 1 : g + 1] + (double)row_mins[g]"),
    ("dequant_f16_drops_min", "    v = v + row_mins[g];\n", "\n"),
    ("dequant_f16_scaled", "    return oracle_f32_to_f16(v);\n}\n\nvoid oracle_dequant_rows",
     "    return oracle_f32_to_f16(v * 1.0001f);\n}\n\nvoid oracle_dequant_rows"),
    ("min_misses_last_element", "for (int i = 1; i < ORACLE_GROUP; ++i) {\n        if (f[i] < mn)",
     "for (int i = 1; i < ORACLE_GROUP - 1; ++i) {\n        if (f[i] < mn)"),
    ("second_group_reads_first", "oracle_quantize_group(x + g * ORACLE_GROUP,", "oracle_quantize_group(x,"),
    ("m16_rows_every_group_reads_group_0", "oracle_quantize_group_m16(x + (size_t)r * d + g * ORACLE_GROUP,",
     "oracle_quantize_group_m16(x + (size_t)r * d,"),
    ("m16_rows_min_to_group_0_slot", "mins + (size_t)r * G + g,\n", "mins + (size_t)r * G,\n"),
    ("m16_rows_scale_to_group_0_slot", "                                      scales + (size_t)r * G + g);",
     "                                      scales + (size_t)r * G);"),
    ("m16_rows_codes_of_group_0", "codes + (size_t)r * (d / 2) + g * (ORACLE_GROUP / 2), mins",
     "codes + (size_t)r * (d / 2), mins"),
    ("f16_round_down", "double r = nearbyint(a / quantum) * quantum;", "double r = floor(a / quantum) * quantum;"),
    ("f16_subnormal_scale", "v = ldexpf((float)frac, -24);", "v = ldexpf((float)frac, -25);"),
    ("score_scale_1_over_d", "double c = 1.0 / sqrt((double)d);\n    for (int t = 0; t < T; ++t)",
     "double c = 1.0 / (double)d;\n    for (int t = 0; t < T; ++t)"),
    ("query_reversed", "double qi = (double)oracle_f16_to_f32(q[i]);", "double qi = (double)oracle_f16_to_f32(q[d - 1 - i]);"),
    ("no_normalisation", "        out[i] = acc / l;\n    }\n    free(s);", "        out[i] = acc;\n    }\n    free(s);"),
    ("softmax_without_exp", "        s[t] = exp(s[t] - m);", "        s[t] = s[t] - m + 1.0;"),
    ("subset_v_index", "            int t = idx[j];", "            int t = j;"),
    ("topk_ties_to_larger", "if (best < 0 || scores[t] > scores[best])", "if (best < 0 || scores[t] >= scores[best])"),
    ("prefill_not_causal", "    for (int t = 0; t <= i; ++t) {\n        const uint16_t *kt",
     "    for (int t = 0; t < s; ++t) {\n        const uint16_t *kt"),
    ("prefill_excludes_self", "    for (int t = 0; t <= i; ++t) {\n        const uint16_t *kt",
     "    for (int t = 0; t < i; ++t) {\n        const uint16_t *kt"),
    ("prefill_scale_1_over_d", "    double c = 1.0 / sqrt((double)d);\n    const uint16_t *qi",
     "    double c = 1.0 / (double)d;\n    const uint16_t *qi"),
    ("prefill_v_from_k", "acc += p[t] * (double)oracle_f16_to_f32(v[", "acc += p[t] * (double)oracle_f16_to_f32(k["),
    ("prefill_query_row_0", "const uint16_t *qi = q + (size_t)i * stride;", "const uint16_t *qi = q;"),
    ("prefill_no_normalisation", "        out_row[e] = acc / l;", "        out_row[e] = acc;"),
    ("prefill_rows_wrong_row", "        prefill_row(d, s, rows[j], stride", "        prefill_row(d, s, j, stride"),
    ("rows_attend_scale_1_over_d", "    double c = 1.0 / sqrt((double)d);\n    if (T < 1)\n        return;\n    double *p",
     "    double c = 1.0 / (double)d;\n    if (T < 1)\n        return;\n    double *p"),
    ("rows_attend_no_exp", "        p[t] = exp(p[t] - m);\n        l += p[t];", "        p[t] = p[t] - m + 1.0;\n        l += p[t];"),
    ("rows_attend_v_from_k", "acc += p[t] * vhat[(size_t)t * d + i];", "acc += p[t] * khat[(size_t)t * d + i];"),
    ("rows_attend_no_normalisation", "        out[i] = acc / l;\n    }\n    free(p);\n}\n\n/* ----",
     "        out[i] = acc;\n    }\n    free(p);\n}\n\n/* ----"),
    ("topk_smallest", "if (best < 0 || scores[t] > scores[best])", "if (best < 0 || scores[t] < scores[best])"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    src = oracle.source_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    bad = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as td:
        path = oracle.compile_variant(bad, os.path.join(td, f"mut_{name}.so"))
        failed = []
        with oracle.use_library(path), np.errstate(all="ignore"):
            for pin in oracle_pins.ALL_PINS:
                try:
                    pin()
                except (AssertionError, ValueError, IndexError, OverflowError):
                    failed.append(pin.__name__)
        assert failed, f"mutant {name} passes every pin"
