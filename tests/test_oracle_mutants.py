"""The pins must catch plausible mistakes in the oracle.

Each case copies oracle.c with one planted mistake (a dropped term, a wrong
sign, index, order or constant), builds it on the CPU, and checks that at
least one pin fails on it.  The real oracle is never modified.
"""
import os

import pytest

import oracle as oracle_pkg
from tests import pins

# (name, original text, mutated text); each original must occur exactly once
MUTANTS = [
    ("round_half_away", "float r = rintf(t);", "float r = roundf(t);"),
    ("truncate", "float r = rintf(t);", "float r = truncf(t);"),
    ("scale_128", "return u2f(amax_bits) / 127.0f;", "return u2f(amax_bits) / 128.0f;"),
    ("scale_times_recip", "return u2f(amax_bits) / 127.0f;",
     "return u2f(amax_bits) * (1.0f / 127.0f);"),
    ("quotient_times_recip", "float t = g / s;", "float t = g * (1.0f / s);"),
    ("no_low_clamp", "    if (r < -128.0f)\n        r = -128.0f;\n", ""),
    ("symmetric_clamp", "r = -128.0f;", "r = -127.0f;"),
    ("no_zero_scale_rule", "    if (s == 0.0f)\n        return 0;\n", ""),
    ("absmax_signed", "f2u(g[i]) & 0x7fffffffu", "f2u(g[i])"),
    ("absmax_first_only", "        if (a > m)\n            m = a;", "        if (i == 0)\n            m = a;"),
    ("reduce_reverse_order", "for (int32_t w = 0; w < W; ++w) {",
     "for (int32_t w = W - 1; w >= 0; --w) {"),
    ("reduce_fused_multiply_add", "float d = (float)q[w][i] * s[w][u];\n                acc = acc + d;",
     "acc = fmaf((float)q[w][i], s[w][u], acc);"),
    ("reduce_rank0_scale", "float d = (float)q[w][i] * s[w][u];", "float d = (float)q[w][i] * s[0][u];"),
    ("reduce_pairwise",
     "float acc = 0.0f;\n            for (int32_t w = 0; w < W; ++w) {\n"
     "                float d = (float)q[w][i] * s[w][u];\n                acc = acc + d;\n            }",
     "float acc = 0.0f, acc2 = 0.0f;\n            for (int32_t w = 0; w < W; ++w) {\n"
     "                float d = (float)q[w][i] * s[w][u];\n"
     "                if (w & 1) acc2 = acc2 + d; else acc = acc + d;\n            }\n"
     "            acc = acc + acc2;"),
    ("half_exponent_bias", "v = ldexpf((float)(1024 + f), e - 25);", "v = ldexpf((float)(1024 + f), e - 24);"),
    ("half_subnormal_scale", "v = ldexpf((float)f, -24);", "v = ldexpf((float)f, -25);"),
    ("unscale_dropped", "g[i] = v * in_mul;", "g[i] = v;"),
    ("plan_floor_split", "int64_t c = (numel + k - 1) / k;", "int64_t c = numel / k + (numel % k ? 0 : 0);\n    if (c < 1) c = 1;"),
    ("plan_no_alignment", "int64_t denom = chunk_bytes - chunk_bytes % align_bytes;", "int64_t denom = chunk_bytes;"),
    ("plan_round_count", "int64_t k = nbytes / denom;", "int64_t k = (nbytes + denom - 1) / denom;"),
    ("requantize_with_amax_off_by_one", "float s = oracle_scale(amax[u]);", "float s = oracle_scale(amax[u] + 1);"),
    ("sum_reverse_order", "for (int32_t rank = 0; rank < W; ++rank) {",
     "for (int32_t rank = W - 1; rank >= 0; --rank) {"),
    ("sum_mean_times_recip", "r_out[i] = r_out[i] / (float)W;",
     "r_out[i] = r_out[i] * (1.0f / (float)W);"),
    ("sum_skips_unscale", "oracle_load(x[rank], kind, in_mul, n, g);",
     "oracle_load(x[rank], kind, 1.0f, n, g);"),
    ("report_dequant_in_double", "double d = (double)((float)q[i] * scale[u]);",
     "double d = (double)q[i] * (double)scale[u];"),
    ("report_scale_of_unit0", "double d = (double)((float)q[i] * scale[u]);",
     "double d = (double)((float)q[i] * scale[0]);"),
    ("report_signed_ref_sum", "sum_ref = sum_ref + fabs(r);", "sum_ref = sum_ref + r;"),
    ("report_cos_wrong_norm", "o[9] = dr / sqrt(dd * rr);", "o[9] = dr / sqrt(dd * dd);"),
    ("report_no_zero_ratio_rule", "    if (a == 0.0 && b == 0.0)\n        return 0.0;\n", ""),
    ("report_max_ref_of_error", "if (abs_bits(r) > max_ref)\n                max_ref = abs_bits(r);",
     "if (abs_bits(e) > max_ref)\n                max_ref = abs_bits(e);"),
    ("report_mean_rel_inverted", "o[5] = ratio_or_zero(sum_err, sum_ref);",
     "o[5] = ratio_or_zero(sum_ref, sum_err);"),
    ("chunker_no_capacity", "int64_t first = count > capacity ? count - capacity : 0;",
     "int64_t first = 0;"),
    ("chunker_alpha_swapped", "e = alpha * x + (1.0 - alpha) * e;",
     "e = (1.0 - alpha) * x + alpha * e;"),
    ("chunker_tie_to_smaller", "(e == best_cost && c > best_size)", "(e == best_cost && c < best_size)"),
    ("chunker_raw_latency", "double x = lat[j] / (double)c;", "double x = lat[j];"),
    ("chunker_start_from_zero", "                e = x;\n                started = 1;",
     "                e = alpha * x;\n                started = 1;"),
    ("chunker_capacity_off_by_one", "int64_t first = count > capacity ? count - capacity : 0;",
     "int64_t first = count > capacity ? count - capacity + 1 : 0;"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle_pkg.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, source, name, old, new):
    assert source.count(old) == 1, "mutation anchor not found once: " + name
    src = tmp_path / ("oracle_%s.c" % name)
    src.write_text(source.replace(old, new))
    so = str(tmp_path / ("liboracle_%s.so" % name))
    oracle_pkg.build(str(src), so)
    o = oracle_pkg.Oracle(oracle_pkg.load(so))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake " + name
