"""The pins must catch plausible mistakes in the oracle.

Each case compiles a copy of oracle/tq_oracle.c with one planted mistake (on
the CPU, into a temporary directory), points the oracle wrapper at it, and
requires that at least one of the pin tests fails.  The real oracle is
restored afterwards.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_fake_quantize_f32 as fq32
from tests import test_oracle_format as fmt
from tests import test_oracle_matmul as mm
from tests import test_oracle_scale as sc
from tests import test_oracle_w4a16 as w4

SRC = os.path.join(os.path.dirname(oracle.__file__), "tq_oracle.c")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MUTATIONS = {
    "digit_order_msd_first": ("byte += (code[5 * b + i] + 1) * p3;",
                              "byte += (code[5 * b + (4 - i)] + 1) * p3;"),
    "dropped_last_term_in_sum": ("    for (int64_t j = 0; j < G; ++j) {\n        uint64_t sig; int e;",
                                 "    for (int64_t j = 0; j < G - 1; ++j) {\n        uint64_t sig; int e;"),
    "tie_rounds_up": ("else if (2 * r == G) up = f_pos ? 1 : (int)(q & 1);",
                      "else if (2 * r == G) up = 1;"),
    "code_tie_away_from_zero": ("code[j] = (int8_t)(v > half ? 1 : (v < -half ? -1 : 0));",
                                "code[j] = (int8_t)(v >= half ? 1 : (v <= -half ? -1 : 0));"),
    "code_sign_flipped": ("code[j] = (int8_t)(v > half ? 1 : (v < -half ? -1 : 0));",
                          "code[j] = (int8_t)(v > half ? -1 : (v < -half ? 1 : 0));"),
    "padding_trit_minus_one": ("code[t] = 0;  /* padding = 0 */", "code[t] = -1;  /* padding */"),
    "invalid_threshold_off_by_one": ("int valid = v < 243;", "int valid = v < 242;"),
    "padding_not_checked": ("else if (valid && d != 1) st |= OR_BAD_PADDING;", "else {}"),
    "scale_of_first_group_only": ("wrow[g * G + j] = (double)crow[g * G + j] * s;",
                                  "wrow[g * G + j] = (double)crow[g * G + j] * f16_to_double(scales[n * nG]);"),
    "x_transposed": ("const double *xm = xd + m * K;", "const double *xm = xd + m;"),
    "bound_not_absolute": ("bacc += fabs(t);", "bacc += t;"),
    "w4_nibbles_high_first": ("return (int)((row[k / 8] >> (4 * (k % 8))) & 0xFu);",
                              "return (int)((row[k / 8] >> (4 * (7 - k % 8))) & 0xFu);"),
    "w4_matmul_nibbles_high_first": ("const double q = (double)((word >> (4 * i)) & 0xFu);",
                                     "const double q = (double)((word >> (4 * (7 - i))) & 0xFu);"),
    "w4_bias_dropped": ("acc += a * (q * s + b);", "acc += a * (q * s);"),
    "w4_first_group_parameters_only": (
        "const double s = bf16_any_to_double(scales[n * nG + g]);",
        "const double s = bf16_any_to_double(scales[n * nG]);"),
    "w4_bound_without_bias": ("bacc += fabs(a) * (fabs(q * s) + fabs(b));",
                              "bacc += fabs(a) * fabs(q * s);"),
    "w4_activation_off_by_one_word": ("x[m * K + g * G + 8 * p + i]", "x[m * K + g * G + 8 * (p ^ 1) + i]"),
    "f32_sum_in_bf16_units": ("gst = scale_bits_of_sum(&A, G, 125, &sbits);",
                              "gst = scale_bits_of_sum(&A, G, 109, &sbits);"),
    "f32_mantissa_cut_to_bf16": ("    uint64_t m = u & 0x7FFFFFu;",
                                 "    uint64_t m = u & 0x7F0000u;"),
    "f32_code_tie_to_one": ("double c = v > 0.5 * s ? 1.0 : (v < -0.5 * s ? -1.0 : 0.0);",
                            "double c = v >= 0.5 * s ? 1.0 : (v <= -0.5 * s ? -1.0 : 0.0);"),
    "f32_flagged_group_keeps_codes": ("                if (!gst) {\n                    double v = f32_to_double(wg[j]);",
                                      "                if (1) {\n                    double v = f32_to_double(wg[j]);"),
}

PINS = [
    fmt.test_all_243_codewords_decode,
    fmt.test_all_243_codewords_encode_bijection,
    lambda: fmt.test_invalid_bytes_rejected(GOLDEN),
    fmt.test_group_alignment_and_padding_ranges,
    fmt.test_bad_padding_flagged,
    fmt.test_zero_group_and_zero_scale,
    lambda: fmt.test_hand_worked_group(GOLDEN),
    lambda: sc.test_scale_vs_fraction_normal(64),
    lambda: sc.test_scale_vs_fraction_wide_exponents(64),
    sc.test_scale_constructed_midpoints,
    sc.test_codes_tie_fixture,
    sc.test_codes_vs_numpy_rint,
    lambda: mm.test_matmul_vs_exact_rationals(3, 320, 64, 2),
    mm.test_matmul_vs_numpy_matmul,
    mm.test_one_hot_rows_exact,
    lambda: w4.test_packing_layout_fixture(GOLDEN),
    lambda: w4.test_orientation_example(GOLDEN),
    lambda: w4.test_matmul_vs_factored_form(17, 1024, 128, 2),
    w4.test_nonnegative_terms_bound_equals_y,
    lambda: fq32.test_normal_groups_match_exact_definition(64),
    lambda: fq32.test_wide_exponents_match_exact_definition(64),
    fq32.test_scale_uses_the_fp32_values,
    fq32.test_code_ties_at_fp32_resolution,
    fq32.test_flags_and_underflow,
]


FUNCTIONS = ("oracle_packed_row_bytes", "oracle_quantize_pack", "oracle_unpack", "oracle_matmul",
             "oracle_dequantize", "oracle_fake_quantize", "oracle_fake_quantize_f32",
             "oracle_quantize_pack2",
             "oracle_unpack2", "oracle_matmul2", "oracle_w4_unpack", "oracle_w4a16_dequantize",
             "oracle_w4a16_matmul", "oracle_quantize_pack_mt", "oracle_matmul_mt",
             "oracle_matmul2_mt", "oracle_w4a16_matmul_mt")


def _load_variant(path, real):
    """The mutated library, with every function's signature copied from the
    real oracle's."""
    lib = ctypes.CDLL(path)
    for f in FUNCTIONS:
        getattr(lib, f).argtypes = getattr(real, f).argtypes
        getattr(lib, f).restype = getattr(real, f).restype
    return lib


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must match exactly once"
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "libm.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O1", "-std=c11", "-w", "-fPIC", "-pthread", "-shared", "-o",
                               so, c, "-lm"])
        saved = oracle._load()
        oracle._lib = _load_variant(so, saved)
        failures = 0
        try:
            for pin in PINS:
                try:
                    pin()
                except (AssertionError, oracle.OracleError):
                    failures += 1
        finally:
            oracle._lib = saved
        assert failures > 0, "no pin caught mutation %s" % name
    finally:
        shutil.rmtree(d)
