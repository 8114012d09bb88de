"""Planted mistakes in the oracle must be caught by its pins.

Each case copies flexq_oracle.c, applies one plausible mistake (a dropped term,
a wrong index, sign or rounding, a transposed operand), builds the mutant on
the CPU, swaps it in for the real oracle and runs the pin tests: at least one
pin has to fail.  The real oracle source is never modified.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "flexq_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("mul_then_add_instead_of_fma", "acc = fmaf(t, s_a, acc);", "acc = t * s_a + acc;"),
    ("weight_qmax_32", "float s = amax / 31.0f;", "float s = amax / 32.0f;"),
    ("act_scale_of_first_group", "float s_a = w->sa[m * G + g];", "float s_a = w->sa[m * G];"),
    ("swapped_nibbles", "uint32_t b0 = lo[j] | (lo[4 + j] << 4);",
     "uint32_t b0 = lo[4 + j] | (lo[j] << 4);"),
    ("round_half_away", "q = (int)rintf(oracle_f16_to_f32(src[i]) / s);",
     "q = (int)roundf(oracle_f16_to_f32(src[i]) / s);"),
    ("dropped_last_product", "for (int64_t i = 0; i < len; ++i) d +=",
     "for (int64_t i = 0; i + 1 < len; ++i) d +="),
    ("unsigned_6bit_decode", "q[4 * p + j] = (int8_t)(v >= 32 ? v - 64 : v);",
     "q[4 * p + j] = (int8_t)v;"),
    ("weight_scale_transposed", "float t = (float)d * oracle_f16_to_f32(w->sw[n * G + g]);",
     "float t = (float)d * oracle_f16_to_f32(w->sw[g * w->N + n]);"),
    ("act_amax_sign", "float a = fabsf(oracle_f16_to_f32(src[i]));\n        if (a > amax) amax = a;\n      }\n      float s = 0.0f;",
     "float a = oracle_f16_to_f32(src[i]);\n        if (a > amax) amax = a;\n      }\n      float s = 0.0f;"),
    ("scale_not_rounded_to_fp16", "sf = oracle_f16_to_f32(s16);", "sf = s;"),
    ("tile_minor_major_swapped", "return 3 * (((n / 16) * units_per_row + u) * 16 + (n % 16));",
     "return 3 * (((n / 16) * 16 + (n % 16)) * units_per_row + u);"),
    ("act_a6_units_column_major", "oracle_pack_unit(qa + m * K + u * 16, qp + 3 * (m * (K / 16) + u));",
     "oracle_pack_unit(qa + m * K + u * 16, qp + 3 * (u * M + m));"),
    ("act_a6_accepts_8bit_codes", "if (qa[i] < -32 || qa[i] > 31) return -3;",
     "if (qa[i] < -128 || qa[i] > 127) return -3;"),
    ("block_rows_outside_halves", "return b * 16 * K + g * 2048 + h * 1024 + r * 64 + c;",
     "return b * 16 * K + g * 2048 + r * 128 + h * 64 + c;"),
]

PIN_TESTS = [
    (pins.test_pack_unit_golden, {"codes": list(range(-8, 8)),
                                  "words": [0xFBEAD9C8, 0x73625140, 0x0F0F0F0F]}),
    (pins.test_pack_unit_round_trip_every_code_every_position, {}),
    (pins.test_unit_offset_is_a_bijection_and_tiles_are_contiguous, {}),
    (pins.test_quant_act_matches_exact_rational_rounding, {"abits": 6}),
    (pins.test_quant_act_matches_exact_rational_rounding, {"abits": 8}),
    (pins.test_quant_w6_matches_exact_rational_rounding, {}),
    (pins.test_quant_w6_ties_reduce_to_round_half_even, {}),
] + [
    (pins.test_quant_act_ties_reduce_to_round_half_even,
     dict(zip(("abits", "xs", "scale", "codes"), row))) for row in pins._golden_ties()
] + [
    (pins.test_quant_act_invariants, {"abits": 6}),
    (pins.test_group_dots_match_numpy_integer_matmul, {"abits": 6}),
    (pins.test_gemm_within_fp32_bound_of_fp64_brute_force, {"abits": 8}),
    (pins.test_gemm_accumulation_in_exact_rationals, {}),
    (pins.test_gemm_power_of_two_scales_are_exact, {}),
    (pins.test_pack_act_a6_golden_units_in_row_order, {}),
    (pins.test_pack_act_a6_is_the_weight_unit_grid_transposed, {}),
    (pins.test_pack_act_a6_round_trip_and_range, {}),
    (pins.test_block_act_is_the_padded_reshape, {}),
    (pins.test_block_act_places_one_code_by_hand, {}),
]


def _build_mutant(orig, new, workdir):
    text = open(SRC).read()
    assert text.count(orig) == 1, f"mutation anchor not unique/present: {orig!r}"
    path = os.path.join(workdir, "mutant.c")
    with open(path, "w") as f:
        f.write(text.replace(orig, new))
    so = os.path.join(workdir, "libmutant.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                           "-ffp-contract=off", "-fno-fast-math", "-I",
                           os.path.dirname(SRC), path, "-o", so, "-lm"])
    return so


@pytest.mark.parametrize("name,orig,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, new):
    real = oracle._load()
    with tempfile.TemporaryDirectory() as d:
        so = _build_mutant(orig, new, d)
        oracle._lib = None
        saved = oracle._LIB_PATH
        oracle._LIB_PATH = so
        try:
            oracle._load()
            caught = []
            for fn, kw in PIN_TESTS:
                try:
                    fn(**kw)
                except (AssertionError, ValueError, IndexError):
                    caught.append(fn.__name__)
        finally:
            oracle._LIB_PATH = saved
            oracle._lib = real
    assert caught, f"no pin caught the planted mistake {name}"
