"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake in the copy (a dropped term, a
transposed operand, a wrong sign or exponent, the wrong nibble order, a
missing absolute value or scale, a narrower accumulator, a single rounding
where the definition has two), compiles it on the CPU, points the oracle
front end at it and runs the pin tests: at least one of them must fail.
Nothing here touches a GPU.
"""
import contextlib
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_golden
import test_oracle_dequant as t_dq
import test_oracle_f16 as t_f16
import test_oracle_f64emu as t_fe
import test_oracle_int4 as t_i4
import test_oracle_int8 as t_i8
import test_oracle_quant as t_qz

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "i8_dropped_last_k": ("for (int64_t k = 0; k < K; ++k)\n                s += (int64_t)A[i * K + k] * (int64_t)B[j * K + k];",
                          "for (int64_t k = 0; k < K - 1; ++k)\n                s += (int64_t)A[i * K + k] * (int64_t)B[j * K + k];"),
    "i8_transposed_b": ("s += (int64_t)A[i * K + k] * (int64_t)B[j * K + k];\n            if (s < INT32_MIN",
                        "s += (int64_t)A[i * K + k] * (int64_t)B[(k % N) * K + (j % K)];\n            if (s < INT32_MIN"),
    "i8_wrong_sign": ("s += (int64_t)A[i * K + k] * (int64_t)B[j * K + k];\n            if (s < INT32_MIN",
                      "s -= (int64_t)A[i * K + k] * (int64_t)B[j * K + k];\n            if (s < INT32_MIN"),
    "i8_int32_accumulator": ("int oracle_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B,\n              int32_t *C, int64_t row_begin, int64_t row_end)\n{\n    if (bad_range(M, row_begin, row_end))\n        return ORACLE_BAD_RANGE;\n    int status = ORACLE_OK;\n#pragma omp parallel for schedule(dynamic, 1)\n    for (int64_t i = row_begin; i < row_end; ++i) {\n        for (int64_t j = 0; j < N; ++j) {\n            int64_t s = 0;",
                             "int oracle_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B,\n              int32_t *C, int64_t row_begin, int64_t row_end)\n{\n    if (bad_range(M, row_begin, row_end))\n        return ORACLE_BAD_RANGE;\n    int status = ORACLE_OK;\n#pragma omp parallel for schedule(dynamic, 1)\n    for (int64_t i = row_begin; i < row_end; ++i) {\n        for (int64_t j = 0; j < N; ++j) {\n            int32_t s = 0;"),
    "i4_wrong_twos_complement": ("return d >= 8 ? d - 16 : d;", "return d >= 8 ? d - 15 : d;"),
    # (a consistent nibble-order swap in both operands permutes k identically
    # and leaves C unchanged, so it is not a mistake; pairing different k of A
    # and B is)
    "i4_mismatched_pairing": ("s += nibble_value(a, k) * nibble_value(b, k);",
                              "s += nibble_value(a, k) * nibble_value(b, k ^ 1);"),
    "i4_unsigned_nibble": ("return d >= 8 ? d - 16 : d;", "return d;"),
    "f16_exponent_bias": ("mag = ldexp((double)(1024 + f), e - 25);", "mag = ldexp((double)(1024 + f), e - 24);"),
    "f16_subnormal_scale": ("mag = ldexp((double)f, -24);", "mag = ldexp((double)f, -25);"),
    "f16_den_without_abs": ("d += fabs(a) * fabs(b);", "d += a * b;"),
    "f16_float_accumulator": ("double s = 0.0, d = 0.0;", "float s = 0.0f; double d = 0.0;"),
    "dq_missing_col_scale": ("t = t * col_scale[j];", "t = t * 1.0f;"),
    "qz_divide_by_128": ("volatile float s = (float)amax / 127.0f;", "volatile float s = (float)amax / 128.0f;"),
    "qz_round_half_away": ("float r = rintf(t);", "float r = roundf(t);"),
    "qz_reciprocal_multiply": ("volatile float t = v / s;", "volatile float t = v * (1.0f / s);"),
    "fe_scale_exponent_off_by_one": ("Bi[j * K + k] = (int64_t)rint(ldexp(B_t[j * K + k], bits - eB[j]));",
                                     "Bi[j * K + k] = (int64_t)rint(ldexp(B_t[j * K + k], bits - eB[j] + 1));"),
    "fe_round_half_away": ("Ai[k] = (int64_t)rint(ldexp(A[i * K + k], bits - eA));",
                           "Ai[k] = (int64_t)round(ldexp(A[i * K + k], bits - eA));"),
    "fe_double_accumulator": ("__int128 x = 0;", "double x = 0;"),
    "dq_single_rounding": ("volatile float t = (float)(int32_t)s;\n            t = t * row_scale[i];\n            t = t * col_scale[j];",
                           "volatile float t = (float)((double)(int32_t)s * row_scale[i] * col_scale[j]);"),
}

# the pins each mutation's family is checked with (each call raises on a failed pin)
PINS = {
    "i8": [lambda: t_i8.test_brute_force_tiny(3, 5, 7), lambda: t_i8.test_brute_force_tiny(8, 8, 16),
           lambda: t_i8.test_numpy_int64_matmul(64, 48, 80), t_i8.test_identity, t_i8.test_permutation,
           lambda: t_i8.test_closed_forms(16), t_i8.test_int32_range_guard, t_i8.test_transpose_symmetry,
           test_golden.test_int8_worked],
    "i4": [t_i4.test_decode_exhaustive, lambda: t_i4.test_matches_integer_product(5, 7, 32),
           lambda: t_i4.test_closed_forms(32), test_golden.test_int4_worked],
    "f16": [t_f16.test_decode_all_patterns, t_f16.test_decode_landmarks,
            lambda: t_f16.test_integer_valued_equals_int_oracle(7, 9, 16),
            lambda: t_f16.test_exact_rational_bound(2, 3, 64, 100.0), t_f16.test_subnormal_and_signs,
            test_golden.test_fp16_worked],
    "qz": [lambda: t_qz.test_exact_rational(6, 64, 1.0), lambda: t_qz.test_exact_rational(4, 200, 30.0),
           t_qz.test_integer_row_with_127_is_identity, t_qz.test_zero_row, t_qz.test_ties_to_even,
           t_qz.test_extremes_map_to_127, t_qz.test_reconstruction_bound, t_qz.test_tie_fixtures],
    "fe": [lambda: t_fe.test_exact_inputs_give_correctly_rounded_product(53),
           lambda: t_fe.test_truncation_bound(20), t_fe.test_power_of_two_row_scaling_is_exact,
           t_fe.test_scaling_rounds_ties_to_even, t_fe.test_zero_rows_and_columns,
           t_fe.test_cancellation_needs_the_exact_integer_sum],
    "dq": [t_dq.test_power_of_two_scales_exact, lambda: t_dq.test_three_rounding_bound(33, 7, 512),
           t_dq.test_scale_index_orientation, test_golden.test_dequant_worked,
           test_golden.test_dequant_two_roundings],
}


@contextlib.contextmanager
def oracle_library(path):
    saved = oracle._lib
    oracle._lib = oracle._configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        oracle._lib = saved


def build_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation {name} does not apply"
    c = tmp_path / f"{name}.c"
    c.write_text(src.replace(old, new, 1))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC",
                    str(c), "-o", str(so), "-lm"], check=True)
    return str(so)


def test_unmutated_copy_passes_every_pin(tmp_path):
    so = build_variant(tmp_path, "identity", "#define ORACLE_OK 0", "#define ORACLE_OK 0")
    with oracle_library(so):
        for family in PINS.values():
            for pin in family:
                pin()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(tmp_path, name):
    old, new = MUTATIONS[name]
    so = build_variant(tmp_path, name, old, new)
    family = name.split("_")[0]
    caught = []
    with oracle_library(so):
        for pin in PINS[family]:
            try:
                pin()
            except (AssertionError, oracle.OracleError, pytest.fail.Exception):
                caught.append(pin)
    assert caught, f"no pin caught mutation {name}"
    np.testing.assert_equal(len(caught) > 0, True)
