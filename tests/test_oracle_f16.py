"""Pins of the fp16 oracle: the binary16 decoder over every bit pattern, exact
agreement with the integer oracle on integer-valued operands, and the fp64
summation against exact rational arithmetic within the recursive-summation
error bound."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from precision_dense_gemm_02_amd import inputs


def test_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(65536):
        v = oracle.f16_decode(b)
        if np.isfinite(ref[b]):
            assert v == ref[b], hex(b)
            if ref[b] == 0:
                assert np.signbit(v) == np.signbit(ref[b])
        else:
            assert v is None, hex(b)


def test_decode_landmarks():
    assert oracle.f16_decode(0x3C00) == 1.0
    assert oracle.f16_decode(0xC000) == -2.0
    assert oracle.f16_decode(0x0001) == 2.0 ** -24          # smallest subnormal
    assert oracle.f16_decode(0x03FF) == 1023 * 2.0 ** -24   # largest subnormal
    assert oracle.f16_decode(0x0400) == 2.0 ** -14          # smallest normal
    assert oracle.f16_decode(0x7BFF) == 65504.0             # largest finite
    assert oracle.f16_decode(0x7C00) is None
    assert oracle.f16_decode(0x7E00) is None


@pytest.mark.parametrize("M,N,K", [(7, 9, 16), (32, 40, 512)])
def test_integer_valued_equals_int_oracle(M, N, K):
    p = inputs.f16_integer_problem(M, N, K, seed=K)
    ref, den = oracle.gemm_f16(p.a, p.b_t)
    ai = p.a.astype(np.int8)
    bi = p.b_t.astype(np.int8)
    np.testing.assert_array_equal(ref, oracle.gemm_i8(ai, bi).astype(np.float64))
    np.testing.assert_array_equal(den, oracle.gemm_i8(np.abs(ai), np.abs(bi)).astype(np.float64))


def _exact(A, B_t):
    a = [[Fraction(float(x)) for x in row] for row in A.astype(np.float64)]
    b = [[Fraction(float(x)) for x in row] for row in B_t.astype(np.float64)]
    M, K = A.shape
    N = B_t.shape[0]
    s = [[sum((a[i][k] * b[j][k] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    d = [[sum((abs(a[i][k]) * abs(b[j][k]) for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    return s, d


@pytest.mark.parametrize("M,N,K,scale", [(3, 4, 24, 1.0), (2, 3, 64, 100.0), (4, 2, 40, 1e-3)])
def test_exact_rational_bound(M, N, K, scale):
    rng = np.random.default_rng(K)
    A = (rng.standard_normal((M, K)) * scale).astype(np.float16)
    B_t = rng.standard_normal((N, K)).astype(np.float16)
    ref, den = oracle.gemm_f16(A, B_t)
    s, d = _exact(A, B_t)
    u = Fraction(1, 2 ** 53)
    gamma = (K - 1) * u / (1 - (K - 1) * u)
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(ref[i, j]) - s[i][j]) <= gamma * d[i][j]
            assert abs(Fraction(den[i, j]) - d[i][j]) <= gamma * d[i][j]


def test_subnormal_and_signs():
    tiny = np.float16(2.0 ** -24)
    A = np.array([[tiny, -1.0, 0.5, 0.0]], np.float16)
    B_t = np.array([[1.0, 3.0, -0.25, 7.0]], np.float16)
    ref, den = oracle.gemm_f16(A, B_t)
    assert ref[0, 0] == 2.0 ** -24 - 3.0 - 0.125
    assert den[0, 0] == 2.0 ** -24 + 3.0 + 0.125


def test_nonfinite_refused():
    A = np.array([[np.inf, 1.0]], np.float16)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_f16(A, np.ones((1, 2), np.float16))
    A = np.array([[np.nan, 1.0]], np.float16)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_f16(A, np.ones((1, 2), np.float16))


def test_transpose_symmetry():
    p = inputs.f16_problem(9, 14, 64, seed=2)
    r1, d1 = oracle.gemm_f16(p.a, p.b_t)
    r2, d2 = oracle.gemm_f16(p.b_t, p.a)
    # the same products are added in the same k order, so this is bitwise
    np.testing.assert_array_equal(r1, r2.T)
    np.testing.assert_array_equal(d1, d2.T)


def test_rel_error_metric():
    ref = np.array([[1.0, 0.0, -2.0]])
    den = np.array([[2.0, 0.0, 4.0]])
    e = oracle.f16_rel_error(np.array([[1.002, 0.0, -2.0]], np.float32), ref, den)
    assert abs(e["max_rel"] - 0.001) < 1e-6
    e = oracle.f16_rel_error(np.array([[1.0, 1e-30, -2.0]], np.float32), ref, den)
    assert e["max_rel"] == np.inf
