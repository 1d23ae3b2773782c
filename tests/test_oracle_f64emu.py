"""Pins of the fp64-emulation oracle (fp64 product through scaled integers):
exact inputs give the correctly rounded exact product; general inputs stay
inside the truncation bound derived from the definition; power-of-two
scaling of a row passes through exactly; ties in the scaling round to even;
zero rows give zeros.  Exact products come from Python Fractions."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def exact_product(A, B_t):
    M, K = A.shape
    N = B_t.shape[0]
    FA = [[Fraction(float(x)) for x in row] for row in A]
    FB = [[Fraction(float(x)) for x in row] for row in B_t]
    return [[sum(FA[i][k] * FB[j][k] for k in range(K)) for j in range(N)] for i in range(M)]


def frexp_exp(x):
    return int(np.frexp(x)[1]) if x != 0 else 0


@pytest.mark.parametrize("bits", [24, 40, 53])
def test_exact_inputs_give_correctly_rounded_product(bits):
    # integers of at most 11 significant bits times a power of two per row:
    # the scaling to `bits` bits is exact, so C = RN(exact A.B)
    rng = np.random.default_rng(bits)
    M, N, K = 5, 6, 40
    A = rng.integers(-2047, 2048, (M, K)).astype(np.float64) * np.exp2(rng.integers(-30, 30, (M, 1)))
    B_t = rng.integers(-2047, 2048, (N, K)).astype(np.float64) * np.exp2(rng.integers(-30, 30, (N, 1)))
    A[:, 0] = 2047 * np.exp2(np.log2(np.abs(A).max(1)).round())   # keep the row maxima wide
    C = oracle.f64_emu(A, B_t, bits)
    ex = exact_product(A, B_t)
    want = np.array([[float(v) for v in row] for row in ex])
    np.testing.assert_array_equal(C, want)


@pytest.mark.parametrize("bits", [12, 20, 32, 53])
def test_truncation_bound(bits):
    # |C - A.B| <= sum_k (dA_i |b| + |a| dB_j + dA_i dB_j) + ulp(|C|), with
    # dA_i = 2^(eA_i - bits - 1) the half unit of row i's scaled integers
    rng = np.random.default_rng(100 + bits)
    M, N, K = 4, 5, 48
    A = rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, 1)))
    B_t = rng.standard_normal((N, K)) * np.exp2(rng.integers(-8, 8, (N, 1)))
    C = oracle.f64_emu(A, B_t, bits)
    ex = exact_product(A, B_t)
    for i in range(M):
        dA = Fraction(2) ** (frexp_exp(np.abs(A[i]).max()) - bits - 1)
        for j in range(N):
            dB = Fraction(2) ** (frexp_exp(np.abs(B_t[j]).max()) - bits - 1)
            bound = sum(dA * abs(Fraction(B_t[j, k])) + abs(Fraction(A[i, k])) * dB + dA * dB
                        for k in range(K))
            bound += Fraction(np.spacing(abs(C[i, j])))
            assert abs(Fraction(C[i, j]) - ex[i][j]) <= bound, (bits, i, j)
    if bits == 53:
        # and at 53 bits the result is an fp64-accurate product
        np.testing.assert_allclose(C, A @ B_t.T, rtol=1e-13, atol=1e-13 * np.abs(A).max() * np.abs(B_t).max())


def test_power_of_two_row_scaling_is_exact():
    rng = np.random.default_rng(7)
    A = rng.standard_normal((3, 32))
    B_t = rng.standard_normal((4, 32))
    base = oracle.f64_emu(A, B_t, 30)
    A2 = A.copy()
    A2[1] *= 2.0 ** 37
    A2[2] *= 2.0 ** -41
    scaled = oracle.f64_emu(A2, B_t, 30)
    np.testing.assert_array_equal(scaled[0], base[0])
    np.testing.assert_array_equal(scaled[1], base[1] * 2.0 ** 37)
    np.testing.assert_array_equal(scaled[2], base[2] * 2.0 ** -41)


def test_scaling_rounds_ties_to_even():
    # row max 1.0 (exponent 1) at 2 bits: scale 2; 0.25 -> 0.5 -> 0 and
    # 0.75 -> 1.5 -> 2 (half away from zero would give 1 and 2)
    A = np.array([[1.0, 0.25, 0.75, -0.25]])
    B_t = np.eye(4)
    C = oracle.f64_emu(A, B_t, 2)
    np.testing.assert_array_equal(C, [[1.0, 0.0, 1.0, 0.0]])


def test_zero_rows_and_columns():
    A = np.zeros((2, 16))
    A[1, 3] = 5.0
    B_t = np.zeros((3, 16))
    B_t[2, 3] = -2.0
    C = oracle.f64_emu(A, B_t, 53)
    np.testing.assert_array_equal(C, [[0, 0, 0], [0, 0, -10.0]])


def test_refuses_bad_bits_and_nonfinite():
    A = np.ones((2, 8))
    with pytest.raises(oracle.OracleError):
        oracle.f64_emu(A, A, 0)
    with pytest.raises(oracle.OracleError):
        oracle.f64_emu(A, A, 54)
    A[1, 2] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.f64_emu(A, np.ones((2, 8)), 53)


def test_cancellation_needs_the_exact_integer_sum():
    # full 53-bit operands whose products cancel: at 53 bits the scaled sum
    # is 2^54 + 3, which a double accumulator would round to 2^54 before the
    # cancellation; the exact sum rounds once, to 2^54 + 4
    u = 2.0 ** -52
    A = np.array([[1 + 3 * u, 1.0]])
    B_t = np.array([[1 + u, -1.0]])
    C = oracle.f64_emu(A, B_t, 53)
    want = float(exact_product(A, B_t)[0][0])
    assert want == 2.0 ** -50 + 2.0 ** -102
    assert C[0, 0] == want
