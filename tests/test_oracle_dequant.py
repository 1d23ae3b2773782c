"""Pins of the dequantising int8 oracle: power-of-two scales give an exact
closed form; general scales stay within the three-rounding bound of the real
product acc * rs[i] * cs[j] (which also catches a row/column scale swap,
since the scales differ by far more than the bound); unit scales return the
integer product."""
import numpy as np
import pytest

import oracle
from precision_dense_gemm_02_amd import inputs


def test_power_of_two_scales_exact():
    p = inputs.int8_problem(24, 40, 256, seed=21)
    rs = np.full(24, 2.0 ** -8, np.float32)
    cs = np.full(40, 2.0 ** -7, np.float32)
    out = oracle.gemm_i8_dequant(p.a, p.b_t, rs, cs)
    acc = p.a.astype(np.int64) @ p.b_t.astype(np.int64).T     # |acc| <= 2^22: exact in fp32
    np.testing.assert_array_equal(out.astype(np.float64), acc * 2.0 ** -15)


def test_unit_scales_give_integer_product():
    p = inputs.int8_problem(16, 16, 1024, seed=22)
    out = oracle.gemm_i8_dequant(p.a, p.b_t, np.ones(16, np.float32), np.ones(16, np.float32))
    acc = p.a.astype(np.int64) @ p.b_t.astype(np.int64).T
    np.testing.assert_array_equal(out.astype(np.float64), acc.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(16, 64, 4096), (33, 7, 512)])
def test_three_rounding_bound(M, N, K):
    p = inputs.int8_problem(M, N, K, seed=M * N, scales=True)
    out = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale)
    acc = (p.a.astype(np.int64) @ p.b_t.astype(np.int64).T).astype(np.float64)
    exact = acc * p.row_scale.astype(np.float64)[:, None] * p.col_scale.astype(np.float64)[None, :]
    u = 2.0 ** -24
    bound = ((1 + u) ** 3 - 1) * np.abs(exact) + 1e-300
    assert (np.abs(out.astype(np.float64) - exact) <= bound).all()


def test_scale_index_orientation():
    # row scales and column scales far apart: using cs[i] or rs[j] would be
    # off by orders of magnitude
    M, N, K = 3, 5, 16
    A = np.ones((M, K), np.int8)
    B_t = np.ones((N, K), np.int8)
    rs = np.array([1.0, 2.0, 4.0], np.float32)
    cs = np.array([1e-3, 1e-2, 1e-1, 1.0, 10.0], np.float32)
    out = oracle.gemm_i8_dequant(A, B_t, rs, cs)
    for i in range(M):
        for j in range(N):
            assert out[i, j] == np.float32(np.float32(16.0 * rs[i]) * cs[j])
