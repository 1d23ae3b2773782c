"""Pins of the int4 oracle: the nibble decoding against the two's-complement
definition (exhaustive), the packing order (low nibble = even k), and the
product against independent integer arithmetic on the unpacked values."""
import numpy as np
import pytest

import oracle
from precision_dense_gemm_02_amd import inputs


def twos_complement_nibble(n):
    return n - 16 if n >= 8 else n


def test_decode_exhaustive():
    # A row i is the single byte i (K = 2).  B row 0 = 0x01 selects the low
    # nibble (value 1 at k = 0), B row 1 = 0x10 selects the high nibble.
    A = np.arange(256, dtype=np.uint8).reshape(256, 1)
    B = np.array([[0x01], [0x10]], np.uint8)
    C = oracle.gemm_i4(A, B, K=2)
    for byte in range(256):
        assert C[byte, 0] == twos_complement_nibble(byte & 0xF)
        assert C[byte, 1] == twos_complement_nibble(byte >> 4)


def test_pack_unpack_identity_exhaustive():
    # every (even-k value, odd-k value) pair
    lo, hi = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    vals = np.stack([lo.ravel(), hi.ravel()], axis=1).astype(np.int8)   # 256 x 2
    packed = inputs.pack_int4(vals)
    assert packed.shape == (256, 1)
    for r in range(256):
        b = int(packed[r, 0])
        assert twos_complement_nibble(b & 0xF) == vals[r, 0]
        assert twos_complement_nibble(b >> 4) == vals[r, 1]
    # a bijection onto all 256 byte values
    assert sorted(packed.ravel().tolist()) == list(range(256))


def test_low_nibble_is_even_k():
    v = np.array([[1, -2, 3, -8]], np.int8)
    assert inputs.pack_int4(v).tolist() == [[0xE1, 0x83]]


@pytest.mark.parametrize("M,N,K", [(1, 1, 2), (5, 7, 32), (33, 17, 64), (64, 64, 256)])
def test_matches_integer_product(M, N, K):
    p = inputs.int4_problem(M, N, K, seed=M + N + K)
    got = oracle.gemm_i4(p.a_packed, p.b_packed, K)
    expect = p.a_values.astype(np.int64) @ p.b_values.astype(np.int64).T
    np.testing.assert_array_equal(got, expect)
    np.testing.assert_array_equal(got, oracle.gemm_i8(p.a_values, p.b_values))


def test_brute_force_tiny():
    p = inputs.int4_problem(3, 4, 6, seed=5)
    a, b = p.a_values.tolist(), p.b_values.tolist()
    expect = [[sum(a[i][k] * b[j][k] for k in range(6)) for j in range(4)] for i in range(3)]
    assert oracle.gemm_i4(p.a_packed, p.b_packed, 6).tolist() == expect


@pytest.mark.parametrize("K", [2, 32, 4096])
def test_closed_forms(K):
    m8 = inputs.pack_int4(np.full((2, K), -8, np.int8))
    p7 = inputs.pack_int4(np.full((3, K), 7, np.int8))
    assert (oracle.gemm_i4(m8, m8, K) == 64 * K).all()
    assert (oracle.gemm_i4(m8, p7, K) == -56 * K).all()
    assert (oracle.gemm_i4(p7, p7, K) == 49 * K).all()


def test_linearity():
    rng = np.random.default_rng(12)
    M, N, K = 11, 13, 64
    A = rng.integers(-8, 8, (M, K), dtype=np.int8)
    B1 = rng.integers(-4, 4, (N, K), dtype=np.int8)
    B2 = rng.integers(-4, 4, (N, K), dtype=np.int8)
    Ap = inputs.pack_int4(A)
    lhs = oracle.gemm_i4(Ap, inputs.pack_int4(B1 + B2), K)
    rhs = (oracle.gemm_i4(Ap, inputs.pack_int4(B1), K).astype(np.int64)
           + oracle.gemm_i4(Ap, inputs.pack_int4(B2), K))
    np.testing.assert_array_equal(lhs, rhs)


def test_odd_k_refused():
    with pytest.raises(oracle.OracleError):
        oracle._check(oracle._load().oracle_i4(1, 1, 3, 0, 0, 0, 0, 1))
