"""GPU parity of the INT4 path through the FP6 E3M2 matrix cores.

The re-encoding is checked against E3M2 decoded from the format's definition
(sign bit, three exponent bits with bias 3, two mantissa bits; this file's
own decoder), and the GEMM bit for bit against the int4 oracle."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

E3M2_CONFIGS = (0, 20, 22, 45)   # the kernel configurations that run the E3M2 kind


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


@pytest.fixture
def forced(request):
    os.environ["LPGEMM_FORCE_CONFIG"] = str(request.param)
    yield request.param
    del os.environ["LPGEMM_FORCE_CONFIG"]


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def e3m2_value(code):
    """Value of a six-bit E3M2 code: (-1)^s * 2^(e-3) * (1 + m/4), or
    2^-2 * (m/4) when e = 0."""
    s, e, m = (code >> 5) & 1, (code >> 2) & 7, code & 3
    mag = (m / 4.0) * 2.0 ** -2 if e == 0 else (1.0 + m / 4.0) * 2.0 ** (e - 3)
    return -mag if s else mag


def unpack_groups(rows6):
    """rows x K bytes of E3M2 operand rows -> rows x K decoded values, slot
    order as stored (32 six-bit fields per 32-byte group, little-endian, the
    last 8 bytes of a group zero)."""
    rows, K = rows6.shape
    g = rows6.reshape(rows, K // 32, 32)
    assert (g[:, :, 24:] == 0).all(), "group padding must be zero"
    bits = np.unpackbits(g[:, :, :24], axis=2, bitorder="little")   # rows x G x 192
    w = np.array([1 << i for i in range(6)], np.int64)
    codes = (bits.reshape(rows, K // 32, 32, 6).astype(np.int64) * w).sum(axis=3)
    table = np.array([e3m2_value(c) for c in range(64)])
    return table[codes].reshape(rows, K)


# within each group of 32 the codes are stored for k = 0, 2, 4, 6, 1, 3, 5, 7, 8, ...
SLOT_K = np.array([8 * (s // 8) + [0, 2, 4, 6, 1, 3, 5, 7][s % 8] for s in range(32)])


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 64), (37, 96), (256, 4096)])
def test_encoding_decodes_to_the_int4_values(rows, K):
    print("[case] e3m2 encode", rows, K, flush=True)
    p = inputs.int4_problem(rows, 1, K, seed=rows + K)
    enc = lp.i4_to_e3m2(_dev(p.a_packed))
    torch.cuda.synchronize()
    vals = unpack_groups(enc.cpu().numpy())
    want = p.a_values.astype(np.float64).reshape(rows, K // 32, 32)[:, :, SLOT_K].reshape(rows, K)
    np.testing.assert_array_equal(vals, want)


def test_encoding_every_nibble():
    # every int4 value at every position of a group
    v = np.tile(np.arange(-8, 8, dtype=np.int8), 2)[None, :]          # 1 x 32
    v = np.concatenate([np.roll(v, s, axis=1) for s in range(32)], axis=0)
    enc = lp.i4_to_e3m2(_dev(inputs.pack_int4(v)))
    torch.cuda.synchronize()
    vals = unpack_groups(enc.cpu().numpy())
    np.testing.assert_array_equal(vals, v.astype(np.float64)[:, SLOT_K])


SHAPES = [(1, 1, 32), (1, 1, 64), (33, 47, 96), (64, 96, 4096), (257, 300, 544), (300, 520, 1056)]


@pytest.mark.parametrize("forced", E3M2_CONFIGS, indirect=True)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_matches_int4_oracle(forced, M, N, K):
    print("[case] e3m2 gemm cfg", forced, M, N, K, flush=True)
    p = inputs.int4_problem(M, N, K, seed=M * 7 + N + K)
    out = lp.gemm_i4_via_e3m2(_dev(p.a_packed), _dev(p.b_packed))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i4(p.a_packed, p.b_packed, K))


@pytest.mark.parametrize("forced", E3M2_CONFIGS, indirect=True)
def test_range_limit(forced):
    # |C| = 64 K at the largest K: 8386560 < 2^24, still exact in fp32
    M, N, K = 40, 72, 131040
    print("[case] e3m2 range cfg", forced, M, N, K, flush=True)
    a = np.full((M, K), -8, np.int8)
    b = np.full((N, K), -8, np.int8)
    b[1::2] = 7
    out = lp.gemm_i4_via_e3m2(_dev(inputs.pack_int4(a)), _dev(inputs.pack_int4(b)))
    torch.cuda.synchronize()
    ref = np.where(np.arange(N)[None, :] % 2 == 1, -56 * K, 64 * K).astype(np.int32)
    np.testing.assert_array_equal(out.cpu().numpy(), np.broadcast_to(ref, (M, N)))


def test_agrees_with_direct_int4_path_at_8192():
    n = 8192
    print("[case] e3m2 8192 sampled", flush=True)
    p = inputs.int4_problem(n, n, n, seed=inputs.seed_for("i4", n))
    a, b = _dev(p.a_packed), _dev(p.b_packed)
    via = lp.gemm_i4_via_e3m2(a, b)
    direct = lp.gemm_i4(a, b)
    torch.cuda.synchronize()
    assert torch.equal(via, direct)
    rows = [0, 1, 255, 256, 4095, 8191]
    np.testing.assert_array_equal(via[rows].cpu().numpy(),
                                  oracle.gemm_i4(p.a_packed, p.b_packed, n, rows=rows))


def test_degenerate_sizes():
    a = torch.empty((0, 16), dtype=torch.uint8, device="cuda")
    b = torch.zeros((5, 16), dtype=torch.uint8, device="cuda")
    assert lp.gemm_i4_via_e3m2(a, b).shape == (0, 5)
    # K = 0: an empty sum
    a0 = torch.empty((3, 0), dtype=torch.uint8, device="cuda")
    b0 = torch.empty((4, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((3, 4), 7, dtype=torch.int32, device="cuda")
    lp.gemm_i4_e3m2(a0, b0, out=out)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_weights_converted_once():
    # the same converted B serves several activations
    K, N = 1024, 200
    p = inputs.int4_problem(8, N, K, seed=5)
    b6 = lp.i4_to_e3m2(_dev(p.b_packed))
    for s in range(3):
        q = inputs.int4_problem(16 + s, 1, K, seed=100 + s)
        out = lp.gemm_i4_e3m2(lp.i4_to_e3m2(_dev(q.a_packed)), b6)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i4(q.a_packed, p.b_packed, K))
