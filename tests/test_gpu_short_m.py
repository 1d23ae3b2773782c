"""The automatic choice for 33 to 128 rows, against the oracle over all of C:
33-64 rows take the 128-row band kernel (128 x 64 tiles, three 256-byte
stages) once its tiles number more than half the CUs and the skinny kernel
over two 32-row bands otherwise (int4: always the skinny kernel); 65-128
rows the band kernel for every kind, and so do small grids above 128 rows;
half-size large tiles between half a round and one (below).  Integer kinds bit for bit, fp16 on
integer-valued operands (exact in fp32) and on random ones within the
bound; C is filled beforehand so that an unwritten element shows."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

SHAPES = [(33, 14336), (64, 14336), (48, 8200), (64, 4096), (96, 14336), (128, 4100)]
K = 1040
K_I4 = 1056


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("M,N", SHAPES)
def test_i8_and_dequant(M, N):
    print("[case] short M i8/dequant", M, N, K, flush=True)
    p = inputs.int8_problem(M, N, K, seed=M * 31 + N, scales=True)
    out = lp.gemm_i8(_dev(p.a), _dev(p.b_t), out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i8(p.a, p.b_t))
    out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale),
                             out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("M,N", SHAPES)
def test_i4(M, N):
    print("[case] short M i4", M, N, K_I4, flush=True)
    p = inputs.int4_problem(M, N, K_I4, seed=M * 37 + N)
    out = lp.gemm_i4(_dev(p.a_packed), _dev(p.b_packed), K_I4,
                     out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i4(p.a_packed, p.b_packed, K_I4))


@pytest.mark.parametrize("M,N", SHAPES)
def test_f16(M, N):
    print("[case] short M f16", M, N, K, flush=True)
    q = inputs.f16_integer_problem(M, N, K, seed=M * 41 + N)
    out = lp.gemm_f16(_dev(q.a), _dev(q.b_t), out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8(q.a.astype(np.int8), q.b_t.astype(np.int8))
    np.testing.assert_array_equal(out.cpu().numpy(), ref.astype(np.float32))
    r = inputs.f16_problem(M, N, K, seed=M * 43 + N)
    out = lp.gemm_f16(_dev(r.a), _dev(r.b_t))
    torch.cuda.synchronize()
    ref, den = oracle.gemm_f16(r.a, r.b_t)
    assert oracle.f16_rel_error(out.cpu().numpy(), ref, den)["max_rel"] <= 1e-3


# Above 128 rows, grids of 128 x 64 tiles between a quarter of a round and
# one round at K >= 2048 take the band kernel too (on 256 CUs: 768 x 768,
# 72 tiles; 300 x 4100, 195 tiles, ragged on both sides; 1024 x 1024 x
# 8192, 128 tiles, compared on sampled rows)
@pytest.mark.parametrize("M,N,K2", [(768, 768, 4096), (300, 4100, 2064), (1024, 1024, 8192)])
def test_band_tiles_small_grids(M, N, K2):
    print("[case] band tiles, small grid", M, N, K2, flush=True)
    rows = None if M * N * K2 < 4e9 else sorted({0, 1, 127, 128, 511, 512, M - 1} | set(range(3, M, 97)))
    p = inputs.int8_problem(M, N, K2, seed=M + N + K2, scales=True)
    out = lp.gemm_i8(_dev(p.a), _dev(p.b_t), out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got if rows is None else got[rows], oracle.gemm_i8(p.a, p.b_t, rows=rows))
    out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale),
                             out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
    np.testing.assert_array_equal((got if rows is None else got[rows]).view(np.uint32), ref.view(np.uint32))
    q = inputs.f16_integer_problem(M, N, K2, seed=M + N + K2 + 1)
    out = lp.gemm_f16(_dev(q.a), _dev(q.b_t), out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.gemm_i8(q.a.astype(np.int8), q.b_t.astype(np.int8), rows=rows).astype(np.float32)
    np.testing.assert_array_equal(got if rows is None else got[rows], ref)


# int4 small grids from K = 4096 on take 32 x 32 tiles whose eight waves
# split K (768 x 768 x 8192; 1000 x 1000 x 4096, ragged), sampled rows
@pytest.mark.parametrize("M,N,K2", [(768, 768, 8192), (1000, 1000, 4096)])
def test_i4_small_grids_long_k(M, N, K2):
    print("[case] int4 small grid, long K", M, N, K2, flush=True)
    rows = sorted({0, 1, 31, 32, 500, M - 1} | set(range(5, M, 89)))
    p = inputs.int4_problem(M, N, K2, seed=M + N + K2)
    out = lp.gemm_i4(_dev(p.a_packed), _dev(p.b_packed), K2,
                     out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy()[rows], oracle.gemm_i4(p.a_packed, p.b_packed, K2, rows=rows))


# Between half a round and one round of 128 x 256 tiles (int4: 256 x 128)
# at K >= 2048: the half-size large tiles (on 256 CUs: 2048 x 4096, 256
# tiles; 1500 x 4100, 192, ragged on both sides), sampled rows
@pytest.mark.parametrize("M,N,K2", [(2048, 4096, 4096), (1500, 4100, 2064)])
def test_half_size_large_tiles(M, N, K2):
    print("[case] half-size large tiles", M, N, K2, flush=True)
    rows = sorted({0, 1, 127, 128, 255, 256, M - 1} | set(range(7, M, 113)))
    p = inputs.int8_problem(M, N, K2, seed=M + N + K2, scales=True)
    out = lp.gemm_i8(_dev(p.a), _dev(p.b_t), out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy()[rows], oracle.gemm_i8(p.a, p.b_t, rows=rows))
    out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale),
                             out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
    np.testing.assert_array_equal(out.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32))
    q = inputs.f16_integer_problem(M, N, K2, seed=M + N + K2 + 1)
    out = lp.gemm_f16(_dev(q.a), _dev(q.b_t), out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8(q.a.astype(np.int8), q.b_t.astype(np.int8), rows=rows).astype(np.float32)
    np.testing.assert_array_equal(out.cpu().numpy()[rows], ref)
    K4 = (K2 + 31) // 32 * 32
    r = inputs.int4_problem(M, N, K4, seed=M + N + K4 + 2)
    out = lp.gemm_i4(_dev(r.a_packed), _dev(r.b_packed), K4,
                     out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy()[rows], oracle.gemm_i4(r.a_packed, r.b_packed, K4, rows=rows))
