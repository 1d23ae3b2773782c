"""The automatic choice for 33 to 128 rows, against the oracle over all of C:
33-64 rows take the 128-row band kernel (128 x 64 tiles, three 256-byte
stages) once its tiles number more than half the CUs and the skinny kernel
over two 32-row bands otherwise (int4: always the skinny kernel); 65-128
rows the band kernel for every kind.  Integer kinds bit for bit, fp16 on
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
