"""Every kernel configuration, forced with LPGEMM_FORCE_CONFIG, against the
oracle on ragged shapes (M, N off the tile grid, K with a partial stage)."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

CONFIGS = range(47)


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


SHAPES = [(1, 1), (300, 520), (530, 260)]


@pytest.mark.parametrize("forced", CONFIGS, indirect=True)
@pytest.mark.parametrize("M,N", SHAPES)
def test_i8(forced, M, N):
    for K in (16, 400):
        print("[case] cfg", forced, "i8", M, N, K, flush=True)
        p = inputs.int8_problem(M, N, K, seed=M + N + K + forced)
        out = lp.gemm_i8(_dev(p.a), _dev(p.b_t))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i8(p.a, p.b_t))


@pytest.mark.parametrize("forced", CONFIGS, indirect=True)
@pytest.mark.parametrize("M,N", SHAPES)
def test_i4(forced, M, N):
    for K in (32, 416, 544):
        print("[case] cfg", forced, "i4", M, N, K, flush=True)
        p = inputs.int4_problem(M, N, K, seed=M + N + K + forced)
        out = lp.gemm_i4(_dev(p.a_packed), _dev(p.b_packed), K)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i4(p.a_packed, p.b_packed, K))


@pytest.mark.parametrize("forced", CONFIGS, indirect=True)
@pytest.mark.parametrize("M,N", SHAPES)
def test_f16(forced, M, N):
    for K in (8, 200):
        print("[case] cfg", forced, "f16", M, N, K, flush=True)
        p = inputs.f16_problem(M, N, K, seed=M + N + K + forced)
        out = lp.gemm_f16(_dev(p.a), _dev(p.b_t))
        torch.cuda.synchronize()
        ref, den = oracle.gemm_f16(p.a, p.b_t)
        assert oracle.f16_rel_error(out.cpu().numpy(), ref, den)["max_rel"] <= 1e-3


@pytest.mark.parametrize("forced", CONFIGS, indirect=True)
def test_dequant(forced):
    M, N, K = 300, 520, 400
    print("[case] cfg", forced, "dequant", M, N, K, flush=True)
    p = inputs.int8_problem(M, N, K, seed=forced, scales=True)
    out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("forced", CONFIGS, indirect=True)
def test_int4_range_limit(forced):
    M, N, K = 40, 72, 131040
    print("[case] cfg", forced, "i4 range", M, N, K, flush=True)
    a = np.full((M, K), -8, np.int8)
    b = np.full((N, K), -8, np.int8)
    b[1::2] = 7
    out = lp.gemm_i4(_dev(inputs.pack_int4(a)), _dev(inputs.pack_int4(b)), K)
    torch.cuda.synchronize()
    ref = np.where(np.arange(N)[None, :] % 2 == 1, -56 * K, 64 * K).astype(np.int32)
    np.testing.assert_array_equal(out.cpu().numpy(), np.broadcast_to(ref, (M, N)))


@pytest.mark.parametrize("forced", CONFIGS, indirect=True)
@pytest.mark.parametrize("M", [1, 16, 32])
def test_skinny_long_k(forced, M):
    # several load rounds per wave of the split-K kernels, with a ragged last
    # K-block and N off the 32-column tile grid
    N = 100
    for K in (4112, 1040):
        print("[case] cfg", forced, "i8 long K", M, N, K, flush=True)
        p = inputs.int8_problem(M, N, K, seed=M + K + forced, scales=True)
        out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale))
        torch.cuda.synchronize()
        ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale)
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        f = inputs.f16_problem(M, N, K, seed=M + K + forced)
        out = lp.gemm_f16(_dev(f.a), _dev(f.b_t))
        torch.cuda.synchronize()
        ref, den = oracle.gemm_f16(f.a, f.b_t)
        assert oracle.f16_rel_error(out.cpu().numpy(), ref, den)["max_rel"] <= 1e-3
