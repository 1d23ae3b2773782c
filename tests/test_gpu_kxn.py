"""GPU parity of the INT8 GEMM with B stored K x N row-major (N contiguous):
the copy of B into LDS by k-rows and the transposed LDS reads
(ds_read_b64_tr_b8) that build the MFMA's B fragments, bit for bit against
the int8 oracle."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

KXN_CONFIGS = (0, 20, 22, 46)   # the configurations that run the K x N layout


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


def _check(M, N, K, seed):
    p = inputs.int8_problem(M, N, K, seed=seed)
    b_kxn = np.ascontiguousarray(p.b_t.T)            # the same B, stored K x N
    out = lp.gemm_i8_kxn(_dev(p.a), _dev(b_kxn))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i8(p.a, p.b_t))


SHAPES = [(1, 16, 16), (33, 48, 96), (64, 96, 4096), (257, 304, 400), (300, 528, 1040), (130, 272, 128)]


@pytest.mark.parametrize("forced", KXN_CONFIGS, indirect=True)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_matches_oracle(forced, M, N, K):
    print("[case] kxn cfg", forced, M, N, K, flush=True)
    _check(M, N, K, seed=M + N + K + forced)


def test_patterned_columns():
    # every column and k-row distinct: a wrong k or column pairing, or a
    # transposed-read lane mix-up, changes the result
    M, N, K = 64, 256, 256
    a = ((np.arange(M)[:, None] * 7 + np.arange(K)[None, :] * 3) % 255 - 127).astype(np.int8)
    b = ((np.arange(K)[:, None] * 5 + np.arange(N)[None, :] * 11) % 253 - 126).astype(np.int8)
    out = lp.gemm_i8_kxn(_dev(a), _dev(b))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i8(a, np.ascontiguousarray(b.T)))


@pytest.mark.parametrize("forced", KXN_CONFIGS, indirect=True)
def test_range_limit(forced):
    M, N, K = 40, 32, 131056
    print("[case] kxn range cfg", forced, flush=True)
    a = np.full((M, K), -128, np.int8)
    b = np.full((K, N), -128, np.int8)
    b[:, 1::2] = 127
    out = lp.gemm_i8_kxn(_dev(a), _dev(b))
    torch.cuda.synchronize()
    ref = np.where(np.arange(N)[None, :] % 2 == 1, -16256 * K, 16384 * K).astype(np.int32)
    np.testing.assert_array_equal(out.cpu().numpy(), np.broadcast_to(ref, (M, N)))


def test_agrees_with_k_contiguous_path_at_8192():
    n = 8192
    print("[case] kxn 8192", flush=True)
    p = inputs.int8_problem(n, n, n, seed=inputs.seed_for("i8", n))
    a, b_t = _dev(p.a), _dev(p.b_t)
    kxn = lp.gemm_i8_kxn(a, b_t.t().contiguous())
    ref = lp.gemm_i8(a, b_t)
    torch.cuda.synchronize()
    assert torch.equal(kxn, ref)
    rows = [0, 255, 256, 8191]
    np.testing.assert_array_equal(kxn[rows].cpu().numpy(), oracle.gemm_i8(p.a, p.b_t, rows=rows))


def test_k_zero_and_empty():
    a = torch.empty((3, 0), dtype=torch.int8, device="cuda")
    b = torch.empty((0, 32), dtype=torch.int8, device="cuda")
    out = torch.full((3, 32), 5, dtype=torch.int32, device="cuda")
    lp.gemm_i8_kxn(a, b, out=out)
    torch.cuda.synchronize()
    assert (out == 0).all()
    assert lp.gemm_i8_kxn(torch.empty((0, 16), dtype=torch.int8, device="cuda"),
                          torch.zeros((16, 32), dtype=torch.int8, device="cuda")).shape == (0, 32)
