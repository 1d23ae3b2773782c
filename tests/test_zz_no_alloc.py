"""The allocation-free fp64 emulation entry point (lpgemm_f64_emu_noalloc,
for callers that cannot allocate device memory) against the workspace entry
point lpgemm_f64_emu, through the C ABI: bit for bit, on two calls in a row
whose second is smaller (the scratch keeps the first call's contents), and
against the oracle.  Runs alone in a fresh process as well as after the
other tests."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


def _problem(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 7, (M, 1)))
    B_t = rng.standard_normal((N, K)) * np.exp2(rng.integers(-6, 7, (N, 1)))
    return A, B_t


def _noalloc_c_abi(a, b, out, bits):
    lib = lp.load_library()
    M, K = a.shape
    N = b.shape[0]
    stream = torch.cuda.current_stream().cuda_stream
    return lib.lpgemm_f64_emu_noalloc(M, N, K, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                      ctypes.c_void_p(out.data_ptr()), bits, ctypes.c_void_p(stream))


def test_noalloc_matches_workspace_entry_point_twice():
    # second call smaller than the first, and with fewer moduli
    for M, N, K, bits in [(520, 300, 1024, 53), (70, 90, 160, 20)]:
        print("[case] f64 emu noalloc", M, N, K, bits, flush=True)
        A, B_t = _problem(M, N, K, seed=M + N + K)
        a = torch.from_numpy(A).cuda()
        b = torch.from_numpy(B_t).cuda()
        ref = lp.gemm_f64_emu(a, b, bits)
        out = torch.full((M, N), float("nan"), dtype=torch.float64, device="cuda")
        assert _noalloc_c_abi(a, b, out, bits) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        np.testing.assert_array_equal(got.view(np.uint64), ref.cpu().numpy().view(np.uint64))
        rows = [0, M // 2, M - 1]
        np.testing.assert_array_equal(got[rows].view(np.uint64),
                                      oracle.f64_emu(A, B_t, bits, rows=rows).view(np.uint64))


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    n = 2048    # 53 bits: about 192 MiB of intermediates
    assert lp.f64_emu_workspace_bytes(n, n, n, 53) > 64 * 1024 * 1024
    a = torch.zeros((n, n), dtype=torch.float64, device="cuda")
    out = torch.zeros((n, n), dtype=torch.float64, device="cuda")
    assert _noalloc_c_abi(a, a, out, 53) == lp._binding.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    with pytest.raises(lp.LpgemmError):
        lp.gemm_f64_emu_noalloc(a, a, 53, out=out)
