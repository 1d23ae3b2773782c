"""The skinny kernel (M <= 32) with an even share of the columns per
workgroup: where 32-column tiles load some CUs more than others, the
automatic choice gives each workgroup a multiple of 4 columns, so that N
spreads evenly over the workgroups the CUs hold (on 256 CUs: N = 14336, 28
columns in 512 workgroups; 12800 and 13000, 28 with a ragged last one;
28672, 28 in 1024); forced, configuration 63 holds two 32-row B blocks per
workgroup (56 columns at N = 14336).  Workgroup boundaries then fall inside
MFMA blocks, B rows past a workgroup's columns read as zero and their
columns are not stored, so the tests compare all of C against the oracle,
bit for bit (fp16: integer-valued operands, exact in fp32, and random ones
within the bound), with C filled beforehand so that a column left unwritten
shows."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

SHAPES = [(1, 14336), (16, 14336), (32, 14336), (16, 12800), (32, 13000), (16, 4096), (16, 28672), (7, 1000), (16, 100)]
K = 1040   # eight 128-byte K-blocks plus a partial one
K_I4 = 1056   # packed: four 128-byte K-blocks plus a partial one (K a multiple of 32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("M,N", SHAPES)
def test_i8_and_dequant(M, N):
    print("[case] skinny columns i8/dequant", M, N, K, flush=True)
    p = inputs.int8_problem(M, N, K, seed=M * 7 + N, scales=True)
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
    print("[case] skinny columns i4", M, N, K_I4, flush=True)
    p = inputs.int4_problem(M, N, K_I4, seed=M * 5 + N)
    out = lp.gemm_i4(_dev(p.a_packed), _dev(p.b_packed), K_I4,
                     out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i4(p.a_packed, p.b_packed, K_I4))


@pytest.mark.parametrize("M,N", SHAPES)
def test_f16(M, N):
    print("[case] skinny columns f16", M, N, K, flush=True)
    p = inputs.f16_integer_problem(M, N, K, seed=M * 3 + N)
    out = lp.gemm_f16(_dev(p.a), _dev(p.b_t), out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8(p.a.astype(np.int8), p.b_t.astype(np.int8))
    np.testing.assert_array_equal(out.cpu().numpy(), ref.astype(np.float32))
    q = inputs.f16_problem(M, N, K, seed=M * 11 + N)
    out = lp.gemm_f16(_dev(q.a), _dev(q.b_t))
    torch.cuda.synchronize()
    r, d = oracle.gemm_f16(q.a, q.b_t)
    assert oracle.f16_rel_error(out.cpu().numpy(), r, d)["max_rel"] <= 1e-3


@pytest.mark.parametrize("cfg", [14, 63])
def test_forced_widths_equal_automatic(cfg):
    # forced, configurations 14 and 63 take 32 and 64 columns per workgroup;
    # every width gives the same exact sums
    M, N = 16, 14336
    print("[case] skinny columns forced", cfg, M, N, K, flush=True)
    p = inputs.int8_problem(M, N, K, seed=cfg)
    a, b = _dev(p.a), _dev(p.b_t)
    auto = lp.gemm_i8(a, b)
    prev = lp.force_config(cfg)
    try:
        forced = lp.gemm_i8(a, b)
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    assert torch.equal(auto, forced)
    np.testing.assert_array_equal(forced.cpu().numpy(), oracle.gemm_i8(p.a, p.b_t))
