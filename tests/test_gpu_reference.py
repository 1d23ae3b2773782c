"""The tuned kernels against the depth-1 reference kernel (configuration 54:
one unswizzled LDS stage, nothing pipelined), bit for bit.

For fp16 this is a stronger check than the error bound: every kernel that
feeds each accumulator the same K-steps in the same order must produce the
same binary32 result as the reference, so a swizzle, stage-ring or epilogue
mistake that still lands within 1e-3 (a fragment read from a neighbouring
k-step, a stage consumed before it landed) shows up as a bit difference.
The split-K skinny kernels (configurations 8 to 17, and 63) sum in another
order and are checked against the oracle's bound instead
(test_gpu_configs.py).  The
reference itself is checked against the oracle like every configuration."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

REF = 54
SPLIT_K = set(range(8, 18)) | {63}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


def _run(cfg, fn, *args):
    prev = lp.force_config(cfg)
    try:
        out = fn(*args)
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    return out


def _configs():
    return [c for c in range(lp.config_count()) if c != REF and c not in SPLIT_K]


@pytest.mark.parametrize("M,N,K", [(300, 520, 200), (1000, 700, 1032), (130, 4100, 264)])
def test_f16_every_tuned_configuration_equals_reference(M, N, K):
    print("[case] f16 reference, every configuration", M, N, K, flush=True)
    p = inputs.f16_problem(M, N, K, seed=M + N + K)
    a, b = torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b_t).cuda()
    ref = _run(REF, lp.gemm_f16, a, b)
    r, d = oracle.gemm_f16(p.a, p.b_t, rows=[0, M - 1])
    assert oracle.f16_rel_error(ref.cpu().numpy()[[0, M - 1]], r, d)["max_rel"] <= 1e-3
    for cfg in _configs():
        got = _run(cfg, lp.gemm_f16, a, b)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"configuration {cfg}"


@pytest.mark.parametrize("n", [2048, 4096, 8192])
def test_f16_benchmarked_kernels_equal_reference(n):
    # the automatic choice at the square sizes the benchmark times
    # (configurations 22, 0 and 47), full C
    print("[case] f16 reference, automatic", n, flush=True)
    p = inputs.f16_problem(n, n, n, inputs.seed_for("f16", n))
    a, b = torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b_t).cuda()
    ref = _run(REF, lp.gemm_f16, a, b)
    got = lp.gemm_f16(a, b)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def test_int_kinds_reference_equals_oracle():
    # the reference kernel on the integer kinds (exact, so equal to the
    # oracle and to every tuned kernel)
    p = inputs.int8_problem(257, 300, 400, seed=5, scales=True)
    q = inputs.int4_problem(257, 300, 416, seed=6)
    a, b = torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b_t).cuda()
    rs, cs = torch.from_numpy(p.row_scale).cuda(), torch.from_numpy(p.col_scale).cuda()
    c8 = _run(REF, lp.gemm_i8, a, b)
    cd = _run(REF, lp.gemm_i8_dequant, a, b, rs, cs)
    c4 = _run(REF, lp.gemm_i4, torch.from_numpy(q.a_packed).cuda(), torch.from_numpy(q.b_packed).cuda(), 416)
    np.testing.assert_array_equal(c8.cpu().numpy(), oracle.gemm_i8(p.a, p.b_t))
    np.testing.assert_array_equal(cd.cpu().numpy().view(np.uint32),
                                  oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale).view(np.uint32))
    np.testing.assert_array_equal(c4.cpu().numpy(), oracle.gemm_i4(q.a_packed, q.b_packed, 416))


@pytest.mark.parametrize("kind", ["i8", "i4", "f16", "dq"])
def test_llm_projection_2048_equals_reference(kind):
    # M = 2048, N = 14336 = 64 x 224, K = 4096: the automatic choice takes
    # 256 x 224 tiles (configuration 61, four waves of 64 x 224, an epilogue
    # whose 56 lanes per row leave 8 idle), full C against the reference
    M, N, K = 2048, 14336, 4096
    print("[case] reference, LLM projection", kind, M, N, K, flush=True)
    if kind == "f16":
        p = inputs.f16_problem(M, N, K, seed=61)
        args = (torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b_t).cuda())
        fn = lp.gemm_f16
    elif kind == "i4":
        p = inputs.int4_problem(M, N, K, seed=61)
        args = (torch.from_numpy(p.a_packed).cuda(), torch.from_numpy(p.b_packed).cuda(), K)
        fn = lp.gemm_i4
    else:
        p = inputs.llm_problem(M)
        args = (torch.from_numpy(p.a).cuda(), torch.from_numpy(p.b_t).cuda())
        fn = lp.gemm_i8
        if kind == "dq":
            args += (torch.from_numpy(p.row_scale).cuda(), torch.from_numpy(p.col_scale).cuda())
            fn = lp.gemm_i8_dequant
    ref = _run(REF, fn, *args)
    for cfg in (61, 62):   # 62: the persistent grid over the same tiles
        forced = _run(cfg, fn, *args)
        assert torch.equal(forced.view(torch.int32), ref.view(torch.int32)), f"configuration {cfg}"
    got = fn(*args)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    if kind == "dq":
        rows = [0, 1, 255, 256, 1023, M - 1]
        want = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
        np.testing.assert_array_equal(got.cpu().numpy()[rows].view(np.uint32), want.view(np.uint32))
