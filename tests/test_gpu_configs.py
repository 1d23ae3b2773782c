"""Every kernel configuration, pinned with lpgemm_force_config, against the
oracle on ragged shapes (M, N off the tile grid, K with a partial stage)."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

def _config_count() -> int:
    # read from the source so that collection needs no library (the CPU
    # boundary test checks that the built library reports the same count)
    import re
    src = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "precision_dense_gemm_02_amd", "csrc", "dispatch.hpp")
    return int(re.search(r"CFG_COUNT = (\d+)", open(src).read()).group(1))


CONFIGS = range(_config_count())


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


@pytest.fixture
def forced(request):
    prev = lp.force_config(request.param)
    yield request.param
    lp.force_config(prev)


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


# the persistent configuration walks several tiles per workgroup: shapes
# with more 256 x 256 tiles than a 256-CU device has workgroups, ragged
# edges, and stage counts of both parities (the LDS stage holding a tile's
# first K-stage then alternates from tile to tile); configuration 62 is the
# same grid over 256 x 224 tiles, whose epilogue stages 16 rows per wave
PERSIST_CFG = 47
PERSIST_CFGS = [PERSIST_CFG, 62]


@pytest.mark.parametrize("cfg", PERSIST_CFGS)
@pytest.mark.parametrize("M,N,K", [(4100, 4100, 16), (4100, 4100, 272), (4100, 4100, 400),
                                   (8192, 4160, 1040), (8192, 8192, 128), (4100, 14336, 272)])
def test_persistent_i8_rounds(M, N, K, cfg):
    print("[case] persistent i8", cfg, M, N, K, flush=True)
    p = inputs.int8_problem(M, N, K, seed=M + N + K)
    prev = lp.force_config(cfg)
    try:
        out = lp.gemm_i8(_dev(p.a), _dev(p.b_t), out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    rows = sorted({r for r in list(range(0, M, 97)) + [M - 1, 255, 256, 4095, 4096] if r < M})
    np.testing.assert_array_equal(out.cpu().numpy()[rows], oracle.gemm_i8(p.a, p.b_t, rows=rows))


@pytest.mark.parametrize("cfg", [PERSIST_CFG, 52])
@pytest.mark.parametrize("K", [32, 544, 800])
def test_persistent_i4_rounds(K, cfg):
    # configuration 52 is the persistent grid for int4 as well (sign-extending
    # expansion); 47 runs configuration 0 for int4
    M, N = 4100, 4100
    print("[case] persistent i4", cfg, M, N, K, flush=True)
    p = inputs.int4_problem(M, N, K, seed=K)
    prev = lp.force_config(cfg)
    try:
        out = lp.gemm_i4(_dev(p.a_packed), _dev(p.b_packed), K)
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    rows = list(range(0, M, 131)) + [M - 1]
    np.testing.assert_array_equal(out.cpu().numpy()[rows], oracle.gemm_i4(p.a_packed, p.b_packed, K, rows=rows))


@pytest.mark.parametrize("cfg", PERSIST_CFGS)
@pytest.mark.parametrize("K", [8, 136, 200])
def test_persistent_f16_rounds(K, cfg):
    M, N = 4100, 4100
    print("[case] persistent f16", cfg, M, N, K, flush=True)
    p = inputs.f16_integer_problem(M, N, K, seed=K)
    prev = lp.force_config(cfg)
    try:
        out = lp.gemm_f16(_dev(p.a), _dev(p.b_t))
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    rows = list(range(0, M, 131)) + [M - 1]
    ref = oracle.gemm_i8(p.a.astype(np.int8), p.b_t.astype(np.int8), rows=rows)
    np.testing.assert_array_equal(out.cpu().numpy()[rows], ref.astype(np.float32))


@pytest.mark.parametrize("cfg", PERSIST_CFGS)
def test_persistent_dequant_llm_2048(cfg):
    # the LLM projection at M = 2048: 448 tiles of 256 x 256, a full round and
    # a partial one; 512 tiles of 256 x 224, two full rounds
    print("[case] persistent dequant llm 2048", cfg, flush=True)
    p = inputs.llm_problem(2048)
    prev = lp.force_config(cfg)
    try:
        out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale))
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    rows = list(range(0, 2048, 61)) + [2047]
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
    np.testing.assert_array_equal(out.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32))
