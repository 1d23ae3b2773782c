"""Seeded random shapes through the automatic choice, against the oracle on
sampled rows: every kind on shapes drawn log-uniformly (M from 1 to 4200, N
from 64 to 16000, K a multiple of 32 from 128 to 6016), so that the rules' rarely
taken paths (ragged 224-column tiles, column shares of the skinny kernel,
half-size large tiles with ragged edges, band tiles, persistent grids with
a partial tile) meet shapes no hand-picked test names.  Which configuration
each shape takes on this device is printed and the set is required to be
broad."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


def _shapes(n=40, seed=42):
    # M alternately from 200-4200 and 1-200 (log-uniform), N from 64 to
    # 16000 (every fifth a multiple of 224), K a multiple of 32 from 128 to
    # 6016
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        lo, hi = (np.log(200), np.log(4200)) if i % 2 == 0 else (0.0, np.log(200))
        M = max(1, int(np.exp(rng.uniform(lo, hi))))
        N = int(np.exp(rng.uniform(np.log(64), np.log(16000))))
        if i % 5 == 0:
            N = 224 * max(1, N // 224)
        K = 32 * int(np.exp(rng.uniform(np.log(4), np.log(188))))
        out.append((M, N, K))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _rows(M, rng):
    return sorted({0, M - 1} | set(rng.integers(0, M, size=4).tolist()))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_shape(M, N, K):
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    cfgs = {k: lp.auto_config(k, M, N, K, cu) for k in ("i8", "dq", "i4", "f16")}
    print("[case] random shape", M, N, K, "configurations", cfgs, flush=True)
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    rows = _rows(M, rng)
    p = inputs.int8_problem(M, N, K, seed=M + N + K, scales=True)
    out = lp.gemm_i8(_dev(p.a), _dev(p.b_t), out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy()[rows], oracle.gemm_i8(p.a, p.b_t, rows=rows))
    out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale),
                             out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
    np.testing.assert_array_equal(out.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32))
    q = inputs.int4_problem(M, N, K, seed=M + N + K + 1)
    out = lp.gemm_i4(_dev(q.a_packed), _dev(q.b_packed), K,
                     out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy()[rows], oracle.gemm_i4(q.a_packed, q.b_packed, K, rows=rows))
    f = inputs.f16_integer_problem(M, N, K, seed=M + N + K + 2)
    out = lp.gemm_f16(_dev(f.a), _dev(f.b_t), out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.gemm_i8(f.a.astype(np.int8), f.b_t.astype(np.int8), rows=rows).astype(np.float32)
    np.testing.assert_array_equal(out.cpu().numpy()[rows], ref)


def test_the_shapes_reach_many_configurations():
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    seen = {lp.auto_config(k, M, N, K, cu) for (M, N, K) in SHAPES for k in ("i8", "dq", "i4", "f16")}
    print("[case] configurations reached", sorted(seen), flush=True)
    assert len(seen) >= 8
