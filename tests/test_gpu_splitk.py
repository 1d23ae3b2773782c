"""The split-K entry points (lpgemm_*_splitk) against the oracle and against
the unsplit entry points.

Integer kinds: the parts are exact int32 sums, so the split result must equal
the oracle and the unsplit call bit for bit.  fp16: the parts are added in a
fixed order, so the split result must be deterministic, within the fp16
bound, and exact on integer-valued operands.  The shapes are chosen so that a
256-CU MI355X splits them 2, 3 and 4 ways, with ragged K (a last stage that
runs past K) and ragged M and N (edge tiles)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

SPLIT_CFG = 60
SLOT = 128 * 128 * 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split counts below assume 256 CUs")


def _say(*what):
    print("[case]", *what, flush=True)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _tiles(M, N):
    return ((M + 127) // 128) * ((N + 127) // 128)


def _tiles64(M, N):
    return ((M + 63) // 64) * ((N + 63) // 64)


def _split_shape(M, N):
    # the library's rule on 256 CUs: M > 64, at most 64 tiles of 128 x 128,
    # and above 128 rows more than 64 tiles of 64 x 64
    return M > 64 and _tiles(M, N) <= 64 and (M <= 128 or _tiles64(M, N) > 64)


def _expected_splits(M, N, row_bytes, kind="i8"):
    # ... and at least 32 K-stages of 256 bytes: then 4 parts, but below 64
    # stages only while the unsplit choice's 128 x 64 tiles fill less than
    # half the CUs (int4, which keeps 64 x 64 tiles, always)
    if not _split_shape(M, N):
        return 1
    nks = (row_bytes + 255) // 256
    if nks < 32:
        return 1
    if nks < 64 and kind != "i4" and 2 * (-(-M // 128)) * (-(-N // 64)) >= 256:
        return 1
    return 4


def _counters_zero(ws, M=None, N=None):
    # the first 4 KiB of every workspace: one counter per tile, zero between calls
    return bool((ws[:4096].view(torch.int32) == 0).all().item())


# int8 (row bytes = K) splits four ways on 256 CUs: 40 tiles of 33
# K-stages, 32 tiles of 64, 48 tiles of 33 (fp16 rows are twice as long;
# int4 rows half as long, so only the second shape splits for int4).  Ragged
# M, N and K (a last stage that runs past K) throughout.
SHAPES = [(600, 1000, 8208), (128, 4096, 16384), (200, 3000, 8208)]


def test_workspace_query_matches_rule():
    for M, N in [(300, 520), (600, 1000), (1000, 1000), (200, 3000), (128, 4096), (64, 4096), (128, 14336),
                 (2048, 2048), (512, 512)]:
        t = _tiles(M, N)
        want = 4096 + t * 4 * SLOT if _split_shape(M, N) else 0
        assert lp.splitk_workspace_bytes(M, N) == want, (M, N)
    assert lp.splitk_workspace_bytes(128, 14336) == 0   # 112 tiles: no split
    assert lp.splitk_workspace_bytes(300, 520) == 0     # 45 tiles of 64 x 64: the unsplit kernel splits K itself
    assert [_expected_splits(M, N, K) for M, N, K in SHAPES] == [4, 4, 4]
    assert [_expected_splits(M, N, K // 2, "i4") for M, N, K in SHAPES] == [1, 4, 1]
    assert _expected_splits(1000, 1000, 8208) == 1   # 128 band tiles at 33 stages: unsplit


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_i8_splitk_exact(M, N, K):
    _say("i8 split-K", M, N, K, "splits", _expected_splits(M, N, K))
    p = inputs.int8_problem(M, N, K, seed=M + N + K)
    a, b = _dev(p.a), _dev(p.b_t)
    ws = lp.splitk_workspace(M, N)
    got = lp.gemm_i8_splitk(a, b, ws)
    again = lp.gemm_i8_splitk(a, b, ws)   # the same workspace, counters reset
    plain = lp.gemm_i8(a, b)
    torch.cuda.synchronize()
    rows = None if M * N * K < 2 ** 31 else [0, 1, 63, 64, 100, M - 1]
    if _expected_splits(M, N, K) > 1:
        assert bool((ws[4096:] != 0).any().item())   # the parts went through the workspace
    ref = oracle.gemm_i8(p.a, p.b_t, rows=rows)
    g = got.cpu().numpy()
    np.testing.assert_array_equal(g if rows is None else g[rows], ref)
    assert torch.equal(got, again) and torch.equal(got, plain)
    assert _counters_zero(ws, M, N)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_i4_splitk_exact(M, N, K):
    K = (K + 31) // 32 * 32
    _say("i4 split-K", M, N, K, "splits", _expected_splits(M, N, K // 2, "i4"))
    q = inputs.int4_problem(M, N, K, seed=M + 2 * N + K)
    a, b = _dev(q.a_packed), _dev(q.b_packed)
    ws = lp.splitk_workspace(M, N)
    got = lp.gemm_i4_splitk(a, b, ws, K)
    plain = lp.gemm_i4(a, b, K)
    torch.cuda.synchronize()
    rows = None if M * N * K < 2 ** 31 else [0, 5, 64, 127]
    ref = oracle.gemm_i4(q.a_packed, q.b_packed, K, rows=rows)
    g = got.cpu().numpy()
    np.testing.assert_array_equal(g if rows is None else g[rows], ref)
    assert torch.equal(got, plain)
    assert _counters_zero(ws, M, N)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_dequant_splitk_exact(M, N, K):
    _say("dequant split-K", M, N, K)
    p = inputs.int8_problem(M, N, K, seed=3 * M + N + K, scales=True)
    a, b = _dev(p.a), _dev(p.b_t)
    rs, cs = _dev(p.row_scale), _dev(p.col_scale)
    ws = lp.splitk_workspace(M, N)
    got = lp.gemm_i8_dequant_splitk(a, b, rs, cs, ws)
    plain = lp.gemm_i8_dequant(a, b, rs, cs)
    torch.cuda.synchronize()
    rows = None if M * N * K < 2 ** 31 else [0, 2, 64, 126, 127]
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
    g = got.cpu().numpy()
    np.testing.assert_array_equal((g if rows is None else g[rows]).view(np.uint32), ref.view(np.uint32))
    assert torch.equal(got.view(torch.int32), plain.view(torch.int32))
    assert _counters_zero(ws, M, N)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_f16_splitk_bound_and_deterministic(M, N, K):
    _say("f16 split-K", M, N, K, "splits", _expected_splits(M, N, 2 * K))
    p = inputs.f16_problem(M, N, K, seed=M + N + 5 * K)
    a, b = _dev(p.a), _dev(p.b_t)
    ws = lp.splitk_workspace(M, N)
    got = lp.gemm_f16_splitk(a, b, ws)
    again = lp.gemm_f16_splitk(a, b, ws)
    torch.cuda.synchronize()
    rows = [0, 1, 64, M // 2, M - 1]
    ref, den = oracle.gemm_f16(p.a, p.b_t, rows=rows)
    err = oracle.f16_rel_error(got.cpu().numpy()[rows], ref, den)
    assert err["max_rel"] <= 1e-3, err
    assert torch.equal(got.view(torch.int32), again.view(torch.int32))
    assert _counters_zero(ws, M, N)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_f16_splitk_integer_valued_exact(M, N, K):
    # integer values in [-8, 7]: every part and every sum of parts is an
    # integer below 2^24, so the split sum must be exact
    _say("f16 split-K integer-valued", M, N, K)
    p = inputs.f16_integer_problem(M, N, K, seed=M + 7 * N + K)
    ws = lp.splitk_workspace(M, N)
    got = lp.gemm_f16_splitk(_dev(p.a), _dev(p.b_t), ws)
    torch.cuda.synchronize()
    rows = [0, 63, 64, M - 1]
    ref = oracle.gemm_i8(p.a.astype(np.int8), p.b_t.astype(np.int8), rows=rows)
    np.testing.assert_array_equal(got.cpu().numpy()[rows], ref.astype(np.float32))


def _check_i8(got, p, rows=None):
    g = got.cpu().numpy()
    np.testing.assert_array_equal(g if rows is None else g[rows], oracle.gemm_i8(p.a, p.b_t, rows=rows))


def test_workspace_reuse_across_shapes_and_small_workspace():
    # one workspace for several shapes in a row, small and large tile counts
    # interleaved (the counters sit in the same 4 KiB for every shape and are
    # zero after each call); a workspace one byte short runs the product
    # unsplit without touching it
    ws = lp.splitk_workspace(1000, 1000)
    for (m, n, k, rows) in [(600, 1000, 8208, [0, 1, 300, 599]), (1000, 1000, 8208, [0, 1, 500, 998, 999]),
                            (300, 520, 256, None), (128, 4096, 16384, [0, 64, 127]),
                            (600, 1000, 8208, [0, 2, 301, 599])]:
        _say("split-K reuse", m, n, k, "splits", _expected_splits(m, n, k))
        p = inputs.int8_problem(m, n, k, seed=m + n + k + 1 + (rows is None))
        got = lp.gemm_i8_splitk(_dev(p.a), _dev(p.b_t), ws)
        torch.cuda.synchronize()
        _check_i8(got, p, rows)
        assert _counters_zero(ws)
    M, N, K = 600, 1000, 8208
    p = inputs.int8_problem(M, N, K, seed=9)
    short = torch.zeros(lp.splitk_workspace_bytes(M, N) - 1, dtype=torch.uint8, device="cuda")
    got = lp.gemm_i8_splitk(_dev(p.a), _dev(p.b_t), short)
    torch.cuda.synchronize()
    _check_i8(got, p, [0, 1, 599])
    assert bool((short == 0).all().item())


def test_edge_cases():
    # K = 0 (zeros), K of one stage (cannot split), M <= 64 (the skinny
    # kernel), M = 65 (one edge row past a full band, split four ways)
    ws = lp.splitk_workspace(128, 4096)
    assert _expected_splits(65, 520, 8192) == 4
    for (M, N, K) in [(300, 520, 0), (300, 520, 256), (64, 520, 8192), (65, 520, 8192), (1, 1, 16)]:
        _say("split-K edge", M, N, K, "splits", _expected_splits(M, N, K))
        p = inputs.int8_problem(M, N, K, seed=M + N + K + 2)
        got = lp.gemm_i8_splitk(_dev(p.a), _dev(p.b_t), ws)
        torch.cuda.synchronize()
        _check_i8(got, p)
    assert _counters_zero(ws)


def test_forced_split_on_a_large_shape():
    # configuration 60 forced: a product the automatic rule would not split
    # (256 tiles) runs two ways when the workspace holds it
    M = N = 2048
    K = 2048
    _say("split-K forced", M, N, K)
    t = _tiles(M, N)
    need = 4096 + t * 2 * SLOT
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    p = inputs.int8_problem(M, N, K, seed=17)
    a, b = _dev(p.a), _dev(p.b_t)
    prev = lp.force_config(SPLIT_CFG)
    try:
        got = lp.gemm_i8_splitk(a, b, ws)
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    rows = [0, 127, 128, 1000, 2047]
    np.testing.assert_array_equal(got.cpu().numpy()[rows], oracle.gemm_i8(p.a, p.b_t, rows=rows))
    assert torch.equal(got, lp.gemm_i8(a, b))
    assert _counters_zero(ws)
    # the parts were written: the workspace holds more than the counters
    assert bool((ws[4096:] != 0).any().item())


@pytest.mark.parametrize("M,N,splits", [(1000, 1200, 3), (1200, 1280, 2)])
@pytest.mark.parametrize("kind", ["i8", "i4", "f16", "dq"])
def test_forced_two_and_three_parts(kind, M, N, splits):
    # configuration 60 forced on 80 and 100 tiles: as many parts as fill the
    # 256 CUs once (3, 2), every kind, ragged K
    K = 2080
    _say("split-K forced", kind, M, N, K, "splits", splits)
    t = _tiles(M, N)
    ws = torch.zeros(4096 + t * splits * SLOT, dtype=torch.uint8, device="cuda")
    rows = [0, 1, 127, 128, M // 2, M - 1]
    prev = lp.force_config(SPLIT_CFG)
    try:
        if kind == "i4":
            q = inputs.int4_problem(M, N, K, seed=M + N + 1)
            a, b = _dev(q.a_packed), _dev(q.b_packed)
            got = lp.gemm_i4_splitk(a, b, ws, K)
            torch.cuda.synchronize()
            ref = oracle.gemm_i4(q.a_packed, q.b_packed, K, rows=rows)
            np.testing.assert_array_equal(got.cpu().numpy()[rows], ref)
        elif kind == "f16":
            p = inputs.f16_integer_problem(M, N, K, seed=M + N + 2)
            got = lp.gemm_f16_splitk(_dev(p.a), _dev(p.b_t), ws)
            torch.cuda.synchronize()
            ref = oracle.gemm_i8(p.a.astype(np.int8), p.b_t.astype(np.int8), rows=rows)
            np.testing.assert_array_equal(got.cpu().numpy()[rows], ref.astype(np.float32))
        else:
            p = inputs.int8_problem(M, N, K, seed=M + N + 3, scales=True)
            a, b = _dev(p.a), _dev(p.b_t)
            if kind == "i8":
                got = lp.gemm_i8_splitk(a, b, ws)
                ref = oracle.gemm_i8(p.a, p.b_t, rows=rows)
            else:
                got = lp.gemm_i8_dequant_splitk(a, b, _dev(p.row_scale), _dev(p.col_scale), ws)
                ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32))
    finally:
        lp.force_config(prev)
    assert _counters_zero(ws)
    assert bool((ws[4096:4096 + t * splits * SLOT] != 0).any().item())


def test_graph_replays():
    # the split kernel under HIP graph capture: every replay equals the eager
    # result (the counters are reset by the kernel itself, no memset node)
    M, N, K = 128, 4096, 16384
    _say("split-K graph", M, N, K, "splits", _expected_splits(M, N, K))
    p = inputs.int8_problem(M, N, K, seed=21, scales=True)
    a, b = _dev(p.a), _dev(p.b_t)
    rs, cs = _dev(p.row_scale), _dev(p.col_scale)
    ws = lp.splitk_workspace(M, N)
    eager = lp.gemm_i8_dequant_splitk(a, b, rs, cs, ws)
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lp.gemm_i8_dequant_splitk(a, b, rs, cs, ws, out=out)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lp.gemm_i8_dequant_splitk(a, b, rs, cs, ws, out=out)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))
    assert _counters_zero(ws)
    rows = [0, 77, 127]
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
    np.testing.assert_array_equal(eager.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32))


def test_two_streams_two_workspaces():
    # split-K products in flight together on two streams, each with its own
    # workspace, repeatedly: no cross-talk between the workspaces' counters
    # or slots, and each stream's results stay exact
    _say("split-K two streams")
    shapes = [(600, 1000, 8208), (200, 3000, 8208)]
    probs = [inputs.int8_problem(M, N, K, seed=40 + i) for i, (M, N, K) in enumerate(shapes)]
    dev = [(_dev(p.a), _dev(p.b_t)) for p in probs]
    wss = [lp.splitk_workspace(M, N) for (M, N, _) in shapes]
    outs = [torch.empty((M, N), dtype=torch.int32, device="cuda") for (M, N, _) in shapes]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(10):
        for s, (a, b), ws, out in zip(streams, dev, wss, outs):
            with torch.cuda.stream(s):
                lp.gemm_i8_splitk(a, b, ws, out=out)
    torch.cuda.synchronize()
    for p, out, ws, (M, N, K) in zip(probs, outs, wss, shapes):
        rows = None if M * N * K < 2 ** 31 else [0, 1, M // 2, M - 1]
        _check_i8(out, p, rows)
        assert _counters_zero(ws)
