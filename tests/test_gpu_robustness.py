"""Robustness of the newer entry points on the GPU: captured into a HIP
graph and replayed several times (with eager work and synchronisation in
between), run on two streams at once, and called back to back with changing
shapes.  Every result must equal the eager result, or the oracle, bit for
bit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _bits(t):
    return t.cpu().numpy().view(np.uint8)


def test_graph_replays_of_newer_entry_points():
    print("[case] graph capture of quantiser, W8A8, E3M2, K x N, fp64 emulation", flush=True)
    rng = np.random.default_rng(5)
    w = inputs.w8a8_problem(48, 320, 512, seed=6)
    p4 = inputs.int4_problem(96, 160, 256, 7)
    p8 = inputs.int8_problem(130, 272, 400, 8)
    A = rng.standard_normal((70, 160)); B_t = rng.standard_normal((90, 160))
    x, wq, ws = _dev(w.x), _dev(w.w), _dev(w.w_scale)
    a4, b4 = _dev(p4.a_packed), _dev(p4.b_packed)
    a8, bkn = _dev(p8.a), _dev(p8.b_t.T)
    ad, bd = _dev(A), _dev(B_t)
    # preallocated outputs and intermediates: the graph owns no allocation
    q = torch.empty((48, 512), dtype=torch.int8, device="cuda")
    s = torch.empty((48,), dtype=torch.float32, device="cuda")
    y = torch.empty((48, 320), dtype=torch.float32, device="cuda")
    a6 = torch.empty((96, 256), dtype=torch.uint8, device="cuda")
    b6 = torch.empty((160, 256), dtype=torch.uint8, device="cuda")
    c6 = torch.empty((96, 160), dtype=torch.int32, device="cuda")
    ckn = torch.empty((130, 272), dtype=torch.int32, device="cuda")
    wsp = torch.empty((lp.f64_emu_workspace_bytes(70, 90, 160, 53),), dtype=torch.uint8, device="cuda")
    cd = torch.empty((70, 90), dtype=torch.float64, device="cuda")

    def work():
        lp.quantize_rows_f16(x, q_out=q, scale_out=s)
        lp.gemm_i8_dequant(q, wq, s, ws, out=y)
        lp.i4_to_e3m2(a4, out=a6)
        lp.i4_to_e3m2(b4, out=b6)
        lp.gemm_i4_e3m2(a6, b6, out=c6)
        lp.gemm_i8_kxn(a8, bkn, out=ckn)
        lp.gemm_f64_emu(ad, bd, 53, workspace=wsp, out=cd)

    outs = [q, s, y, a6, b6, c6, ckn, cd]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [_bits(o.clone()) for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for o in outs:
            o.fill_(-1 if o.dtype != torch.uint8 else 255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            np.testing.assert_array_equal(_bits(o), e, err_msg=f"replay {rep}")
        if rep == 1:   # eager work on the same operands between replays
            lp.gemm_i8(a8, _dev(p8.b_t))
            torch.cuda.synchronize()
    # and the eager results are right
    np.testing.assert_array_equal(c6.cpu().numpy(), oracle.gemm_i4(p4.a_packed, p4.b_packed, 256))
    np.testing.assert_array_equal(ckn.cpu().numpy(), oracle.gemm_i8(p8.a, p8.b_t))
    np.testing.assert_array_equal(cd.cpu().numpy().view(np.uint64), oracle.f64_emu(A, B_t, 53).view(np.uint64))


def test_two_streams_at_once():
    print("[case] two streams", flush=True)
    p8 = inputs.int8_problem(1024, 1024, 1024, 31)
    ph = inputs.f16_problem(1024, 1024, 512, 32)
    a8, b8 = _dev(p8.a), _dev(p8.b_t)
    ah, bh = _dev(ph.a), _dev(ph.b_t)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        c8 = [lp.gemm_i8(a8, b8) for _ in range(4)]
    with torch.cuda.stream(s2):
        ch = [lp.gemm_f16(ah, bh) for _ in range(4)]
    torch.cuda.synchronize()
    ref8 = oracle.gemm_i8(p8.a, p8.b_t, rows=range(0, 1024, 97))
    for c in c8:
        np.testing.assert_array_equal(c.cpu().numpy()[::97], ref8)
    for c in ch[1:]:
        assert torch.equal(c, ch[0])


def test_back_to_back_shapes():
    # every call carries its own shape; nothing may leak from one call to the next
    print("[case] back to back shapes", flush=True)
    shapes = [(16, 14336 // 16, 4096), (300, 520, 400), (1, 16, 16), (2048, 256, 512), (33, 47, 96)]
    for it, (M, N, K) in enumerate(shapes * 2):
        p = inputs.int8_problem(M, N, K, seed=1000 + it, scales=True)
        out = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale))
        torch.cuda.synchronize()
        rows = sorted({0, M // 2, M - 1})
        ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale, rows=rows)
        np.testing.assert_array_equal(out.cpu().numpy()[rows].view(np.uint32), ref.view(np.uint32))
