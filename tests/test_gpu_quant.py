"""GPU parity of the per-row int8 quantiser and of the W8A8 projection built
from it (quantise, then the dequantising int8 GEMM), bit for bit against the
oracle."""
import json
import os

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


def _quant_check(x16):
    print("[case] quantize", x16.shape, flush=True)
    q, s = lp.quantize_rows_f16(_dev(x16))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_rows_f16(x16)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


# K spans every register-held width (up to 512, 1024, 2048, 4096 and 8192
# halves per row) and the two-pass kernel for longer rows; M is not always a
# multiple of the four rows a workgroup takes
@pytest.mark.parametrize("M,K", [(1, 8), (16, 4096), (128, 4096), (33, 72), (700, 1000), (9, 2048),
                                 (5, 8192), (3, 8200), (2, 16384), (2048, 512)])
@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0])
def test_quantize_matches_oracle(M, K, scale):
    rng = np.random.default_rng(M * 31 + K)
    _quant_check((rng.standard_normal((M, K)) * scale).astype(np.float16))


def test_quantize_special_rows():
    x = np.zeros((6, 64), np.float16)
    x[1] = np.arange(-32, 32)                         # integers, amax 32
    x[2, :8] = [127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]  # ties to even at scale 1
    x[3] = np.float16(2.0 ** -24) * np.arange(64)     # subnormals only
    x[4, 7] = -65504.0                                # largest magnitude
    x[5] = np.float16(-1.0)                           # constant row
    _quant_check(x)


def test_quantize_tie_fixtures():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantize_ties.json")))
    rows = np.array([[int(b, 16) for b in c["row_f16_bits"]] for c in g["cases"]], np.uint16)
    x = np.zeros((rows.shape[0], 8), np.uint16)
    x[:, :2] = rows
    x16 = x.view(np.float16)
    q, _ = lp.quantize_rows_f16(_dev(x16))
    torch.cuda.synchronize()
    for i, c in enumerate(g["cases"]):
        assert q[i, :2].cpu().tolist() == c["expected_q"]
    _quant_check(x16)


def test_quantize_k_zero():
    x = torch.empty((5, 0), dtype=torch.float16, device="cuda")
    q, s = lp.quantize_rows_f16(x)
    torch.cuda.synchronize()
    assert q.shape == (5, 0) and (s == 0).all()


@pytest.mark.parametrize("M", [16, 128])
def test_w8a8_linear_llm(M):
    print("[case] w8a8 llm", M, flush=True)
    rng = np.random.default_rng(M)
    x = rng.standard_normal((M, inputs.LLM_K)).astype(np.float16)
    w = inputs.int8_problem(1, inputs.LLM_N, inputs.LLM_K, seed=inputs.seed_for("llm", M)).b_t
    ws = rng.uniform(0.001, 0.01, inputs.LLM_N).astype(np.float32)
    y = lp.w8a8_linear(_dev(x), _dev(w), _dev(ws))
    torch.cuda.synchronize()
    q, s = oracle.quantize_rows_f16(x)
    ref = oracle.gemm_i8_dequant(q, w, s, ws)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_w8a8_linear_llm_2048_sampled_rows():
    M = 2048
    print("[case] w8a8 llm sampled", M, flush=True)
    rng = np.random.default_rng(M)
    x = (rng.standard_normal((M, inputs.LLM_K)) * rng.uniform(0.01, 10.0, (M, 1))).astype(np.float16)
    w = inputs.int8_problem(1, inputs.LLM_N, inputs.LLM_K, seed=inputs.seed_for("llm", M)).b_t
    ws = rng.uniform(0.001, 0.01, inputs.LLM_N).astype(np.float32)
    y = lp.w8a8_linear(_dev(x), _dev(w), _dev(ws))
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 255, 256, 1000, 1500, 2046, 2047]
    q, s = oracle.quantize_rows_f16(x, rows=rows)
    ref = oracle.gemm_i8_dequant(q, w, s, ws)
    np.testing.assert_array_equal(y[rows].cpu().numpy().view(np.uint32), ref.view(np.uint32))


def _all_scales_rows(K, step=1):
    """One row per positive finite fp16 absmax a (every `step`-th): column 0
    holds a, the other columns fp16 values of magnitude <= a (positive fp16
    bit patterns order like their values), with both signs."""
    a = np.arange(1, 0x7C00, step, dtype=np.int64)[:, None]
    j = np.arange(1, K, dtype=np.int64)[None, :]
    mag = (j * 7919 + a * 104729) % (a + 1)
    bits = np.concatenate([np.broadcast_to(a, (a.shape[0], 1)), mag | ((j & 1) << 15)], axis=1)
    return bits.astype(np.uint16).view(np.float16)


@pytest.mark.parametrize("K,step", [(4096, 1), (16384, 61)])
def test_quantize_every_scale(K, step):
    """Every scale the quantiser can produce, on the register-held kernel
    (K = 4096) and on the two-pass kernel for long rows (sampled scales)."""
    x = _all_scales_rows(K, step)
    _quant_check(x)
    _quant_check(np.ascontiguousarray(x[:500]))    # fewer rows than SIMDs: a workgroup per row
