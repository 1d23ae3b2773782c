"""The skinny kernels' pipeline at every count of rounds per wave.

The waves of a skinny workgroup split K; each wave contracts its share in
rounds of R 128-byte blocks, with its A fragments loaded into registers
ahead of use and its B blocks copied into LDS one round ahead.  The code
takes a different shape for whole groups of rounds, for each length of the
remainder (one to four rounds, with no load past the last one) and, for the
eight-wave kernel and the fused W8A8 kernel, for the variant that loads A
one round ahead.  These tests run each configuration at K giving every
wave 1 to 11 rounds, plus a partial last block, and compare all of C with
the oracle bit for bit (dequant: the fp32 bits)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import precision_dense_gemm_02_amd as lp  # noqa: E402
from precision_dense_gemm_02_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

# (configuration, waves, 128-byte blocks per round): K = 128 * waves * R *
# rounds gives every wave exactly `rounds` rounds
SKINNY = [(14, 4, 2), (15, 8, 1)]
ROUNDS = list(range(1, 12))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lp.load_library()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("cfg,waves,r", SKINNY)
@pytest.mark.parametrize("rounds", ROUNDS)
@pytest.mark.parametrize("partial", [False, True])
def test_i8_and_dequant(cfg, waves, r, rounds, partial):
    K = 128 * waves * r * rounds - (96 if partial else 0)
    M, N = 19, 70
    print("[case] skinny rounds", cfg, rounds, K, flush=True)
    p = inputs.int8_problem(M, N, K, seed=inputs.seed_for("i8", 131 * cfg + K), scales=True)
    prev = lp.force_config(cfg)
    try:
        out = lp.gemm_i8(_dev(p.a), _dev(p.b_t), out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
        outd = lp.gemm_i8_dequant(_dev(p.a), _dev(p.b_t), _dev(p.row_scale), _dev(p.col_scale),
                                  out=torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"))
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i8(p.a, p.b_t))
    ref = oracle.gemm_i8_dequant(p.a, p.b_t, p.row_scale, p.col_scale)
    np.testing.assert_array_equal(outd.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("cfg,waves,r", SKINNY)
@pytest.mark.parametrize("rounds", [1, 2, 3, 5, 8])
def test_i4(cfg, waves, r, rounds):
    # packed int4: 64 values per 32-byte step, K a multiple of 32
    K = 2 * 128 * waves * r * rounds
    M, N = 23, 45
    print("[case] skinny rounds i4", cfg, rounds, K, flush=True)
    p = inputs.int4_problem(M, N, K, seed=inputs.seed_for("i4", 131 * cfg + K))
    prev = lp.force_config(cfg)
    try:
        out = lp.gemm_i4(_dev(p.a_packed), _dev(p.b_packed), K,
                         out=torch.full((M, N), -7, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
    finally:
        lp.force_config(prev)
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.gemm_i4(p.a_packed, p.b_packed, K))


@pytest.mark.parametrize("rounds", ROUNDS)
def test_w8a8_fused(rounds):
    # four waves of one 128-byte block per round
    K = 128 * 4 * rounds
    M, N = 9, 50
    print("[case] skinny rounds w8a8 fused", rounds, K, flush=True)
    p = inputs.w8a8_problem(M, N, K, seed=inputs.seed_for("w8a8", 3 * K + 1))
    y = lp.w8a8_linear_fused(_dev(p.x), _dev(p.w), _dev(p.w_scale))
    torch.cuda.synchronize()
    q, s = oracle.quantize_rows_f16(p.x)
    ref = oracle.gemm_i8_dequant(q, p.w, s, p.w_scale)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
