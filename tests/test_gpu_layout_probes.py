"""The lane layouts the GEMM kernels assume, pinned on the device one
instruction at a time (tests/hip/layout_probes.hip): the 32 x 32 int8, fp16
and FP6 E3M2 MFMA operand and accumulator layouts, the transposing LDS read
of the K x N path, and where a direct-to-LDS load puts each lane's bytes.
Each probe's output is compared with the plain definition computed here on
the host (a matrix product of small integers, or byte copies), so a wrong
row, column or k-range assumption for any lane fails."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = os.path.join(HERE, "hip", "liblayout_probes.so")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROBES):
        raise RuntimeError(f"{PROBES} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBES)
    for name in ("probe_mfma_i8", "probe_mfma_f16", "probe_mfma_e3m2", "probe_ds_read_tr8", "probe_lds_dma"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_void_p] * 4
        f.restype = ctypes.c_int
    return lib


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _call(lib, name, *tensors):
    stream = torch.cuda.current_stream().cuda_stream
    assert getattr(lib, name)(*[ctypes.c_void_p(t.data_ptr()) for t in tensors], ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mfma_i8_operand_and_accumulator_layout(lib, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-128, 128, size=(32, 32), dtype=np.int8)
    bt = rng.integers(-128, 128, size=(32, 32), dtype=np.int8)
    if seed == 2:   # index-encoding operands: every (row, k) distinct
        a = ((np.arange(32)[:, None] * 33 + np.arange(32)[None, :] * 5) % 251 - 125).astype(np.int8)
        bt = ((np.arange(32)[:, None] * 17 + np.arange(32)[None, :] * 29) % 241 - 120).astype(np.int8)
    c = torch.zeros((32, 32), dtype=torch.int32, device="cuda")
    _call(lib, "probe_mfma_i8", _dev(a), _dev(bt), c)
    ref = a.astype(np.int64) @ bt.astype(np.int64).T
    np.testing.assert_array_equal(c.cpu().numpy(), ref.astype(np.int32))


@pytest.mark.parametrize("seed", [0, 1])
def test_mfma_f16_operand_and_accumulator_layout(lib, seed):
    # small integers: every product and sum is exact in fp32
    rng = np.random.default_rng(10 + seed)
    a = rng.integers(-8, 8, size=(32, 16)).astype(np.float16)
    bt = rng.integers(-8, 8, size=(32, 16)).astype(np.float16)
    c = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    _call(lib, "probe_mfma_f16", _dev(a.view(np.uint16)), _dev(bt.view(np.uint16)), c)
    ref = a.astype(np.float64) @ bt.astype(np.float64).T
    np.testing.assert_array_equal(c.cpu().numpy(), ref.astype(np.float32))


def _e3m2_code(v: int) -> int:
    """FP6 E3M2 code of a small integer, from the format's definition: sign
    bit, three exponent bits with bias 3, two mantissa bits."""
    if v == 0:
        return 0
    m, e = abs(v), 0
    while m >= 2:
        m /= 2
        e += 1
    frac = (m - 1) * 4
    assert frac == int(frac), v
    return (0x20 if v < 0 else 0) | ((e + 3) << 2) | int(frac)


def _e3m2_value(code: int) -> float:
    s = -1.0 if code & 0x20 else 1.0
    e, f = (code >> 2) & 7, code & 3
    return s * (f / 4 * 2.0 ** -2 if e == 0 else (1 + f / 4) * 2.0 ** (e - 3))


def _pack6(codes: np.ndarray) -> np.ndarray:
    """Rows of 64 six-bit codes -> rows of 48 bytes (two 24-byte halves,
    code i of a half in bits 6 i .. 6 i + 5, little-endian)."""
    out = np.zeros((codes.shape[0], 48), np.uint8)
    for r in range(codes.shape[0]):
        for h in range(2):
            bits = 0
            for i in range(32):
                bits |= int(codes[r, 32 * h + i]) << (6 * i)
            out[r, 24 * h:24 * h + 24] = np.frombuffer(bits.to_bytes(24, "little"), np.uint8)
    return out


def test_e3m2_codes_round_trip():
    for v in range(-8, 8):
        assert _e3m2_value(_e3m2_code(v)) == v


def test_mfma_e3m2_operand_and_accumulator_layout(lib):
    rng = np.random.default_rng(20)
    a = rng.integers(-8, 8, size=(32, 64))
    bt = rng.integers(-8, 8, size=(32, 64))
    code = np.vectorize(_e3m2_code)
    c = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    _call(lib, "probe_mfma_e3m2", _dev(_pack6(code(a))), _dev(_pack6(code(bt))), c)
    np.testing.assert_array_equal(c.cpu().numpy(), (a @ bt.T).astype(np.float32))


def test_ds_read_tr8_lane_layout(lib):
    rng = np.random.default_rng(30)
    data = rng.integers(0, 256, size=1024, dtype=np.uint8)
    rows = rng.permutation(128)[:64]           # distinct 8-byte rows of the 1 KiB
    addr = (8 * rows).astype(np.int32)
    out = torch.zeros(64 * 8, dtype=torch.uint8, device="cuda")
    _call(lib, "probe_ds_read_tr8", _dev(data), _dev(addr), out)
    got = out.cpu().numpy().reshape(64, 8)
    want = np.zeros((64, 8), np.uint8)
    for g in range(4):
        for h in range(2):
            for c in range(8):
                for b in range(8):
                    want[16 * g + 8 * h + c, b] = data[addr[16 * g + 2 * b + h] + c]
    np.testing.assert_array_equal(got, want)


def test_direct_to_lds_load_lane_layout(lib):
    rng = np.random.default_rng(40)
    data = rng.integers(0, 256, size=4096, dtype=np.uint8)
    voff = (16 * rng.permutation(256)[:64]).astype(np.uint32)
    voff[5] = 4096            # past the buffer's end: reads as zero
    voff[9] = 0x80000000
    out = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    _call(lib, "probe_lds_dma", _dev(data), _dev(voff), out)
    got = out.cpu().numpy().reshape(64, 16)
    for lane in range(64):
        o = int(voff[lane])
        want = data[o:o + 16] if o + 16 <= 4096 else np.zeros(16, np.uint8)
        np.testing.assert_array_equal(got[lane], want, err_msg=f"lane {lane}")
