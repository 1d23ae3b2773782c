"""The C-ABI library without a GPU: it loads, exports what the header declares,
and rejects bad arguments on the host before any HIP call (fake pointer
values are safe here because validation never dereferences them)."""
import ctypes

import pytest

from precision_dense_gemm_02_amd import _binding as b

ENTRY = ("lpgemm_i8", "lpgemm_i4", "lpgemm_f16")
FAKE = 0x10000          # 16-byte aligned, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    return b.load_library()


def test_exports_every_declared_symbol(lib):
    names = b.declared_functions()
    assert set(names) == {"lpgemm_i8", "lpgemm_i4", "lpgemm_f16", "lpgemm_i8_dequant",
                          "lpgemm_quantize_rows_f16", "lpgemm_w8a8_fused", "lpgemm_i4_to_e3m2",
                          "lpgemm_i4_e3m2",
                          "lpgemm_i8_kxn", "lpgemm_f64_emu", "lpgemm_f64_emu_noalloc",
                          "lpgemm_f64_emu_moduli",
                          "lpgemm_f64_emu_workspace",
                          "lpgemm_status_string", "lpgemm_version", "lpgemm_config_count",
                          "lpgemm_force_config", "lpgemm_auto_config", "lpgemm_splitk_workspace", "lpgemm_i8_splitk",
                          "lpgemm_i4_splitk", "lpgemm_f16_splitk", "lpgemm_i8_dequant_splitk"}
    for n in names:
        assert hasattr(lib, n), n


def test_config_count_and_force_hook(lib):
    import re
    src = open(b.HEADER_PATH.replace("include/lpgemm.h",
                                     "precision_dense_gemm_02_amd/csrc/dispatch.hpp")).read()
    assert b.config_count() == int(re.search(r"CFG_COUNT = (\d+)", src).group(1))
    prev = b.force_config(3)
    try:
        assert b.force_config(5) == 3
        assert b.force_config(b.config_count()) == 5      # out of range: automatic
        assert b.force_config(-7) == -1
    finally:
        b.force_config(prev)


def test_version_and_strings(lib):
    assert b.version() == 301
    for code in range(6):
        assert b.status_string(code)
    assert b.status_string(99) == "unknown status"


WS = 0x20000       # 256-byte aligned, never dereferenced
WS_BYTES = 1 << 30


def _call(lib, name, M, N, K, A=FAKE, B=FAKE, C=FAKE, rs=FAKE, cs=FAKE, ws=WS, ws_bytes=WS_BYTES):
    # lpgemm_i4_e3m2 has lpgemm_i4's signature and rules; lpgemm_i8_kxn
    # lpgemm_i8's, plus N % 16 == 0 (the generic cases use N = 4 -> 16); the
    # split-K entry points those of their unsuffixed kind, plus a workspace
    if name == "lpgemm_i8_kxn" and N == 4:
        N = 16
    if name == "lpgemm_i8_dequant":
        return lib.lpgemm_i8_dequant(M, N, K, A, B, rs, cs, C, None)
    if name == "lpgemm_i8_dequant_splitk":
        return lib.lpgemm_i8_dequant_splitk(M, N, K, A, B, rs, cs, C, ws, ws_bytes, None)
    if name.endswith("_splitk"):
        return getattr(lib, name)(M, N, K, A, B, C, ws, ws_bytes, None)
    return getattr(lib, name)(M, N, K, A, B, C, None)


SPLITK = ("lpgemm_i8_splitk", "lpgemm_i4_splitk", "lpgemm_f16_splitk", "lpgemm_i8_dequant_splitk")
ALL = ENTRY + ("lpgemm_i8_dequant", "lpgemm_i4_e3m2", "lpgemm_i8_kxn") + SPLITK
K_OK = {"lpgemm_i8": 64, "lpgemm_i4": 64, "lpgemm_f16": 64, "lpgemm_i8_dequant": 64}


@pytest.mark.parametrize("name", ALL)
def test_negative_sizes(lib, name):
    for M, N, K in ((-1, 4, 64), (4, -1, 64), (4, 4, -16)):
        assert _call(lib, name, M, N, K) == b.LPGEMM_ERROR_INVALID_VALUE
    assert _call(lib, name, 2 ** 31, 4, 64) == b.LPGEMM_ERROR_INVALID_VALUE


@pytest.mark.parametrize("name,bad_k", [
    ("lpgemm_i8", [8, 17, 131072, 131088]),
    ("lpgemm_i8_splitk", [8, 17, 131072, 131088]),
    ("lpgemm_i4_splitk", [16, 48, 131072]),
    ("lpgemm_f16_splitk", [4, 12, 1048584]),
    ("lpgemm_i8_dequant_splitk", [8, 24, 131072]),
    ("lpgemm_i8_dequant", [8, 24, 131072]),
    ("lpgemm_i4", [16, 48, 131072, 131104]),
    ("lpgemm_i4_e3m2", [16, 48, 131072, 131104]),
    ("lpgemm_i8_kxn", [8, 17, 131072, 131088]),
    ("lpgemm_f16", [4, 12, 1048584]),
])
def test_unsupported_k(lib, name, bad_k):
    for K in bad_k:
        assert _call(lib, name, 4, 4, K) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE, K


@pytest.mark.parametrize("name", ALL)
def test_null_pointers(lib, name):
    assert _call(lib, name, 4, 4, 64, A=None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert _call(lib, name, 4, 4, 64, B=None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert _call(lib, name, 4, 4, 64, C=None) == b.LPGEMM_ERROR_INVALID_VALUE
    # K = 0 is an empty sum: A and B may be NULL, C may not
    assert _call(lib, name, 4, 4, 0, C=None) == b.LPGEMM_ERROR_INVALID_VALUE


@pytest.mark.parametrize("name", ["lpgemm_i8_dequant", "lpgemm_i8_dequant_splitk"])
def test_null_scales(lib, name):
    assert _call(lib, name, 4, 4, 64, rs=None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert _call(lib, name, 4, 4, 64, cs=None) == b.LPGEMM_ERROR_INVALID_VALUE


@pytest.mark.parametrize("name", SPLITK)
def test_splitk_workspace_checks(lib, name):
    # after the unsuffixed entry point's checks, before the device
    assert _call(lib, name, 4, 4, 64, ws_bytes=-1) == b.LPGEMM_ERROR_INVALID_VALUE
    assert _call(lib, name, 4, 4, 64, ws=WS + 16) == b.LPGEMM_ERROR_MISALIGNED
    assert _call(lib, name, 4, 4, 64, A=MISALIGNED, ws_bytes=-1) == b.LPGEMM_ERROR_MISALIGNED
    bad_k = {"lpgemm_i4_splitk": 48, "lpgemm_f16_splitk": 12}.get(name, 24)
    assert _call(lib, name, 4, 4, bad_k, ws_bytes=-1) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    # an empty product reads no pointer, the workspace included
    assert _call(lib, name, 0, 4, 64, A=None, B=None, C=None, rs=None, cs=None, ws=WS + 16, ws_bytes=-1) == 0


def test_splitk_workspace_query_bad_sizes(lib):
    assert lib.lpgemm_splitk_workspace(-1, 16) == -1
    assert lib.lpgemm_splitk_workspace(16, -1) == -1
    assert lib.lpgemm_splitk_workspace(2 ** 31, 16) == -1


@pytest.mark.parametrize("name", ALL)
def test_misaligned(lib, name):
    for kw in ("A", "B", "C"):
        assert _call(lib, name, 4, 4, 64, **{kw: MISALIGNED}) == b.LPGEMM_ERROR_MISALIGNED, kw


def test_misaligned_scales(lib):
    assert _call(lib, "lpgemm_i8_dequant", 4, 4, 64, rs=FAKE + 2) == b.LPGEMM_ERROR_MISALIGNED
    assert _call(lib, "lpgemm_i8_dequant", 4, 4, 64, cs=FAKE + 1) == b.LPGEMM_ERROR_MISALIGNED
    # 4-byte alignment is enough for scales
    # (not called with valid pointers here: that would reach the device check)


@pytest.mark.parametrize("name", ALL)
def test_empty_product_is_noop(lib, name):
    # M = 0 or N = 0: success without reading any pointer (all NULL here)
    assert _call(lib, name, 0, 5, 64, A=None, B=None, C=None, rs=None, cs=None) == 0
    assert _call(lib, name, 5, 0, 64, A=None, B=None, C=None, rs=None, cs=None) == 0


def test_error_order(lib):
    # a negative size wins over a bad K and a misaligned pointer
    assert _call(lib, "lpgemm_i8", -1, 4, 8, A=MISALIGNED) == b.LPGEMM_ERROR_INVALID_VALUE
    # a bad K wins over a null or misaligned pointer
    assert _call(lib, "lpgemm_i8", 4, 4, 8, A=None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    # a null pointer wins over misalignment
    assert _call(lib, "lpgemm_i8", 4, 4, 64, A=None, B=MISALIGNED) == b.LPGEMM_ERROR_INVALID_VALUE


def test_python_wrapper_type_checks():
    torch = pytest.importorskip("torch")
    a = torch.zeros((4, 64), dtype=torch.int8)
    with pytest.raises(TypeError):
        b.gemm_i8(a.float(), a)
    with pytest.raises(ValueError):                 # CPU tensors are refused
        b.gemm_i8(a, a)
    with pytest.raises(TypeError):
        b.gemm_f16(a, a)
    with pytest.raises(TypeError):
        b.gemm_i4(a, a)
    with pytest.raises(TypeError):
        b.gemm_i8([1], a)


def test_lpgemm_error_carries_status():
    e = b.LpgemmError(b.LPGEMM_ERROR_MISALIGNED, "lpgemm_i8")
    assert e.status == 2 and "aligned" in str(e)


def test_signature_types(lib):
    assert lib.lpgemm_i8.argtypes[0] is ctypes.c_int64
    assert lib.lpgemm_i8_dequant.restype is ctypes.c_int


def test_quantize_validation(lib):
    q = lib.lpgemm_quantize_rows_f16
    assert q(-1, 64, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert q(4, -8, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert q(4, 12, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert q(4, b.MAX_K_QUANT + 8, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert q(0, 64, None, None, None, None) == b.LPGEMM_SUCCESS          # empty: no-op
    assert q(4, 64, FAKE, FAKE, None, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert q(4, 64, None, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert q(4, 64, FAKE, None, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert q(4, 0, None, None, None, None) == b.LPGEMM_ERROR_INVALID_VALUE   # scale still needed
    assert q(4, 64, MISALIGNED, FAKE, FAKE, None) == b.LPGEMM_ERROR_MISALIGNED
    assert q(4, 64, FAKE, MISALIGNED, FAKE, None) == b.LPGEMM_ERROR_MISALIGNED
    assert q(4, 64, FAKE, FAKE, FAKE + 2, None) == b.LPGEMM_ERROR_MISALIGNED


def test_w8a8_fused_validation(lib):
    f = lib.lpgemm_w8a8_fused
    assert f(-1, 64, 64, FAKE, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, -1, 64, FAKE, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 64, 24, FAKE, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE   # K % 16
    assert f(4, 64, 131072, FAKE, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert f(33, 64, 64, FAKE, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE   # M > 32
    assert f(0, 64, 64, None, None, None, None, None) == b.LPGEMM_SUCCESS       # empty: no-op
    assert f(4, 0, 64, None, None, None, None, None) == b.LPGEMM_SUCCESS
    assert f(4, 64, 64, None, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 64, 64, FAKE, None, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 64, 64, FAKE, FAKE, None, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 64, 64, FAKE, FAKE, FAKE, None, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 64, 64, MISALIGNED, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_MISALIGNED
    assert f(4, 64, 64, FAKE, MISALIGNED, FAKE, FAKE, None) == b.LPGEMM_ERROR_MISALIGNED
    assert f(4, 64, 64, FAKE, FAKE, FAKE + 2, FAKE, None) == b.LPGEMM_ERROR_MISALIGNED
    assert f(4, 64, 64, FAKE, FAKE, FAKE, MISALIGNED, None) == b.LPGEMM_ERROR_MISALIGNED


def test_i4_to_e3m2_validation(lib):
    f = lib.lpgemm_i4_to_e3m2
    assert f(-1, 64, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, -32, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 48, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert f(4, 131104, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert f(0, 64, None, None, None) == b.LPGEMM_SUCCESS       # empty: no-op
    assert f(4, 0, None, None, None) == b.LPGEMM_SUCCESS
    assert f(4, 64, None, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 64, FAKE, None, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 64, MISALIGNED, FAKE, None) == b.LPGEMM_ERROR_MISALIGNED
    assert f(4, 64, FAKE, MISALIGNED, None) == b.LPGEMM_ERROR_MISALIGNED


def test_kxn_shape_rules(lib):
    f = lib.lpgemm_i8_kxn
    # N must be a multiple of 16 (16-byte aligned k-rows) and K * N < 2^31
    assert f(4, 40, 64, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert f(4, 32768, 65536, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    # a shape error ranks before pointer errors, after negative sizes
    assert f(4, 40, 64, None, None, None, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert f(-4, 40, 64, FAKE, FAKE, FAKE, None) == b.LPGEMM_ERROR_INVALID_VALUE
    # M = 0 or N = 0 is still a no-op
    assert f(0, 40, 64, None, None, None, None) == b.LPGEMM_SUCCESS
    assert f(4, 0, 64, None, None, None, None) == b.LPGEMM_SUCCESS


MODULI = [256, 255, 253, 251, 247, 241, 239, 233, 229, 227, 223, 217, 211, 199, 197, 193, 191, 181,
          179, 173]


def test_f64_emu_moduli_and_workspace(lib):
    import math
    assert all(math.gcd(a, b) == 1 for i, a in enumerate(MODULI) for b in MODULI[i + 1:])
    for K in (0, 16, 1024, 4096, 131056):
        for bits in (1, 8, 24, 40, 53):
            s = lib.lpgemm_f64_emu_moduli(K, bits)
            bound = 2 * max(K, 1) * 2 ** (2 * bits)
            assert math.prod(MODULI[:s]) > bound, (K, bits, s)
            assert s == 1 or math.prod(MODULI[:s - 1]) <= bound, (K, bits, s)
    assert lib.lpgemm_f64_emu_moduli(4096, 53) == 16
    assert lib.lpgemm_f64_emu_moduli(16, 0) == -1
    assert lib.lpgemm_f64_emu_moduli(16, 54) == -1
    # eA, eB, residues, the reduced products (one byte each) padded to 256 bytes
    M, N, K, bits = 33, 47, 64, 24
    s = lib.lpgemm_f64_emu_moduli(K, bits)
    pad = lambda x: (x + 255) // 256 * 256
    want = pad(4 * M) + pad(4 * N) + pad(s * M * K) + pad(s * N * K) + s * pad(M * N)
    assert lib.lpgemm_f64_emu_workspace(M, N, K, bits) == want
    assert lib.lpgemm_f64_emu_workspace(-1, N, K, bits) == -1


def test_f64_emu_validation(lib):
    f = lib.lpgemm_f64_emu
    WS = 0x20000       # 256-byte aligned, never dereferenced
    big = 1 << 40
    assert f(-1, 4, 64, FAKE, FAKE, FAKE, 53, WS, big, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 64, FAKE, FAKE, FAKE, 0, WS, big, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 64, FAKE, FAKE, FAKE, 54, WS, big, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 24, FAKE, FAKE, FAKE, 53, WS, big, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert f(0, 4, 64, None, None, None, 53, None, 0, None) == b.LPGEMM_SUCCESS   # empty
    assert f(4, 4, 64, FAKE, FAKE, None, 53, WS, big, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 64, FAKE, FAKE, FAKE, 53, None, big, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 64, FAKE, FAKE, FAKE, 53, WS, 100, None) == b.LPGEMM_ERROR_INVALID_VALUE  # too small
    assert f(4, 4, 64, MISALIGNED, FAKE, FAKE, 53, WS, big, None) == b.LPGEMM_ERROR_MISALIGNED
    assert f(4, 4, 64, FAKE, FAKE, FAKE, 53, WS + 16, big, None) == b.LPGEMM_ERROR_MISALIGNED


def test_f64_emu_noalloc_validation(lib):
    # the workspace entry point's checks, then the fixed scratch's limit,
    # all on the host before any HIP call
    f = lib.lpgemm_f64_emu_noalloc
    assert f(-1, 4, 64, FAKE, FAKE, FAKE, 53, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 64, FAKE, FAKE, FAKE, 0, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 24, FAKE, FAKE, FAKE, 53, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert f(0, 4, 64, None, None, None, 53, None) == b.LPGEMM_SUCCESS   # empty
    assert f(4, 4, 64, FAKE, FAKE, None, 53, None) == b.LPGEMM_ERROR_INVALID_VALUE
    assert f(4, 4, 64, MISALIGNED, FAKE, FAKE, 53, None) == b.LPGEMM_ERROR_MISALIGNED
    limit = 64 * 1024 * 1024
    # the largest square size whose workspace fits, and the next multiple of 16
    n = 16
    while lib.lpgemm_f64_emu_workspace(n + 16, n + 16, n + 16, 53) <= limit:
        n += 16
    assert lib.lpgemm_f64_emu_workspace(n, n, n, 53) <= limit
    assert f(n + 16, n + 16, n + 16, FAKE, FAKE, FAKE, 53, None) == b.LPGEMM_ERROR_UNSUPPORTED_SHAPE
    assert n >= 1024


def test_layout_probe_library_exports():
    # the device probes of tests/test_gpu_layout_probes.py (test
    # infrastructure, built by the same build step), loadable without a GPU
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "liblayout_probes.so")
    probes = ctypes.CDLL(path)
    for name in ("probe_mfma_i8", "probe_mfma_f16", "probe_mfma_e3m2", "probe_ds_read_tr8", "probe_lds_dma"):
        assert hasattr(probes, name), name
