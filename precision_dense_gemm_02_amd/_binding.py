"""ctypes binding of liblpgemm.so, the C ABI declared in include/lpgemm.h.

Argument marshalling only: every function checks the torch tensors it is
given (dtype, shape, contiguity, device), allocates the output with torch when
none is passed, and calls the library entry point of the same name on the
current torch stream.  All arithmetic runs in the library's HIP kernels.  If
the library has not been built the first call raises -- there is no other
implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblpgemm.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "lpgemm.h")

LPGEMM_SUCCESS = 0
LPGEMM_ERROR_INVALID_VALUE = 1
LPGEMM_ERROR_MISALIGNED = 2
LPGEMM_ERROR_UNSUPPORTED_SHAPE = 3
LPGEMM_ERROR_ARCH = 4
LPGEMM_ERROR_LAUNCH = 5

MAX_K_INT = 131071
MAX_K_F16 = 1048576
MAX_K_QUANT = 1048576


class LpgemmError(RuntimeError):
    """A non-success status from the library."""

    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = status_string(status)
        super().__init__(f"{what}: {msg} (status {status})" if what else f"{msg} (status {status})")


_lib = None
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def load_library():
    """Load liblpgemm.so (once) and declare the entry points' signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m precision_dense_gemm_02_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name in ("lpgemm_i8", "lpgemm_i4", "lpgemm_f16"):
            f = getattr(lib, name)
            f.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p]
            f.restype = ctypes.c_int
        lib.lpgemm_i8_dequant.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p]
        lib.lpgemm_i8_dequant.restype = ctypes.c_int
        lib.lpgemm_quantize_rows_f16.argtypes = [_i64, _i64, _p, _p, _p, _p]
        lib.lpgemm_quantize_rows_f16.restype = ctypes.c_int
        lib.lpgemm_w8a8_fused.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p]
        lib.lpgemm_w8a8_fused.restype = ctypes.c_int
        lib.lpgemm_f64_emu_moduli.argtypes = [_i64, ctypes.c_int]
        lib.lpgemm_f64_emu_moduli.restype = ctypes.c_int
        lib.lpgemm_f64_emu_workspace.argtypes = [_i64, _i64, _i64, ctypes.c_int]
        lib.lpgemm_f64_emu_workspace.restype = _i64
        lib.lpgemm_f64_emu.argtypes = [_i64, _i64, _i64, _p, _p, _p, ctypes.c_int, _p, _i64, _p]
        lib.lpgemm_f64_emu.restype = ctypes.c_int
        lib.lpgemm_f64_emu_noalloc.argtypes = [_i64, _i64, _i64, _p, _p, _p, ctypes.c_int, _p]
        lib.lpgemm_f64_emu_noalloc.restype = ctypes.c_int
        lib.lpgemm_i8_kxn.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p]
        lib.lpgemm_i8_kxn.restype = ctypes.c_int
        lib.lpgemm_i4_to_e3m2.argtypes = [_i64, _i64, _p, _p, _p]
        lib.lpgemm_i4_to_e3m2.restype = ctypes.c_int
        lib.lpgemm_i4_e3m2.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p]
        lib.lpgemm_i4_e3m2.restype = ctypes.c_int
        lib.lpgemm_status_string.argtypes = [ctypes.c_int]
        lib.lpgemm_status_string.restype = ctypes.c_char_p
        lib.lpgemm_version.argtypes = []
        lib.lpgemm_version.restype = ctypes.c_int
        for name in ("lpgemm_i8_splitk", "lpgemm_i4_splitk", "lpgemm_f16_splitk"):
            f = getattr(lib, name)
            f.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _i64, _p]
            f.restype = ctypes.c_int
        lib.lpgemm_i8_dequant_splitk.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _i64, _p]
        lib.lpgemm_i8_dequant_splitk.restype = ctypes.c_int
        lib.lpgemm_splitk_workspace.argtypes = [_i64, _i64]
        lib.lpgemm_splitk_workspace.restype = _i64
        lib.lpgemm_config_count.argtypes = []
        lib.lpgemm_config_count.restype = ctypes.c_int
        lib.lpgemm_force_config.argtypes = [ctypes.c_int]
        lib.lpgemm_force_config.restype = ctypes.c_int
        lib.lpgemm_auto_config.argtypes = [ctypes.c_int, _i64, _i64, _i64, ctypes.c_int]
        lib.lpgemm_auto_config.restype = ctypes.c_int
        _lib = lib
    return _lib


def declared_functions() -> list:
    """Names of the functions include/lpgemm.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lpgemm_\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    try:
        return load_library().lpgemm_status_string(int(status)).decode()
    except RuntimeError:
        return f"status {status}"


def version() -> int:
    return int(load_library().lpgemm_version())


def config_count() -> int:
    """Number of kernel configurations the GEMM entry points know."""
    return int(load_library().lpgemm_config_count())


def force_config(config: int) -> int:
    """Pin kernel configuration `config` for later GEMM calls in this process
    (-1: automatic choice per shape); returns the previous setting."""
    return int(load_library().lpgemm_force_config(int(config)))


AUTO_KINDS = {"i8": 0, "i4": 1, "f16": 2, "dq": 3}


def auto_config(kind: str, M: int, N: int, K: int, cu_count: int) -> int:
    """The configuration the automatic choice takes for an M x N x K product
    of `kind` ("i8", "i4", "f16" or "dq") on `cu_count` compute units (-1:
    nothing is launched or the arguments are out of range)."""
    return int(load_library().lpgemm_auto_config(AUTO_KINDS[kind], int(M), int(N), int(K), int(cu_count)))


def _check(status: int, what: str) -> None:
    if status != LPGEMM_SUCCESS:
        raise LpgemmError(status, what)


def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _operand(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _output(out, shape, dtype, device):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if out.dtype != dtype or tuple(out.shape) != tuple(shape) or out.device != device \
            or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {dtype} tensor of shape {shape} on {device}")
    return out


def _same_device(*ts):
    d = ts[0].device
    for t in ts[1:]:
        if t.device != d:
            raise ValueError("all tensors must be on the same device")
    return d


def gemm_i8(a, b_t, out=None):
    """int32 C = A . B; a: M x K int8, b_t: N x K int8 (B stored K-contiguous)."""
    torch = _torch()
    _operand(a, torch.int8, "a")
    _operand(b_t, torch.int8, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    dev = _same_device(a, b_t)
    M, K = a.shape
    N = b_t.shape[0]
    out = _output(out, (M, N), torch.int32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i8(M, N, K, a.data_ptr(), b_t.data_ptr(), out.data_ptr(),
                                        _stream_handle(dev)), "lpgemm_i8")
    return out


def gemm_i8_kxn(a, b_kxn, out=None):
    """int32 C = A . B with B stored K x N row-major (N contiguous); a: M x K
    int8, b_kxn: K x N int8."""
    torch = _torch()
    _operand(a, torch.int8, "a")
    _operand(b_kxn, torch.int8, "b_kxn")
    if a.shape[1] != b_kxn.shape[0]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_kxn {tuple(b_kxn.shape)}")
    dev = _same_device(a, b_kxn)
    M, K = a.shape
    N = b_kxn.shape[1]
    out = _output(out, (M, N), torch.int32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i8_kxn(M, N, K, a.data_ptr(), b_kxn.data_ptr(), out.data_ptr(),
                                            _stream_handle(dev)), "lpgemm_i8_kxn")
    return out


def gemm_i4(a_packed, b_packed, K: Optional[int] = None, out=None):
    """int32 C = A . B over signed int4 packed two per byte along k (low nibble
    = even k); a_packed: M x K/2 uint8, b_packed: N x K/2 uint8."""
    torch = _torch()
    _operand(a_packed, torch.uint8, "a_packed")
    _operand(b_packed, torch.uint8, "b_packed")
    if a_packed.shape[1] != b_packed.shape[1]:
        raise ValueError("packed K mismatch")
    if K is None:
        K = 2 * a_packed.shape[1]
    if 2 * a_packed.shape[1] != K:
        raise ValueError(f"K={K} does not match packed width {a_packed.shape[1]}")
    dev = _same_device(a_packed, b_packed)
    M = a_packed.shape[0]
    N = b_packed.shape[0]
    out = _output(out, (M, N), torch.int32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i4(M, N, K, a_packed.data_ptr(), b_packed.data_ptr(),
                                        out.data_ptr(), _stream_handle(dev)), "lpgemm_i4")
    return out


def gemm_f16(a, b_t, out=None):
    """fp32 C = A . B; a: M x K fp16, b_t: N x K fp16 (B stored K-contiguous)."""
    torch = _torch()
    _operand(a, torch.float16, "a")
    _operand(b_t, torch.float16, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    dev = _same_device(a, b_t)
    M, K = a.shape
    N = b_t.shape[0]
    out = _output(out, (M, N), torch.float32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_f16(M, N, K, a.data_ptr(), b_t.data_ptr(), out.data_ptr(),
                                         _stream_handle(dev)), "lpgemm_f16")
    return out


def gemm_i8_dequant(a, b_t, row_scale, col_scale, out=None):
    """fp32 C = ((float)(A . B) * row_scale[i]) * col_scale[j]."""
    torch = _torch()
    _operand(a, torch.int8, "a")
    _operand(b_t, torch.int8, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    M, K = a.shape
    N = b_t.shape[0]
    for t, n, name in ((row_scale, M, "row_scale"), (col_scale, N, "col_scale")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 1 \
                or t.shape[0] != n or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 GPU vector of length {n}")
    dev = _same_device(a, b_t, row_scale, col_scale)
    out = _output(out, (M, N), torch.float32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i8_dequant(M, N, K, a.data_ptr(), b_t.data_ptr(),
                                                row_scale.data_ptr(), col_scale.data_ptr(),
                                                out.data_ptr(), _stream_handle(dev)),
               "lpgemm_i8_dequant")
    return out


def splitk_workspace_bytes(M: int, N: int) -> int:
    """Workspace bytes the split-K entry points use for an M x N product on
    the current device (0: the product runs unsplit)."""
    n = int(load_library().lpgemm_splitk_workspace(M, N))
    if n < 0:
        raise ValueError(f"lpgemm_splitk_workspace({M}, {N}) failed")
    return n


def splitk_workspace(M: int, N: int, device=None):
    """A zeroed uint8 GPU tensor for the split-K entry points on an M x N
    product (at least 256 bytes).  Zeroed once here; every call leaves it
    reusable, so keep it for later calls of the same or smaller size."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        n = splitk_workspace_bytes(M, N)
    return torch.zeros((max(n, 256),), dtype=torch.uint8, device=dev)


def _workspace(ws, dev):
    torch = _torch()
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_cuda \
            or not ws.is_contiguous() or ws.device != dev:
        raise ValueError("workspace must be a contiguous uint8 tensor on the operands' GPU")
    return ws.data_ptr(), ws.numel()


def gemm_i8_splitk(a, b_t, workspace, out=None):
    """gemm_i8 with K split over workgroups for products with few 128 x 128
    tiles; `workspace` from splitk_workspace (zeroed once, reusable)."""
    torch = _torch()
    _operand(a, torch.int8, "a")
    _operand(b_t, torch.int8, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    dev = _same_device(a, b_t)
    M, K = a.shape
    N = b_t.shape[0]
    wp, wn = _workspace(workspace, dev)
    out = _output(out, (M, N), torch.int32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i8_splitk(M, N, K, a.data_ptr(), b_t.data_ptr(), out.data_ptr(), wp, wn,
                                               _stream_handle(dev)), "lpgemm_i8_splitk")
    return out


def gemm_i4_splitk(a_packed, b_packed, workspace, K: Optional[int] = None, out=None):
    """gemm_i4 with K split over workgroups (see gemm_i8_splitk)."""
    torch = _torch()
    _operand(a_packed, torch.uint8, "a_packed")
    _operand(b_packed, torch.uint8, "b_packed")
    if a_packed.shape[1] != b_packed.shape[1]:
        raise ValueError("packed K mismatch")
    if K is None:
        K = 2 * a_packed.shape[1]
    if 2 * a_packed.shape[1] != K:
        raise ValueError(f"K={K} does not match packed width {a_packed.shape[1]}")
    dev = _same_device(a_packed, b_packed)
    M = a_packed.shape[0]
    N = b_packed.shape[0]
    wp, wn = _workspace(workspace, dev)
    out = _output(out, (M, N), torch.int32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i4_splitk(M, N, K, a_packed.data_ptr(), b_packed.data_ptr(),
                                               out.data_ptr(), wp, wn, _stream_handle(dev)), "lpgemm_i4_splitk")
    return out


def gemm_f16_splitk(a, b_t, workspace, out=None):
    """gemm_f16 with K split over workgroups (see gemm_i8_splitk); the parts
    are added in a fixed order."""
    torch = _torch()
    _operand(a, torch.float16, "a")
    _operand(b_t, torch.float16, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    dev = _same_device(a, b_t)
    M, K = a.shape
    N = b_t.shape[0]
    wp, wn = _workspace(workspace, dev)
    out = _output(out, (M, N), torch.float32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_f16_splitk(M, N, K, a.data_ptr(), b_t.data_ptr(), out.data_ptr(), wp, wn,
                                                _stream_handle(dev)), "lpgemm_f16_splitk")
    return out


def gemm_i8_dequant_splitk(a, b_t, row_scale, col_scale, workspace, out=None):
    """gemm_i8_dequant with K split over workgroups (see gemm_i8_splitk)."""
    torch = _torch()
    _operand(a, torch.int8, "a")
    _operand(b_t, torch.int8, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    M, K = a.shape
    N = b_t.shape[0]
    for t, n, name in ((row_scale, M, "row_scale"), (col_scale, N, "col_scale")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 1 \
                or t.shape[0] != n or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 GPU vector of length {n}")
    dev = _same_device(a, b_t, row_scale, col_scale)
    wp, wn = _workspace(workspace, dev)
    out = _output(out, (M, N), torch.float32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i8_dequant_splitk(M, N, K, a.data_ptr(), b_t.data_ptr(),
                                                       row_scale.data_ptr(), col_scale.data_ptr(),
                                                       out.data_ptr(), wp, wn, _stream_handle(dev)),
               "lpgemm_i8_dequant_splitk")
    return out


def quantize_rows_f16(x, q_out=None, scale_out=None):
    """Per-row int8 quantisation of fp16 x (M x K): returns (q int8 M x K,
    scale fp32 M) with scale = absmax / 127 and q = nearest-even integer to
    x / scale (binary32), clamped to [-127, 127]."""
    torch = _torch()
    _operand(x, torch.float16, "x")
    dev = x.device
    M, K = x.shape
    q_out = _output(q_out, (M, K), torch.int8, dev)
    if scale_out is None:
        scale_out = torch.empty((M,), dtype=torch.float32, device=dev)
    elif scale_out.dtype != torch.float32 or tuple(scale_out.shape) != (M,) or not scale_out.is_contiguous():
        raise ValueError(f"scale_out must be a contiguous fp32 vector of length {M}")
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_quantize_rows_f16(M, K, x.data_ptr(), q_out.data_ptr(),
                                                       scale_out.data_ptr(), _stream_handle(dev)),
               "lpgemm_quantize_rows_f16")
    return q_out, scale_out


def w8a8_linear(x, w, w_scale, out=None):
    """fp32 y = dequant(quantize(x) . w): x fp16 M x K activations, w int8
    N x K weights (K-contiguous), w_scale fp32 per output column.  Two library
    calls on the current stream: lpgemm_quantize_rows_f16 (into buffers this
    function allocates) and lpgemm_i8_dequant."""
    q, s = quantize_rows_f16(x)
    return gemm_i8_dequant(q, w, s, w_scale, out=out)


def w8a8_linear_fused(x, w, w_scale, out=None):
    """The same result as w8a8_linear in one launch (lpgemm_w8a8_fused): the
    kernel quantises the rows of x itself.  x fp16 M x K with M <= 32, w int8
    N x K, w_scale fp32 N."""
    torch = _torch()
    _operand(x, torch.float16, "x")
    _operand(w, torch.int8, "w")
    if x.shape[1] != w.shape[1]:
        raise ValueError(f"K mismatch: x {tuple(x.shape)}, w {tuple(w.shape)}")
    M, K = x.shape
    N = w.shape[0]
    if not isinstance(w_scale, torch.Tensor) or w_scale.dtype != torch.float32 or w_scale.dim() != 1 \
            or w_scale.shape[0] != N or not w_scale.is_cuda or not w_scale.is_contiguous():
        raise ValueError(f"w_scale must be a contiguous fp32 GPU vector of length {N}")
    dev = _same_device(x, w, w_scale)
    out = _output(out, (M, N), torch.float32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_w8a8_fused(M, N, K, x.data_ptr(), w.data_ptr(), w_scale.data_ptr(),
                                                out.data_ptr(), _stream_handle(dev)), "lpgemm_w8a8_fused")
    return out


def i4_to_e3m2(packed, out=None):
    """Re-encode packed int4 rows (rows x K/2 uint8, low nibble = even k) as
    the FP6 E3M2 operand rows that gemm_i4_e3m2 takes (rows x K uint8)."""
    torch = _torch()
    _operand(packed, torch.uint8, "packed")
    rows, half = packed.shape
    K = 2 * half
    out = _output(out, (rows, K), torch.uint8, packed.device)
    with torch.cuda.device(packed.device):
        _check(load_library().lpgemm_i4_to_e3m2(rows, K, packed.data_ptr(), out.data_ptr(),
                                                _stream_handle(packed.device)), "lpgemm_i4_to_e3m2")
    return out


def gemm_i4_e3m2(a_e3m2, b_e3m2, out=None):
    """int32 C = A . B for int4 operands re-encoded by i4_to_e3m2 (M x K and
    N x K uint8); equal to gemm_i4 on the packed operands."""
    torch = _torch()
    _operand(a_e3m2, torch.uint8, "a_e3m2")
    _operand(b_e3m2, torch.uint8, "b_e3m2")
    if a_e3m2.shape[1] != b_e3m2.shape[1]:
        raise ValueError("K mismatch")
    dev = _same_device(a_e3m2, b_e3m2)
    M, K = a_e3m2.shape
    N = b_e3m2.shape[0]
    out = _output(out, (M, N), torch.int32, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_i4_e3m2(M, N, K, a_e3m2.data_ptr(), b_e3m2.data_ptr(),
                                             out.data_ptr(), _stream_handle(dev)), "lpgemm_i4_e3m2")
    return out


def gemm_i4_via_e3m2(a_packed, b_packed, out=None):
    """gemm_i4 through the FP6 matrix cores: both operands are re-encoded
    (into buffers this function allocates), then multiplied; three library
    calls on the current stream."""
    return gemm_i4_e3m2(i4_to_e3m2(a_packed), i4_to_e3m2(b_packed), out=out)


def f64_emu_moduli(K: int, bits: int = 53) -> int:
    """Number of moduli (one int8 GEMM each) the fp64 emulation uses."""
    return int(load_library().lpgemm_f64_emu_moduli(K, bits))


def f64_emu_workspace_bytes(M: int, N: int, K: int, bits: int = 53) -> int:
    return int(load_library().lpgemm_f64_emu_workspace(M, N, K, bits))


def gemm_f64_emu(a, b_t, bits: int = 53, workspace=None, out=None):
    """fp64 C ~ A . B through exact int8 GEMMs and the Chinese remainder
    theorem; a: M x K float64, b_t: N x K float64 (B K-contiguous); rows of A
    and columns of B are scaled to integers of `bits` bits.  `workspace`: a
    uint8 GPU tensor of at least f64_emu_workspace_bytes(...) bytes
    (allocated here when omitted)."""
    torch = _torch()
    _operand(a, torch.float64, "a")
    _operand(b_t, torch.float64, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    dev = _same_device(a, b_t)
    M, K = a.shape
    N = b_t.shape[0]
    need = f64_emu_workspace_bytes(M, N, K, bits)
    if need < 0:
        raise ValueError(f"unsupported fp64-emulation arguments K={K}, bits={bits}")
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.numel() < need or not workspace.is_cuda:
        raise ValueError(f"workspace must be a uint8 GPU tensor of at least {need} bytes")
    out = _output(out, (M, N), torch.float64, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_f64_emu(M, N, K, a.data_ptr(), b_t.data_ptr(), out.data_ptr(), bits,
                                             workspace.data_ptr(), workspace.numel(),
                                             _stream_handle(dev)), "lpgemm_f64_emu")
    return out


def gemm_f64_emu_noalloc(a, b_t, bits: int = 53, out=None):
    """gemm_f64_emu without a workspace: the library's own fixed scratch
    (LPGEMM_F64_EMU_NOALLOC_MAX_WORKSPACE bytes per GPU) holds the
    intermediates, so the call allocates nothing on the device beyond `out`
    when it is omitted.  Calls that overlap on one GPU race on that scratch."""
    torch = _torch()
    _operand(a, torch.float64, "a")
    _operand(b_t, torch.float64, "b_t")
    if a.shape[1] != b_t.shape[1]:
        raise ValueError(f"K mismatch: a {tuple(a.shape)}, b_t {tuple(b_t.shape)}")
    dev = _same_device(a, b_t)
    M, K = a.shape
    N = b_t.shape[0]
    out = _output(out, (M, N), torch.float64, dev)
    with torch.cuda.device(dev):
        _check(load_library().lpgemm_f64_emu_noalloc(M, N, K, a.data_ptr(), b_t.data_ptr(), out.data_ptr(),
                                                     bits, _stream_handle(dev)), "lpgemm_f64_emu_noalloc")
    return out
