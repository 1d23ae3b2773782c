"""CPU oracle for the low-precision dense GEMM (numpy front end of oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may call it; the GPU library never does, and this module
imports nothing from it.

Every function takes numpy arrays in the library's layouts -- A is M x K
row-major, B is stored K-contiguous (an N x K array), the int4 operands are
packed two per byte along k with the low nibble holding the even k -- and
returns new numpy arrays.  ``rows`` restricts the computation to a subset of
output rows (a ``range`` or a sequence of row indices); the result then holds
just those rows, in that order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class OracleError(RuntimeError):
    """An input lies outside the contract of the operation (see oracle.c)."""


_STATUS = {1: "integer result does not fit int32",
           2: "fp16 or fp64 operand is inf or NaN",
           3: "bad row range, odd K or target bits outside [1, 53]",
           4: "working buffer could not be allocated"}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (plain gcc, OpenMP,
    no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _configure(lib):
    """Declare the argument and result types of the oracle entry points."""
    for name in ("oracle_i8", "oracle_i4"):
        f = getattr(lib, name)
        f.argtypes = [_i64, _i64, _i64, _p, _p, _p, _i64, _i64]
        f.restype = ctypes.c_int
    lib.oracle_f16.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _i64, _i64]
    lib.oracle_f16.restype = ctypes.c_int
    lib.oracle_i8_dequant.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _i64, _i64]
    lib.oracle_i8_dequant.restype = ctypes.c_int
    lib.oracle_f16_decode.argtypes = [ctypes.c_uint16, ctypes.POINTER(ctypes.c_int)]
    lib.oracle_f16_decode.restype = ctypes.c_double
    lib.oracle_quantize_rows_f16.argtypes = [_i64, _i64, _p, _p, _p, _i64, _i64]
    lib.oracle_quantize_rows_f16.restype = ctypes.c_int
    lib.oracle_f64_emu.argtypes = [_i64, _i64, _i64, _p, _p, ctypes.c_int, _p, _i64, _i64]
    lib.oracle_f64_emu.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise OracleError(_STATUS.get(status, f"status {status}"))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _row_runs(rows, M):
    """Split the requested rows into contiguous [begin, end) runs."""
    if rows is None:
        return [(0, M)]
    if isinstance(rows, range) and rows.step == 1:
        return [(rows.start, rows.stop)]
    idx = [int(r) for r in rows]
    runs = []
    for r in idx:
        if runs and runs[-1][1] == r:
            runs[-1][1] = r + 1
        else:
            runs.append([r, r + 1])
    return [tuple(r) for r in runs]


def _run_rows(fn, M, N, rows, outs, *args):
    """Call a row-range oracle entry point once per contiguous run of rows and
    stack the pieces in the requested order."""
    pieces = [[] for _ in outs]
    for b, e in _row_runs(rows, M):
        bufs = [np.empty((e - b, N), dtype=dt) for dt in outs]
        _check(fn(*args, *[_ptr(x) for x in bufs], b, e))
        for p, x in zip(pieces, bufs):
            p.append(x)
    res = [np.concatenate(p, axis=0) if p else np.empty((0, N), dt) for p, dt in zip(pieces, outs)]
    return res


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def gemm_i8(A: np.ndarray, B_t: np.ndarray, rows=None) -> np.ndarray:
    """C = A . B for int8 A (M x K) and int8 B stored as N x K; int32 C."""
    A = _c(A, np.int8)
    B_t = _c(B_t, np.int8)
    M, K = A.shape
    N = B_t.shape[0]
    assert B_t.shape[1] == K
    lib = _load()
    (C,) = _run_rows(lambda *a: lib.oracle_i8(M, N, K, _ptr(A), _ptr(B_t), *a),
                     M, N, rows, [np.int32])
    return C


def gemm_i4(A_packed: np.ndarray, B_packed: np.ndarray, K: int, rows=None) -> np.ndarray:
    """C = A . B for signed int4 operands packed two per byte along k (low
    nibble = even k); A_packed is M x K/2, B_packed is N x K/2; int32 C."""
    A_packed = _c(A_packed, np.uint8)
    B_packed = _c(B_packed, np.uint8)
    M = A_packed.shape[0]
    N = B_packed.shape[0]
    assert A_packed.shape[1] * 2 == K and B_packed.shape[1] * 2 == K
    lib = _load()
    (C,) = _run_rows(lambda *a: lib.oracle_i4(M, N, K, _ptr(A_packed), _ptr(B_packed), *a),
                     M, N, rows, [np.int32])
    return C


def gemm_f16(A: np.ndarray, B_t: np.ndarray, rows=None):
    """fp64 reference for fp16 A (M x K) and fp16 B stored as N x K.

    Returns (ref, den): ref = sum_k a*b and den = sum_k |a|*|b|, both fp64."""
    A = _c(A, np.float16).view(np.uint16)
    B_t = _c(B_t, np.float16).view(np.uint16)
    M, K = A.shape
    N = B_t.shape[0]
    assert B_t.shape[1] == K
    lib = _load()
    ref, den = _run_rows(lambda *a: lib.oracle_f16(M, N, K, _ptr(A), _ptr(B_t), *a),
                         M, N, rows, [np.float64, np.float64])
    return ref, den


def gemm_i8_dequant(A: np.ndarray, B_t: np.ndarray, row_scale: np.ndarray,
                    col_scale: np.ndarray, rows=None) -> np.ndarray:
    """fp32 out = ((float)acc * row_scale[i]) * col_scale[j], acc the exact
    int8 product."""
    A = _c(A, np.int8)
    B_t = _c(B_t, np.int8)
    rs = _c(row_scale, np.float32)
    cs = _c(col_scale, np.float32)
    M, K = A.shape
    N = B_t.shape[0]
    assert B_t.shape[1] == K and rs.shape == (M,) and cs.shape == (N,)
    lib = _load()
    (out,) = _run_rows(lambda *a: lib.oracle_i8_dequant(M, N, K, _ptr(A), _ptr(B_t),
                                                         _ptr(rs), _ptr(cs), *a),
                       M, N, rows, [np.float32])
    return out


def quantize_rows_f16(X: np.ndarray, rows=None):
    """Per-row int8 quantisation of fp16 X (M x K): returns (Q int8 M x K,
    scale float32 M) with scale = absmax / 127 and Q = nearest-even integer to
    x / scale, both in binary32, clamped to [-127, 127]."""
    X = _c(X, np.float16).view(np.uint16)
    M, K = X.shape
    lib = _load()
    qs, ss = [], []
    for b, e in _row_runs(rows, M):
        q = np.empty((e - b, K), np.int8)
        sc = np.empty(e - b, np.float32)
        _check(lib.oracle_quantize_rows_f16(M, K, _ptr(X), _ptr(q), _ptr(sc), b, e))
        qs.append(q)
        ss.append(sc)
    if not qs:
        return np.empty((0, K), np.int8), np.empty(0, np.float32)
    return np.concatenate(qs, axis=0), np.concatenate(ss)


def f64_emu(A: np.ndarray, B_t: np.ndarray, bits: int, rows=None) -> np.ndarray:
    """fp64 product through scaled integers: rows of A and rows of B_t (the
    columns of B) scaled by powers of two to integers of at most `bits`
    bits (nearest, ties to even), multiplied exactly, converted to double
    once and scaled back.  A: M x K float64, B_t: N x K float64."""
    A = _c(A, np.float64)
    B_t = _c(B_t, np.float64)
    M, K = A.shape
    N = B_t.shape[0]
    assert B_t.shape[1] == K
    lib = _load()
    (C,) = _run_rows(lambda *a: lib.oracle_f64_emu(M, N, K, _ptr(A), _ptr(B_t), int(bits), *a),
                     M, N, rows, [np.float64])
    return C


def f16_decode(bits: int):
    """Exact value of one binary16 bit pattern; None for inf/NaN."""
    fin = ctypes.c_int(0)
    v = _load().oracle_f16_decode(ctypes.c_uint16(bits), ctypes.byref(fin))
    return v if fin.value else None


def f16_rel_error(C: np.ndarray, ref: np.ndarray, den: np.ndarray):
    """Error fields of an fp16 GEMM result against the fp64 reference.

    rel = |C - ref| / den elementwise (where den == 0 the result must be
    exactly 0; such an element counts as error 0 if it is, inf otherwise)."""
    C = np.asarray(C, dtype=np.float64)
    diff = np.abs(C - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, diff / np.where(den > 0, den, 1.0),
                       np.where(C == 0.0, 0.0, np.inf))
    return {
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "rms_rel": float(np.sqrt(np.mean(rel ** 2))) if rel.size else 0.0,
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "rms_abs": float(np.sqrt(np.mean(diff ** 2))) if diff.size else 0.0,
    }


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())
