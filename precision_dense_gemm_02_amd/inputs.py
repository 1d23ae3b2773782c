"""Seeded synthetic inputs for the GEMM workloads.

This module holds only random draws and the storage encoding of the operands
(layout and int4 packing); none of the GEMM arithmetic.  Both the GPU tests
and the CPU oracle consume the host arrays it returns, so the two sides always
see identical bytes.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, PCG64, draws in
the fixed order A, B, row scales, column scales):

* int8  : uniform integers in [-128, 127], both ends inclusive.
* int4  : uniform integers in [-8, 7], packed two per byte along k, the low
          nibble holding the even k, two's complement nibbles.
* fp16  : standard normal fp64 draws rounded to fp16 (round to nearest even),
          the error procedure of the forum post on compiler-generated kernels
          (paragraph on hybrid FP16/FP32 accumulation).
* scales: uniform fp64 in [0.001, 0.01), rounded to fp32.
* W8A8 activations: standard normal fp64 draws times a per-row magnitude
          2^u, u uniform in [-4, 4) (rows of very different ranges, as the
          tokens of a layer's input have), rounded to fp16; then the int8
          weights and the fp32 weight scales as above.

Layouts: A is M x K row-major; B is stored K-contiguous, i.e. as an N x K
row-major array (``b_t``); C is M x N row-major.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

SEED_BASE = 20260

# Workload families and their square sweep sizes; the LLM projection uses
# K = 4096 and N = 14336 with M tokens.
I8_SIZES = (512, 1024, 2048, 4096, 8192)
I4_SIZES = (512, 2048, 8192)
F16_SIZES = (512, 2048, 4096, 8192)
LLM_TOKENS = (16, 128, 2048)
LLM_K = 4096
LLM_N = 14336

# Seed offset per workload family (seed = SEED_BASE + index).
FAMILY_INDEX = {"i8": 1, "i4": 2, "f16": 3, "llm": 4, "w8a8": 5, "f64": 6}


def seed_for(family: str, extra: int = 0) -> int:
    return SEED_BASE + FAMILY_INDEX[family] + 1000 * extra


def pack_int4(values: np.ndarray) -> np.ndarray:
    """Pack signed 4-bit values (int8 array in [-8, 7], last axis even) two per
    byte: element 2t goes to the low nibble of byte t, element 2t+1 to the
    high nibble, each as a two's-complement nibble."""
    v = np.asarray(values)
    if v.shape[-1] % 2:
        raise ValueError("last axis must have even length")
    if v.size and (v.min() < -8 or v.max() > 7):
        raise ValueError("int4 values must lie in [-8, 7]")
    nib = (v.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


@dataclass
class Int8Problem:
    a: np.ndarray            # M x K int8
    b_t: np.ndarray          # N x K int8
    row_scale: Optional[np.ndarray] = None   # M fp32
    col_scale: Optional[np.ndarray] = None   # N fp32


@dataclass
class Int4Problem:
    a_values: np.ndarray     # M x K int8 in [-8, 7]
    b_values: np.ndarray     # N x K int8 in [-8, 7]
    a_packed: np.ndarray     # M x K/2 uint8
    b_packed: np.ndarray     # N x K/2 uint8


@dataclass
class F16Problem:
    a: np.ndarray            # M x K fp16
    b_t: np.ndarray          # N x K fp16


def int8_problem(M: int, N: int, K: int, seed: int, scales: bool = False) -> Int8Problem:
    rng = np.random.default_rng(seed)
    a = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    b_t = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    if not scales:
        return Int8Problem(a, b_t)
    rs = rng.uniform(0.001, 0.01, size=M).astype(np.float32)
    cs = rng.uniform(0.001, 0.01, size=N).astype(np.float32)
    return Int8Problem(a, b_t, rs, cs)


def int4_problem(M: int, N: int, K: int, seed: int) -> Int4Problem:
    rng = np.random.default_rng(seed)
    a = rng.integers(-8, 8, size=(M, K), dtype=np.int8)
    b = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    return Int4Problem(a, b, pack_int4(a), pack_int4(b))


def f16_problem(M: int, N: int, K: int, seed: int) -> F16Problem:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=(M, K)).astype(np.float16)
    b_t = rng.standard_normal(size=(N, K)).astype(np.float16)
    return F16Problem(a, b_t)


def f16_integer_problem(M: int, N: int, K: int, seed: int, lo: int = -8, hi: int = 7) -> F16Problem:
    """fp16 operands holding small integers in [lo, hi]: every partial sum is
    an integer far below 2^24, so an fp32-accumulated product is exact."""
    rng = np.random.default_rng(seed)
    a = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float16)
    b_t = rng.integers(lo, hi + 1, size=(N, K)).astype(np.float16)
    return F16Problem(a, b_t)


def llm_problem(M: int, seed: Optional[int] = None) -> Int8Problem:
    """Quantised LLM projection: M tokens x K=4096 activations, N=14336 x
    K=4096 weights, per-row and per-column fp32 scales."""
    if seed is None:
        seed = seed_for("llm", M)
    return int8_problem(M, LLM_N, LLM_K, seed, scales=True)


@dataclass
class W8A8Problem:
    x: np.ndarray            # M x K fp16 activations
    w: np.ndarray            # N x K int8 weights (K-contiguous)
    w_scale: np.ndarray      # N fp32 weight scales


def w8a8_problem(M: int, N: int = LLM_N, K: int = LLM_K, seed: Optional[int] = None) -> W8A8Problem:
    """fp16 activations for the quantise-then-GEMM projection, with int8
    weights and per-column fp32 weight scales."""
    if seed is None:
        seed = seed_for("w8a8", M)
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-4.0, 4.0, size=(M, 1)))
    x = (rng.standard_normal(size=(M, K)) * mag).astype(np.float16)
    w = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    ws = rng.uniform(0.001, 0.01, size=N).astype(np.float32)
    return W8A8Problem(x, w, ws)
