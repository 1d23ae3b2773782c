"""The oracle against the hand-worked products in tests/golden."""
import json
import os

import numpy as np

import oracle
from precision_dense_gemm_02_amd import inputs

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _mat(rows, dtype):
    return np.array([r["values"] for r in rows], dtype=dtype)


def _vals(c):
    return [[e["value"] for e in row] for row in c]


def test_int8_worked():
    g = G["int8"]
    A = _mat(g["A_rows"], np.int8)
    B_t = _mat(g["B_cols"], np.int8)
    assert A.shape[1] == g["K"]
    assert oracle.gemm_i8(A, B_t).tolist() == _vals(g["C"])


def test_int4_worked():
    g = G["int4"]
    A = _mat(g["A_rows"], np.int8)
    B_t = _mat(g["B_cols"], np.int8)
    Ap, Bp = inputs.pack_int4(A), inputs.pack_int4(B_t)
    assert int(Ap[1, 0]) == g["A_packed_row1_first_byte"]["value"]
    assert oracle.gemm_i4(Ap, Bp, g["K"]).tolist() == _vals(g["C"])


def test_fp16_worked():
    g = G["fp16"]
    ref, den = oracle.gemm_f16(_mat(g["A_rows"], np.float16), _mat(g["B_cols"], np.float16))
    assert ref.tolist() == _vals(g["ref"])
    assert den.tolist() == _vals(g["den"])


def test_dequant_worked():
    g = G["int8"]
    A = _mat(g["A_rows"], np.int8)
    B_t = _mat(g["B_cols"], np.int8)[:1]
    d = G["dequant"]
    out = oracle.gemm_i8_dequant(A, B_t, np.array(d["row_scale"], np.float32),
                                 np.array(d["col_scale"], np.float32))
    assert out.tolist() == _vals(d["out"])


def test_dequant_two_roundings():
    # fixtures where two binary32 roundings differ from one (exact derivation
    # in tests/golden/make_dequant_rounding.py)
    G2 = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dequant_rounding.json")))
    for case in G2["cases"]:
        A = np.array([case["a_row"]], np.int8)
        B_t = np.array([case["b_col"]], np.int8)
        assert int(oracle.gemm_i8(A, B_t)[0, 0]) == case["acc"]
        rs = np.array([int(case["row_scale_bits"], 16)], np.uint32).view(np.float32)
        cs = np.array([int(case["col_scale_bits"], 16)], np.uint32).view(np.float32)
        out = oracle.gemm_i8_dequant(A, B_t, rs, cs)
        assert int(out.view(np.uint32)[0, 0]) == int(case["expected_bits"], 16)
        assert case["expected_bits"] != case["single_rounding_bits"]
