"""The seeded input generators: reproducible, inclusive ranges, int4 packing."""
import numpy as np

from precision_dense_gemm_02_amd import inputs


def test_reproducible():
    a = inputs.int8_problem(64, 32, 128, seed=5, scales=True)
    b = inputs.int8_problem(64, 32, 128, seed=5, scales=True)
    for x, y in ((a.a, b.a), (a.b_t, b.b_t), (a.row_scale, b.row_scale), (a.col_scale, b.col_scale)):
        np.testing.assert_array_equal(x, y)
    c = inputs.int8_problem(64, 32, 128, seed=6)
    assert not np.array_equal(a.a, c.a)


def test_int8_range_inclusive():
    p = inputs.int8_problem(512, 512, 512, seed=1)
    assert p.a.dtype == np.int8 and p.b_t.shape == (512, 512)
    assert p.a.min() == -128 and p.a.max() == 127


def test_int4_range_and_packing():
    p = inputs.int4_problem(256, 128, 512, seed=2)
    assert p.a_values.min() == -8 and p.a_values.max() == 7
    assert p.a_packed.shape == (256, 256) and p.b_packed.shape == (128, 256)
    lo = (p.a_packed & 0xF).astype(np.int16)
    hi = (p.a_packed >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    np.testing.assert_array_equal(lo, p.a_values[:, 0::2])
    np.testing.assert_array_equal(hi, p.a_values[:, 1::2])


def test_f16_distribution():
    p = inputs.f16_problem(512, 512, 512, seed=3)
    a = p.a.astype(np.float64)
    assert p.a.dtype == np.float16 and np.isfinite(a).all()
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1.0) < 0.01


def test_scales_range():
    p = inputs.llm_problem(16)
    assert p.a.shape == (16, 4096) and p.b_t.shape == (14336, 4096)
    for s in (p.row_scale, p.col_scale):
        assert s.dtype == np.float32 and s.min() >= 0.001 and s.max() <= 0.01
