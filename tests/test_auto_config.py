"""The automatic per-shape kernel choice, as host arithmetic
(lpgemm_auto_config): each row pins one measured rule on a 256-CU MI355X,
so that a change to the rules shows here without a GPU.  The numbers are
configuration indices of the library's table (dispatch.hpp)."""
import pytest

import precision_dense_gemm_02_amd as lp

CU = 256

# (kind, M, N, K, configuration, the rule)
TABLE = [
    ("i8", 8192, 8192, 8192, 47, "four whole rounds of 256 x 256 tiles: persistent grid"),
    ("f16", 8192, 8192, 8192, 47, "the same for fp16"),
    ("i4", 8192, 8192, 8192, 0, "int4 keeps the plain grid (registers)"),
    ("i8", 4096, 4096, 4096, 0, "one round of 256 x 256 tiles"),
    ("i8", 3072, 3072, 4096, 0, "144 large tiles, more than half the CUs"),
    ("i8", 5120, 8192, 4096, 0, "2.5 rounds: the plain grid"),
    ("i8", 6144, 8192, 4096, 47, "three whole rounds: persistent"),
    ("dq", 2048, 14336, 4096, 62, "N = 64 x 224: two whole rounds of 256 x 224 tiles"),
    ("dq", 1536, 14336, 4096, 61, "1.5 rounds of 256 x 224 tiles: plain"),
    ("dq", 1024, 14336, 4096, 61, "one round of 256 x 224 tiles"),
    ("dq", 512, 14336, 4096, 65, "128 tiles of 256 x 224, only half the CUs: 224 of 128 x 256"),
    ("i8", 2048, 4096, 4096, 65, "256 tiles of 128 x 256: one round of half-size large tiles"),
    ("i8", 1536, 4096, 4096, 65, "192 of them, three quarters of a round"),
    ("i4", 2048, 4096, 4096, 64, "int4: 256 x 128"),
    ("i8", 1024, 4096, 4096, 22, "128 half-size tiles, half the CUs: 128 x 128"),
    ("i8", 1536, 6144, 2048, 0, "144 large tiles: 256 x 256"),
    ("dq", 8192, 14336, 4096, 47, "seven whole rounds of 256 x 256 beat eight of 224"),
    ("i4", 2048, 14336, 4096, 62, "int4 too (configuration 62 runs 61's plain grid for int4)"),
    ("dq", 256, 14336, 4096, 22, "64 tiles of 224: 128 x 128 tiles, four 128-byte stages"),
    ("i8", 2048, 2048, 2048, 36, "one round of 128 x 128 tiles at K = 2048: two 256-byte stages"),
    ("i8", 2048, 2048, 4096, 22, "K = 4096: four 128-byte stages"),
    ("f16", 2048, 2048, 2048, 22, "fp16: four 128-byte stages"),
    ("i4", 2048, 2048, 2048, 48, "int4: 32-byte fragment reads"),
    ("i8", 1024, 1024, 8192, 34, "128 band tiles at K >= 2048: the band kernel"),
    ("f16", 1024, 1024, 4096, 34, "the same for fp16"),
    ("i8", 1536, 1536, 1536, 36, "288 band tiles, more than a round: one round of 128 x 128 at K <= 2048"),
    ("i8", 1024, 1024, 1024, 6, "K = 1024: 64 x 64 tiles"),
    ("i4", 1024, 1024, 4096, 15, "int4 from K = 4096: 32 x 32 tiles, waves split K"),
    ("i8", 512, 512, 512, 15, "at most half a round of 64 x 64 tiles: waves split K"),
    ("dq", 128, 14336, 4096, 34, "a 128-row band"),
    ("i4", 128, 14336, 4096, 34, "int4 at 128 rows: the band kernel"),
    ("i4", 96, 14336, 4096, 15, "int4 up to 96 rows: eight-wave skinny kernel"),
    ("dq", 64, 14336, 4096, 34, "33-64 rows, 224 band tiles: the band kernel"),
    ("dq", 64, 8192, 4096, 14, "33-64 rows, 128 band tiles: the skinny kernel"),
    ("dq", 16, 14336, 4096, 14, "M <= 32: the skinny kernel"),
    ("i8", 32, 8192, 8192, 14, "256 column tiles of 32: four waves"),
    ("i8", 32, 4096, 4096, 15, "128 column tiles, half the CUs: eight waves"),
    ("dq", 16, 4096, 14336, 15, "the same at K = 14336"),
    ("i8", 64, 4096, 4096, 15, "33-64 rows at few columns: eight waves"),
    ("i4", 16, 14336, 4096, 15, "int4 at M <= 32: eight waves"),
]


@pytest.mark.parametrize("kind,M,N,K,cfg,rule", TABLE)
def test_rule(kind, M, N, K, cfg, rule):
    assert lp.auto_config(kind, M, N, K, CU) == cfg, rule


def test_forced_configuration_does_not_change_the_answer():
    prev = lp.force_config(5)
    try:
        assert lp.auto_config("i8", 8192, 8192, 8192, CU) == 47
    finally:
        lp.force_config(prev)


def test_out_of_range_arguments():
    assert lp.auto_config("i8", 0, 8192, 8192, CU) == -1     # nothing launches
    assert lp.auto_config("i8", 8192, 0, 8192, CU) == -1
    assert lp.auto_config("i8", 8192, 8192, -1, CU) == -1
    assert lp.auto_config("i8", 8192, 8192, 8192, 0) == -1
    assert lp.auto_config("i8", 2 ** 31, 8192, 8192, CU) == -1
    assert lp.load_library().lpgemm_auto_config(4, 64, 64, 64, CU) == -1   # not one of the four kinds
    assert lp.auto_config("i8", 8192, 8192, 0, CU) == 47     # K = 0: C is written as zeros


def test_other_device_sizes():
    # the rules scale with the CU count: on 128 CUs, 8192^3 is eight whole
    # rounds and 2048 x 14336 four
    assert lp.auto_config("i8", 8192, 8192, 8192, 128) == 47
    assert lp.auto_config("dq", 2048, 14336, 4096, 128) == 62
    assert lp.auto_config("dq", 16, 14336, 4096, 128) == 14
