"""Register and LDS budget of every kernel instantiation, as the compiler
reports it for gfx950 (CPU only: hipcc cross-compiles).

No kernel may spill to scratch (a spill inside a GEMM main loop costs far
more than the instructions it saves), and the 256x256 GEMM kernels must fit
one workgroup of four waves per CU: 256 accumulator registers per lane for
the 128x128 quadrant, at most 256 VGPRs, and at most 160 KiB of LDS."""
import shutil

import pytest

from precision_dense_gemm_02_amd import resource_usage

pytestmark = pytest.mark.skipif(shutil.which("c++filt") is None, reason="needs c++filt")


@pytest.fixture(scope="module")
def usage():
    return resource_usage.collect()


def test_every_kernel_is_reported(usage):
    # every configuration of every kind, plus the quantiser, re-encoding and
    # fp64-emulation kernels
    assert len(usage) > 150
    for name in resource_usage.DEFAULT_KERNELS:
        assert any(k.split("(")[0].endswith(name) for k in usage), name


def test_no_kernel_spills(usage):
    spilled = {k: v for k, v in usage.items()
               if v.get("VGPRs Spill", "0") != "0" or v.get("ScratchSize [bytes/lane]", "0") != "0"}
    assert not spilled, sorted(spilled)[:5]


def test_default_256_kernels_fit_one_workgroup_per_cu(usage):
    for k, v in usage.items():
        if "gemm_v3<" in k and "256, 256, 2, 128" in k:
            assert int(v["AGPRs"]) == 256, k
            assert int(v["VGPRs"]) <= 256, k
            assert int(v["LDS Size [bytes/block]"]) <= 160 * 1024, k
            assert int(v["Occupancy [waves/SIMD]"]) == 1, k
