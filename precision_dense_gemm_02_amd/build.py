"""Build liblpgemm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m precision_dense_gemm_02_amd.build

Every call compiles from source: each translation unit of csrc/ (the C entry
points, and one unit per operand kind holding that kind's kernel
instantiations) is compiled to an object in parallel, then the objects are
linked into one shared library next to this file.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblpgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list:
    """The library's translation units."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _filter(stderr: str) -> str:
    # the host pass warns that it does not know the packed-fp32 feature
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16, int(os.environ.get("MAX_JOBS", "16"))))


TEST_HIP = os.path.join(ROOT, "tests", "hip")


def test_probe_sources() -> list:
    """HIP sources of the test suite's device probes (each becomes a shared
    library next to it; the product library never loads them)."""
    return sorted(glob.glob(os.path.join(TEST_HIP, "*.hip")))


def _build_test_probe(src: str, verbose: bool = False) -> str:
    out = os.path.join(os.path.dirname(src), "lib" + os.path.basename(src)[:-4] + ".so")
    cmd = [HIPCC, *FLAGS, "-shared", src, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({r.returncode}):\n{_filter(r.stderr)}")
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    srcs = sources()
    with ThreadPoolExecutor(max_workers=2) as outer:
        probes = [outer.submit(_build_test_probe, p, verbose) for p in test_probe_sources()]
        lib = _build_library(srcs, verbose)
        for f in probes:
            f.result()
    return lib


def _build_library(srcs: list, verbose: bool) -> str:
    with tempfile.TemporaryDirectory(prefix="lpgemm_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src)[:-4] + ".o")
            cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, r.returncode, _filter(r.stderr)

        with ThreadPoolExecutor(max_workers=_jobs()) as ex:
            results = list(ex.map(compile_one, srcs))
        for src, _, rc, err in results:
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _, _ in results],
               "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{_filter(r.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
