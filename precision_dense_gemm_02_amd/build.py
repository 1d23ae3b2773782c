"""Build liblpgemm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m precision_dense_gemm_02_amd.build

Every call compiles from source; the library lands next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblpgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, "lpgemm.hip")]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


PROBES = os.path.join(ROOT, "probes")


def build_probes(verbose: bool = False) -> list:
    """Compile the stand-alone measurement probes in probes/ (executables
    next to their sources; not part of the library)."""
    built = []
    for name in sorted(os.listdir(PROBES)) if os.path.isdir(PROBES) else []:
        if not name.endswith(".hip"):
            continue
        src = os.path.join(PROBES, name)
        exe = src[:-4]
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", exe]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}:\n{r.stderr}")
        built.append(exe)
    return built


if __name__ == "__main__":
    print(build(verbose=True))
    for exe in build_probes(verbose=True):
        print(exe)
