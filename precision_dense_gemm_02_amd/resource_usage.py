"""Registers, LDS, scratch and occupancy of the library's kernels, as the
compiler reports them for gfx950.

    python -m precision_dense_gemm_02_amd.resource_usage [--all]

Compiles every translation unit of csrc/ once more (device code only) with
the compiler's resource-usage remarks and prints a markdown table.  Without --all only the kernels the automatic
configuration choice launches are listed.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

from concurrent.futures import ThreadPoolExecutor

from .build import FLAGS, HIPCC, _jobs, sources

# kernels launched by the automatic choice (the name's prefix up to the
# closing template bracket), and the workloads that run them
DEFAULT_KERNELS = {
    "lpgemm::gemm_v3<0, 256, 256, 2, 128, 0, false, false, 2, true, 0, false, true, true, 0, false, false>": "int8, >= 2 rounds of 256x256 tiles (8192^3), persistent",
    "lpgemm::gemm_v3<0, 256, 256, 2, 128, 0, false, false, 2, true, 0, false, true, false, 0, false, false>": "int8, 1-2 rounds of 256x256 tiles (4096^3)",
    "lpgemm::gemm_v3<1, 256, 256, 2, 128, 0, false, false, 2, false, 0, false, false, false, 0, false, false>": "int4, >= 1 round of 256x256 tiles",
    "lpgemm::gemm_v3<2, 256, 256, 2, 128, 0, false, false, 2, true, 0, false, true, true, 0, false, false>": "fp16, >= 2 rounds (8192^3), persistent",
    "lpgemm::gemm_v3<2, 256, 256, 2, 128, 0, false, false, 2, true, 0, false, true, false, 0, false, false>": "fp16, 1-2 rounds (4096^3)",
    "lpgemm::gemm_v3<3, 256, 256, 2, 128, 0, false, false, 2, true, 0, false, true, false, 0, false, false>": "dequant int8, 1-2 rounds of 256x256 tiles",
    "lpgemm::gemm_v3<0, 256, 224, 2, 128, 0, false, false, 2, true, 0, false, true, true, 0, false, false>": "int8, N a multiple of 224 (N = 14336), >= 2 rounds of 256x224 tiles, persistent",
    "lpgemm::gemm_v3<2, 256, 224, 2, 128, 0, false, false, 2, true, 0, false, true, true, 0, false, false>": "fp16, N a multiple of 224, persistent",
    "lpgemm::gemm_v3<3, 256, 224, 2, 128, 0, false, false, 2, true, 0, false, true, true, 0, false, false>": "dequant int8, N a multiple of 224 (LLM M = 2048), persistent",
    "lpgemm::gemm_v3<1, 256, 224, 2, 128, 0, false, false, 2, false, 0, false, false, false, 0, false, false>": "int4, N a multiple of 224",
    "lpgemm::gemm_v3<0, 128, 256, 3, 128, 0, false, false, 0, true, 0, false, false, false, 0, false, false>": "int8, half a round to one round of 128x256 tiles",
    "lpgemm::gemm_v3<1, 256, 128, 3, 128, 0, false, false, 0, false, 0, false, false, false, 0, false, false>": "int4, half a round to one round of 256x128 tiles",
    "lpgemm::gemm_v3<2, 128, 256, 3, 128, 0, false, false, 0, true, 0, false, false, false, 0, false, false>": "fp16, half a round to one round of 128x256 tiles",
    "lpgemm::gemm_v3<3, 128, 256, 3, 128, 0, false, false, 0, true, 0, false, false, false, 0, false, false>": "dequant int8, half a round to one round of 128x256 tiles",
    "lpgemm::gemm_v3<0, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, 0, false, false>": "int8, 128x128 tiles (2048^3)",
    "lpgemm::gemm_v3<2, 128, 128, 4, 128, 0, false, false, 0, false, 0, false, false, false, 0, false, false>": "fp16, 128x128 tiles (2048^3)",
    "lpgemm::gemm_v3<1, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, 1, false, false>": "int4, 128x128 tiles (2048^3), 32-byte fragment reads",
    "lpgemm::gemm_v3<3, 128, 64, 3, 256, 5, false, false, 0, false, 0, false, false, false, 0, false, false>": "dequant int8, M <= 128 (LLM M = 128), B non-temporal",
    "lpgemm::gemm_v3<0, 128, 64, 3, 256, 0, false, false, 0, false, 0, false, false, false, 0, false, false>": "int8, 128x64 band tiles above 128 rows",
    "lpgemm::gemm_v3<0, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, 0, false, true>": "int8 split-K (few tiles, long K)",
    "lpgemm::gemm_v3<1, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, 1, false, true>": "int4 split-K",
    "lpgemm::gemm_v3<2, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, 0, false, true>": "fp16 split-K",
    "lpgemm::gemm_v3<3, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, 0, false, true>": "dequant int8 split-K",
    "lpgemm::gemm_skinny_pipe<3, 4, 2, false, 1, 1>": "dequant int8, M <= 32 (LLM M = 16: 28 columns per workgroup)",
    "lpgemm::gemm_tiled<0, 64, 64, 2, 2>": "int8, small grids (1024^3, 512^3)",
    "lpgemm::quantize_rows_f16_regs<4, 2>": "W8A8 row quantiser, short M",
    "lpgemm::quantize_rows_f16_regs<1, 8>": "W8A8 row quantiser, M = 2048",
}
FIELDS = ["VGPRs", "AGPRs", "TotalSGPRs", "ScratchSize [bytes/lane]", "LDS Size [bytes/block]",
          "Occupancy [waves/SIMD]", "VGPRs Spill"]


def _remarks(src: str) -> str:
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", "--offload-device-only", src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr[-2000:])
    return r.stderr


def collect() -> dict:
    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        text = "\n".join(ex.map(_remarks, sources()))
    kernels, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([^:]+(?:\[[^\]]*\])?): (\S+) \[-Rpass", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = m.group(2)
    names = subprocess.run(["c++filt"], input="\n".join(kernels), capture_output=True,
                           text=True).stdout.splitlines()
    return {dem: kernels[mang] for mang, dem in zip(kernels, names)}


def main(argv=None) -> None:
    argv = sys.argv[1:] if argv is None else argv
    res = collect()
    print("| kernel | used for | " + " | ".join(FIELDS) + " |")
    print("|---|---|" + "---|" * len(FIELDS))
    for dem, rec in sorted(res.items()):
        key = dem.split("(")[0]
        key = key[len("void "):] if key.startswith("void ") else key
        if "--all" not in argv and key not in DEFAULT_KERNELS:
            continue
        print(f"| `{key}` | {DEFAULT_KERNELS.get(key, '')} | " +
              " | ".join(rec.get(f, "?") for f in FIELDS) + " |")


if __name__ == "__main__":
    main()
