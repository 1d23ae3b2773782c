"""Low-precision dense GEMM for AMD MI355X (gfx950).

C = A . B with INT8 and packed INT4 operands summed exactly in int32, FP16
operands summed in FP32, and an INT8 variant with per-row x per-column fp32
dequantisation; around them, the per-row int8 quantiser of fp16 activations
(W8A8), the INT4 path through the FP6 E3M2 matrix cores, split-K variants
for products with few output tiles, and an fp64 GEMM emulated with exact
INT8 GEMMs.  The work runs in
hand-written HIP kernels behind the C ABI of include/lpgemm.h; this package is
the torch-facing binding (see _binding.py), the in-tree build step (build.py)
and the seeded input generators (inputs.py).
"""
from ._binding import (LpgemmError, auto_config, config_count, f64_emu_moduli, force_config, f64_emu_workspace_bytes, gemm_f16, gemm_f64_emu, gemm_f64_emu_noalloc, gemm_i4, gemm_i4_e3m2, gemm_i4_via_e3m2,  # noqa: F401
                       gemm_f16_splitk, gemm_i4_splitk, gemm_i8_dequant_splitk, gemm_i8_splitk,
                       gemm_i8, gemm_i8_dequant, gemm_i8_kxn, i4_to_e3m2, load_library, quantize_rows_f16,
                       splitk_workspace, splitk_workspace_bytes, status_string, version, w8a8_linear,
                       w8a8_linear_fused)

__all__ = ["LpgemmError", "gemm_i8", "gemm_i8_kxn", "gemm_i4", "gemm_f16", "gemm_i8_dequant",
           "quantize_rows_f16", "w8a8_linear", "w8a8_linear_fused", "i4_to_e3m2", "gemm_i4_e3m2", "gemm_i4_via_e3m2",
           "gemm_f64_emu", "gemm_f64_emu_noalloc", "f64_emu_moduli", "f64_emu_workspace_bytes",
           "gemm_i8_splitk", "gemm_i4_splitk", "gemm_f16_splitk", "gemm_i8_dequant_splitk",
           "splitk_workspace", "splitk_workspace_bytes",
           "load_library", "status_string", "version", "config_count", "force_config", "auto_config"]
