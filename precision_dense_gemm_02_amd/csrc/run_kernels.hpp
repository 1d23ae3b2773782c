// Definition of run<KIND, BKN>: the kernel launch for each configuration.
// Included only by the run_*.hip translation units, each of which
// instantiates it for one operand kind.
#pragma once

#include "dispatch.hpp"

namespace lpgemm {

template <int KIND, bool BKN>
lpgemm_status run(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C,
                  const float* rs, const float* cs, hipStream_t stream, int modulus, void* ws,
                  int64_t ws_bytes) {
  // K x N B: k-rows of N bytes must start 16-byte aligned and the matrix
  // must fit the 32-bit offsets of its buffer resource (a shape error, so it
  // ranks with the K checks: after negative sizes, before pointers)
  if (BKN && M > 0 && N > 0 && K >= 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX &&
      (N % 16 != 0 || K * N >= ((int64_t)1 << 31)))
    return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  bool nothing_to_do = false;
  lpgemm_status st = validate((Kind)KIND, M, N, K, A, B, C, rs, cs, nothing_to_do);
  if (st != LPGEMM_SUCCESS || nothing_to_do) return st;
  // split-K workspace (the *_splitk entry points): may be null
  if (ws_bytes < 0) return LPGEMM_ERROR_INVALID_VALUE;
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return LPGEMM_ERROR_MISALIGNED;
  DeviceInfo dev;
  st = current_device(dev);
  if (st != LPGEMM_SUCCESS) return st;

  GemmArgs args{};
  args.A = static_cast<const uint8_t*>(A);
  args.B = static_cast<const uint8_t*>(B);
  args.C = C;
  args.row_scale = rs;
  args.col_scale = cs;
  args.M = (int)M;
  args.N = (int)N;
  args.modulus = modulus;
  args.inv_modulus = modulus > 0 ? 1.0 / (double)modulus : 0.0;
  // bytes per operand row: fp16 2K, packed int4 K/2, int8 and E3M2 K
  const int64_t row_bytes = KIND == KIND_F16 ? 2 * K : (KIND == KIND_I4 ? K / 2 : K);
  args.row_bytes = (int)row_bytes;

  KernelCfg cfg = BKN ? choose_config_kxn(M, N, dev.cu_count)
                : (KIND == KIND_I4_E3M2 || KIND == KIND_I8_MOD) ? choose_config_e3m2(M, N, dev.cu_count)
                                                                : choose_config(M, N, K, dev.cu_count, KIND);
  // split-K: on the automatic choice, products with few 128 x 128 tiles and
  // a long K split it when the caller gave a workspace
  constexpr bool kCanSplit = !BKN && KIND != KIND_I4_E3M2 && KIND != KIND_I8_MOD;
  const int split_nks = (int)((row_bytes + 255) / 256);
  if (kCanSplit && forced_config() < 0 && splitk_auto_splits(M, N, split_nks, dev.cu_count, KIND) > 1 &&
      splitk_launch_splits(M, N, split_nks, dev.cu_count, KIND, ws, ws_bytes) > 1)
    cfg = CFG_128_S2_R256_SPLITK;
  const int64_t stage_bytes = (KIND == KIND_I4 && expands_int4_in_lds(cfg)) ? K : row_bytes;
  const int rowb = stage_row_bytes(cfg);
  args.k_stages = (int)((stage_bytes + rowb - 1) / rowb);
  // Configuration 0 writes C with non-temporal stores, except for int4,
  // whose shorter main loop measured faster with cached stores (8192^3,
  // steady state: int8 +2%, fp16 +2%, int4 -1%); the byte stores of the
  // reduced kind go through the direct path, where the choice does not
  // apply.  On the general and K x N paths it also issues the next stage's
  // loads in its first two K-steps (int8 +1.5%, fp16 +2%).
  constexpr bool kNtC = KIND != KIND_I4 && KIND != KIND_I8_MOD;
  // ... and pins one MFMA in front of each of a K-step's loads (8192^3, one
  // MI355X: int8 2306 against 2271 TOP/s, fp16 1221 against 1182 TFLOP/s),
  // except for int4, whose expanded operands would then spill
  constexpr bool kPinLoads = KIND != KIND_I4;
  // an int4 knob (gemm_v3's I4MODE), 0 for the other kinds
  constexpr auto kI4 = [](int mode) constexpr { return KIND == KIND_I4 ? mode : 0; };

  if constexpr (BKN) {
    switch (cfg) {
      case CFG_256_S2_R128_PIN_KXN:
        return launch<256, 256>(
            (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, true, 2, true, 0, false, true>, args, 256,
            stream);
      case CFG_256_S2_R128:
        return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, true, 2, true>, args,
                                256, stream);
      case CFG_128_S4_R128:
        return launch<128, 128>((const void*)&gemm_v3<KIND, 128, 128, 4, 128, 0, false, true>, args, 256,
                                stream);
      default:
        return launch<128, 64>((const void*)&gemm_v3<KIND, 128, 64, 6, 128, 0, false, true>, args, 256,
                               stream);
    }
  } else if constexpr (KIND == KIND_I4_E3M2 || KIND == KIND_I8_MOD) {
    switch (cfg) {
      case CFG_256_S2_R128_PIN_E3M2:
        return launch<256, 256>(
            (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 0, kNtC, 0, false, true>, args, 256,
            stream);
      case CFG_256_S2_R128:
        return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 0, kNtC>, args,
                                256, stream);
      case CFG_128_S4_R128:
        return launch<128, 128>((const void*)&gemm_v3<KIND, 128, 128, 4, 128>, args, 256, stream);
      default:
        return launch<128, 64>((const void*)&gemm_v3<KIND, 128, 64, 6, 128>, args, 256, stream);
    }
  } else {
  switch (cfg) {
    case CFG_256_S2_R128:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads>, args, 256,
          stream);
    case CFG_128_S4_R128:
      return launch<128, 128>((const void*)&gemm_v3<KIND, 128, 128, 4, 128>, args, 256, stream);
    case CFG_256x128_S3_R128:
      return launch<256, 128>((const void*)&gemm_v3<KIND, 256, 128, 3, 128, 0, false, false, 0, kNtC>, args, 256, stream);
    case CFG_128x256_S3_R128:
      return launch<128, 256>((const void*)&gemm_v3<KIND, 128, 256, 3, 128, 0, false, false, 0, kNtC>, args, 256, stream);
    case CFG_256x224_S2_R128:
      return launch<256, 224>(
          (const void*)&gemm_v3<KIND, 256, 224, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads>, args, 256,
          stream);
    case CFG_256x224_S2_R128_PERSIST:
      if constexpr (KIND == KIND_I4)
        return launch<256, 224>(
            (const void*)&gemm_v3<KIND, 256, 224, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads>, args, 256,
            stream);
      else
        return launch_persistent<256, 224>(
            (const void*)&gemm_v3<KIND, 256, 224, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads, true>,
            args, 256, stream, dev.cu_count);
    case CFG_256_S2_R128_PERSIST:
      // int4 keeps configuration 0: its kernel already holds 256 VGPRs, and
      // the persistent variant's extra state would spill
      if constexpr (KIND == KIND_I4)
        return launch<256, 256>(
            (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads>, args, 256,
            stream);
      else
        return launch_persistent<256, 256>(
            (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads, true>,
            args, 256, stream, dev.cu_count);
    // int4 knobs; every other kind runs the base configuration's kernel
    case CFG_128_S2_R256_W4:
      return launch<128, 128>(
          (const void*)&gemm_v3<KIND, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, kI4(1)>,
          args, 256, stream);
    case CFG_128_S2_R256_SX:
      return launch<128, 128>(
          (const void*)&gemm_v3<KIND, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, kI4(2)>,
          args, 256, stream);
    case CFG_256_S2_R128_SX:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads, false, kI4(2)>,
          args, 256, stream);
    case CFG_128_S2_R256_BIAS:
      return launch<128, 128>(
          (const void*)&gemm_v3<KIND, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, kI4(4)>,
          args, 256, stream);
    case CFG_256_S2_R128_W4:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads, false, kI4(1)>,
          args, 256, stream);
    case CFG_256_S2_R128_PERSIST_SX:
      return launch_persistent<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads, true, kI4(2)>,
          args, 256, stream, dev.cu_count);
    case CFG_256_S2_R128_PIN_SX:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, true, false, kI4(2)>,
          args, 256, stream);
    case CFG_STREAM_128x64:
      return launch<128, 64>((const void*)&gemm_stream<KIND, 128, 64, 3, 10>, args, 320, stream);
    case CFG_STREAM_128x64_B14:
      return launch<128, 64>((const void*)&gemm_stream<KIND, 128, 64, 2, 14>, args, 320, stream);
    case CFG_STREAM_64x64:
      return launch<64, 64>((const void*)&gemm_stream<KIND, 64, 64, 3, 14>, args, 320, stream);
    case CFG_256_S2_R128_EARLY:
      // int4 keeps configuration 0 (no pinned loads, see kPinLoads)
      if constexpr (KIND == KIND_I4)
        return launch<256, 256>(
            (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, kPinLoads>, args, 256,
            stream);
      else
        return launch<256, 256>(
            (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, true, false, 0, true>,
            args, 256, stream);
    case CFG_REF:
      return launch<128, 128>((const void*)&gemm_ref<KIND>, args, 256, stream);
    case CFG_128_S2_R256_SPLITK:
      if constexpr (kCanSplit)
        return launch_split<128, 128>(
            (const void*)&gemm_v3<KIND, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, false, false, kI4(1),
                                  false, true>,
            args, 256, stream, splitk_launch_splits(M, N, args.k_stages, dev.cu_count, KIND, ws, ws_bytes), ws);
      else
        return LPGEMM_ERROR_LAUNCH;
    case CFG_256_S4_R64:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 4, 64>, args, 256, stream);
    case CFG_256_S3_R64:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 3, 64>, args, 256, stream);
    case CFG_128_S4_R64:
      return launch<128, 128>((const void*)&gemm_v3<KIND, 128, 128, 4, 64>, args, 256, stream);
    case CFG_V1_256x256:
      return launch<256, 256>((const void*)&gemm_tiled<KIND, 256, 256, 2, 4>, args, 512, stream);
    case CFG_V1_128x128:
      return launch<128, 128>((const void*)&gemm_tiled<KIND, 128, 128, 2, 2>, args, 256, stream);
    case CFG_PP_R64:
      return launch<256, 256>((const void*)&gemm_pingpong<KIND, 64>, args, 512, stream);
    case CFG_SKINNY_32:
      return launch<32, 32>((const void*)&gemm_skinny<KIND, 1, 8, 4>, args, 512, stream);
    case CFG_SKINNY_64:
      return launch<64, 32>((const void*)&gemm_skinny<KIND, 2, 8, 2>, args, 512, stream);
    case CFG_SKINNY_32_W16:
      return launch<32, 32>((const void*)&gemm_skinny<KIND, 1, 16, 2>, args, 1024, stream);
    case CFG_SKINNY_LDS_R2:
      return launch<32, 32>((const void*)&gemm_skinny_lds<KIND, 8, 2>, args, 512, stream);
    case CFG_SKINNY_LDS_R4:
      return launch<32, 32>((const void*)&gemm_skinny_lds<KIND, 8, 4>, args, 512, stream);
    case CFG_SKINNY_LDS_W4:
      return launch<32, 32>((const void*)&gemm_skinny_lds<KIND, 4, 4>, args, 256, stream);
    case CFG_SKINNY_PIPE_W4R2: {
      // the automatic choice's even column share for a single 32-row band
      // (forced, or more rows: 32 columns)
      const int w = forced_config() < 0 && M <= 32 ? skinny_columns(N, dev.cu_count, 1) : 0;
      return launch_skinny((const void*)&gemm_skinny_pipe<KIND, 4, 2, false, 1, 1>, args, 256, stream, w > 0 ? w : 32);
    }
    case CFG_SKINNY_PIPE_W4R2_N2: {
      const int w = skinny_columns(N, dev.cu_count, 2);
      return launch_skinny((const void*)&gemm_skinny_pipe<KIND, 4, 2, false, 2>, args, 256, stream, w > 0 ? w : 64);
    }
    case CFG_SKINNY_PIPE_W8R1: {
      // as configuration 14 (int4's choice at M <= 32)
      const int w = forced_config() < 0 && M <= 32 ? skinny_columns(N, dev.cu_count, 1) : 0;
      return launch_skinny((const void*)&gemm_skinny_pipe<KIND, 8, 1>, args, 512, stream, w > 0 ? w : 32);
    }
    case CFG_SKINNY_PIPE_W4R3:
      return launch<32, 32>((const void*)&gemm_skinny_pipe<KIND, 4, 3>, args, 256, stream);
    case CFG_SKINNY_PIPE_W8R2:
      return launch<32, 32>((const void*)&gemm_skinny_pipe<KIND, 8, 2>, args, 512, stream);
    case CFG_128x64_S4_R64:
      return launch<128, 64>((const void*)&gemm_v3<KIND, 128, 64, 4, 64>, args, 256, stream);
    case CFG_256x128_S4_R64:
      return launch<256, 128>((const void*)&gemm_v3<KIND, 256, 128, 4, 64>, args, 256, stream);
    case CFG_128x64_S6_R128:
      return launch<128, 64>((const void*)&gemm_v3<KIND, 128, 64, 6, 128>, args, 256, stream);
    case CFG_128x64_S8_R64:
      return launch<128, 64>((const void*)&gemm_v3<KIND, 128, 64, 8, 64>, args, 256, stream);
    case CFG_128x64_S3_R256:
      // one row band (M <= 128): every B element is read by one workgroup,
      // so B streams non-temporally (graph-timed, one MI355X, weights from
      // HBM: LLM M = 128 17.83 against 18.55 us, fp16 128 x 14336 x 4096
      // 30.0 against 31.2, int8 128 x 8192 x 8192 26.6 against 29.6; with
      // the weights in the Infinity Cache 3-16% slower; above 128 rows B is
      // re-read by every row band and keeps the default policy)
      if (M <= 128)
        return launch<128, 64>((const void*)&gemm_v3<KIND, 128, 64, 3, 256, 5>, args, 256, stream);
      return launch<128, 64>((const void*)&gemm_v3<KIND, 128, 64, 3, 256>, args, 256, stream);
    case CFG_128_S5_R128:
      return launch<128, 128>((const void*)&gemm_v3<KIND, 128, 128, 5, 128>, args, 256, stream);
    case CFG_128_S2_R256:
      return launch<128, 128>((const void*)&gemm_v3<KIND, 128, 128, 2, 256>, args, 256, stream);
    case CFG_128_S2_R256_PIN:
      return launch<128, 128>(
          (const void*)&gemm_v3<KIND, 128, 128, 2, 256, 0, false, false, 0, false, 0, false, kPinLoads>, args, 256,
          stream);
    case CFG_128_S4_R128_PIN:
      return launch<128, 128>(
          (const void*)&gemm_v3<KIND, 128, 128, 4, 128, 0, false, false, 0, false, 0, false, kPinLoads>, args, 256,
          stream);
    case CFG_128x64_S3_R256_PIN:
      return launch<128, 64>(
          (const void*)&gemm_v3<KIND, 128, 64, 3, 256, 0, false, false, 0, false, 0, false, kPinLoads>, args, 256,
          stream);
    case CFG_256_S2_R128_PIN_L1:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 1, kNtC, 0, false, kPinLoads>, args, 256,
          stream);
    case CFG_256_S2_R128_PIN_L3:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 3, kNtC, 0, false, kPinLoads>, args, 256,
          stream);
    case CFG_256_S2_R128_PIN_I4:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, true>, args, 256,
          stream);
    case CFG_256_S2_R128_SCHED:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, false, false>, args, 256,
          stream);
    case CFG_256_S2_R128_PF:
      return launch<256, 256>(
          (const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 0, true>, args, 256, stream);
    case CFG_256_S2_R128_NT:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 1>, args, 256, stream);
    case CFG_256_S2_R128_SC0:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 2>, args, 256, stream);
    case CFG_256_S2_R128_SC01:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 4>, args, 256, stream);
    case CFG_256_S2_R128_SPLIT:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, true>, args, 256, stream);
    case CFG_256_S2_R128_L1:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 1>, args, 256,
                              stream);
    case CFG_256_S2_R128_CACHED_C:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, false>, args,
                              256, stream);
    case CFG_256_S2_R128_B4:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 4>, args,
                              256, stream);
    case CFG_256_S2_R128_B12:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128, 0, false, false, 2, kNtC, 12>, args,
                              256, stream);
    case CFG_256_S5_R64_NT:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 5, 64, 0, false, false, 0, kNtC>, args, 256,
                              stream);
    case CFG_256_S4_R64_NT:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 4, 64, 0, false, false, 0, kNtC>, args, 256,
                              stream);
    case CFG_256_S2_R128_LALL:
      return launch<256, 256>((const void*)&gemm_v3<KIND, 256, 256, 2, 128>, args, 256, stream);
    case CFG_V1_64x64:
      return launch<64, 64>((const void*)&gemm_tiled<KIND, 64, 64, 2, 2>, args, 256, stream);
    default:
      // every configuration the choosers can return has a case above; the
      // stage count was derived from the configuration, so no other kernel
      // may stand in for one
      return LPGEMM_ERROR_INVALID_VALUE;
  }
  }
}

}  // namespace lpgemm
