// Host side of liblpgemm: the C-ABI entry points declared in include/lpgemm.h.
//
// Each call validates its arguments on the host (no HIP call before that),
// checks once per device that the device is gfx950, picks a tile
// configuration for the shape, and enqueues one kernel on the caller's
// stream.  Nothing is allocated and no state is kept between calls apart from
// the per-device property cache.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/lpgemm.h"
#include "f64emu_kernels.hpp"
#include "gemm_kernels.hpp"

namespace lpgemm {
namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  bool probed = false;
  bool is_gfx950 = false;
  int cu_count = 0;
};

std::mutex g_device_mutex;
DeviceInfo g_devices[kMaxDevices];

// Current device's properties, read once per device.
lpgemm_status current_device(DeviceInfo& out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LPGEMM_ERROR_ARCH;
  std::lock_guard<std::mutex> lock(g_device_mutex);
  DeviceInfo& d = g_devices[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LPGEMM_ERROR_ARCH;
    d.is_gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cu_count = prop.multiProcessorCount;
    d.probed = true;
  }
  out = d;
  return d.is_gfx950 ? LPGEMM_SUCCESS : LPGEMM_ERROR_ARCH;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Host-only argument checks, in the order the header documents.  Sets
// `nothing_to_do` when the product is empty (M or N is zero).
lpgemm_status validate(Kind kind, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                       const void* C, const void* rs, const void* cs, bool& nothing_to_do) {
  nothing_to_do = false;
  if (M < 0 || N < 0 || K < 0) return LPGEMM_ERROR_INVALID_VALUE;
  if (M > INT32_MAX || N > INT32_MAX) return LPGEMM_ERROR_INVALID_VALUE;
  switch (kind) {
    case KIND_I8:
    case KIND_I8_DEQUANT:
    case KIND_I8_MOD:
      if (K % 16 != 0 || K > LPGEMM_MAX_K_INT) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
      break;
    case KIND_I4:
    case KIND_I4_E3M2:
      if (K % 32 != 0 || K > LPGEMM_MAX_K_INT) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
      break;
    case KIND_F16:
      if (K % 8 != 0 || K > LPGEMM_MAX_K_F16) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
      break;
  }
  if (M == 0 || N == 0) {
    nothing_to_do = true;
    return LPGEMM_SUCCESS;
  }
  if (!C) return LPGEMM_ERROR_INVALID_VALUE;
  if (K > 0 && (!A || !B)) return LPGEMM_ERROR_INVALID_VALUE;
  if (kind == KIND_I8_DEQUANT && (!rs || !cs)) return LPGEMM_ERROR_INVALID_VALUE;
  if (!aligned16(C)) return LPGEMM_ERROR_MISALIGNED;
  if (K > 0 && (!aligned16(A) || !aligned16(B))) return LPGEMM_ERROR_MISALIGNED;
  if (kind == KIND_I8_DEQUANT && (!aligned4(rs) || !aligned4(cs))) return LPGEMM_ERROR_MISALIGNED;
  return LPGEMM_SUCCESS;
}

// Kernel configurations.  The four-wave direct-to-LDS kernel with 256 x 256
// tiles has the best operand reuse; smaller tiles fill the 256 CUs when the
// product has few 256 x 256 tiles.
enum KernelCfg {
  CFG_256_S2_R128 = 0,   // 4 waves, 256 x 256, 2 stages of 128-byte rows (see kNtC)
  CFG_256_S4_R64 = 1,    // 4 waves, 256 x 256, 4 stages of 64-byte rows
  CFG_256_S3_R64 = 2,    // 4 waves, 256 x 256, 3 stages of 64-byte rows
  CFG_128_S4_R64 = 3,    // 4 waves, 128 x 128, 4 stages of 64-byte rows
  CFG_V1_256x256 = 4,    // 8 waves, 128 x 64 per wave, register-staged loads
  CFG_V1_128x128 = 5,    // 4 waves, 64 x 64 per wave, register-staged loads
  CFG_V1_64x64 = 6,      // 4 waves, 32 x 32 per wave, register-staged loads
  CFG_PP_R64 = 7,        // 8 waves ping-pong, 256 x 256, 4 stages of 64-byte rows
  CFG_SKINNY_32 = 8,     // 32 x 32 tiles, 8 waves split K, 4 K-blocks per load round
  CFG_SKINNY_64 = 9,     // 64 x 32 tiles, 8 waves split K, 2 K-blocks per load round
  CFG_SKINNY_32_W16 = 10,  // 32 x 32 tiles, 16 waves split K, 2 K-blocks per load round
  CFG_SKINNY_LDS_R2 = 11,  // 32 x 32 tiles, 8 waves split K, B through LDS, 2 K-blocks per round
  CFG_SKINNY_LDS_R4 = 12,  // 32 x 32 tiles, 8 waves split K, B through LDS, 4 K-blocks per round
  CFG_SKINNY_LDS_W4 = 13,  // 32 x 32 tiles, 4 waves split K, B through LDS, 4 K-blocks per round
  CFG_SKINNY_PIPE_W4R2 = 14,  // as 13, double-buffered rounds of 2 K-blocks
  CFG_SKINNY_PIPE_W8R1 = 15,  // 8 waves, double-buffered rounds of 1 K-block
  CFG_SKINNY_PIPE_W4R3 = 16,  // 4 waves, double-buffered rounds of 3 K-blocks
  CFG_SKINNY_PIPE_W8R2 = 17,  // 8 waves, double-buffered rounds of 2 K-blocks
  CFG_128x64_S4_R64 = 18,     // 4 waves, 128 x 64, 4 stages of 64-byte rows
  CFG_256x128_S4_R64 = 19,    // 4 waves, 256 x 128, 4 stages of 64-byte rows
  CFG_128x64_S6_R128 = 20,    // 4 waves, 128 x 64, 6 stages of 128-byte rows
  CFG_128x64_S8_R64 = 21,     // 4 waves, 128 x 64, 8 stages of 64-byte rows
  CFG_128_S4_R128 = 22,       // 4 waves, 128 x 128, 4 stages of 128-byte rows
  // ablations of configuration 0
  CFG_256_S2_R128_NT = 23,       // operand loads non-temporal (nt)
  CFG_256_S2_R128_SC0 = 24,      // operand loads sc0
  CFG_256_S2_R128_SC01 = 25,     // operand loads sc0 sc1
  CFG_256_S2_R128_SPLIT = 26,    // split loader: two waves load A, two load B
  CFG_256_S2_R128_L1 = 27,       // the next stage's loads all issued in K-step 0
  CFG_256_S2_R128_LALL = 28,     // ... spread over all K-steps but the last
  CFG_256_S2_R128_CACHED_C = 29, // C written with ordinary (cached) stores
  CFG_256_S2_R128_B4 = 30,       // stage barrier after 4 of the last K-step's 16 MFMAs
  CFG_256_S2_R128_B12 = 31,      // ... after 12
  CFG_256_S5_R64_NT = 32,        // 4 waves, 256 x 256, 5 stages of 64-byte rows (all 160 KiB), NT C
  CFG_256_S4_R64_NT = 33,        // 4 waves, 256 x 256, 4 stages of 64-byte rows, NT C
  CFG_128x64_S3_R256 = 34,       // 4 waves, 128 x 64, 3 stages of 256-byte rows
  CFG_128_S5_R128 = 35,          // 4 waves, 128 x 128, 5 stages of 128-byte rows (all 160 KiB)
  CFG_128_S2_R256 = 36,          // 4 waves, 128 x 128, 2 stages of 256-byte rows
  CFG_256_S2_R128_PF = 37,       // configuration 0 plus an L2 prefetch of the stage after next
  CFG_256_S2_R128_SCHED = 38,    // configuration 0 with the loads placed by the compiler's schedule
  CFG_128_S2_R256_PIN = 39,      // configuration 36 with one MFMA pinned in front of each load
  CFG_128_S4_R128_PIN = 40,      // configuration 22 with one MFMA pinned in front of each load
  CFG_128x64_S3_R256_PIN = 41,   // configuration 34 with one MFMA pinned in front of each load
  CFG_256_S2_R128_PIN_L1 = 42,   // configuration 0 with all of a stage's loads pinned in K-step 0
  CFG_256_S2_R128_PIN_L3 = 43,   // configuration 0 with the loads pinned over K-steps 0-2
  CFG_256_S2_R128_PIN_I4 = 44,   // configuration 0 with pinned loads also for int4
  CFG_256_S2_R128_PIN_E3M2 = 45, // E3M2 on configuration 0 with one MFMA pinned in front of each load
  CFG_256_S2_R128_PIN_KXN = 46,  // K x N B on configuration 0 with one MFMA pinned in front of each load
  CFG_COUNT = 47
};

// Row bytes of one LDS K-stage for a configuration (the register-staged
// kernels expand int4 to int8 on the way into LDS, 128 values per stage).
int stage_row_bytes(KernelCfg c) {
  return (c == CFG_256_S4_R64 || c == CFG_256_S3_R64 || c == CFG_128_S4_R64 || c == CFG_PP_R64 ||
          c == CFG_128x64_S4_R64 || c == CFG_256x128_S4_R64 || c == CFG_128x64_S8_R64 ||
          c == CFG_256_S5_R64_NT || c == CFG_256_S4_R64_NT)
             ? 64
             : ((c == CFG_128x64_S3_R256 || c == CFG_128_S2_R256) ? 256 : 128);
}
bool expands_int4_in_lds(KernelCfg c) { return c >= CFG_V1_256x256 && c <= CFG_V1_64x64; }
bool is_skinny(KernelCfg c) { return c >= CFG_SKINNY_32 && c <= CFG_SKINNY_PIPE_W8R2; }

int tiles(int64_t x, int t) { return (int)((x + t - 1) / t); }

// LPGEMM_FORCE_CONFIG=<n> pins the kernel configuration (one knob at a time
// for ablations); unset or out of range means automatic selection.  Read on
// every call so that a test can walk through the configurations.
int forced_config() {
  const char* e = std::getenv("LPGEMM_FORCE_CONFIG");
  if (!e || !*e) return -1;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  return (end && *end == 0 && v >= 0 && v < CFG_COUNT) ? (int)v : -1;
}

// The E3M2 kind runs only on the LDS-pipelined kernels with 128-byte stage
// rows (two 64-value MFMA steps per stage); the reduced int8 kind of the
// fp64 emulation uses the same three.
bool supports_e3m2(int c) {
  return c == CFG_256_S2_R128 || c == CFG_128x64_S6_R128 || c == CFG_128_S4_R128 || c == CFG_256_S2_R128_PIN_E3M2;
}

KernelCfg choose_config_e3m2(int64_t M, int64_t N, int cu_count) {
  const int f = forced_config();
  if (f >= 0 && supports_e3m2(f)) return (KernelCfg)f;
  if (M <= 128) return CFG_128x64_S6_R128;
  if ((int64_t)tiles(M, 256) * tiles(N, 256) >= cu_count) return CFG_256_S2_R128;
  if ((int64_t)tiles(M, 128) * tiles(N, 128) >= cu_count / 2) return CFG_128_S4_R128;
  return CFG_128x64_S6_R128;
}

KernelCfg choose_config(int64_t M, int64_t N, int cu_count, int kind) {
  const int f = forced_config();
  // configurations 45 and 46 differ from 0 only for the E3M2 kind and for
  // K x N B
  if (f == CFG_256_S2_R128_PIN_E3M2 || f == CFG_256_S2_R128_PIN_KXN) return CFG_256_S2_R128;
  if (f >= 0) return (KernelCfg)f;
  const bool int8_rows = kind == KIND_I8 || kind == KIND_I8_DEQUANT;
  // few rows against many columns: stream B with split-K workgroups
  if (M <= 32) return CFG_SKINNY_PIPE_W4R2;
  if (M <= 64) return CFG_SKINNY_64;
  // a 128-row band: 128 x 64 tiles double the workgroups of 128 x 128.
  // int8 rows stream B in 256-byte pieces per stage (M = 128, K = 4096,
  // N = 14336: 19.2 us against 20.4 us with six 128-byte stages)
  if (M <= 128) return int8_rows ? CFG_128x64_S3_R256 : CFG_128x64_S6_R128;
  const int64_t big = (int64_t)tiles(M, 256) * tiles(N, 256);
  if (big >= cu_count) return CFG_256_S2_R128;
  // 128 x 128 tiles: at 2048^3, two 256-byte stages for int8 and int4
  // (14.5 / 15.0 us against 15.4 / 15.7 us with four 64-byte stages), four
  // 128-byte stages for fp16 (23.1 against 25.4 us)
  const int64_t mid = (int64_t)tiles(M, 128) * tiles(N, 128);
  if (mid >= cu_count / 2) return kind == KIND_F16 ? CFG_128_S4_R128 : CFG_128_S2_R256;
  return CFG_V1_64x64;
}

template <int BM, int BN>
lpgemm_status launch(const void* fn, GemmArgs args, int threads, hipStream_t stream) {
  args.tiles_m = tiles(args.M, BM);
  args.tiles_n = tiles(args.N, BN);
  args.group_m = 8;
  const int64_t nblocks = (int64_t)args.tiles_m * args.tiles_n;
  if (nblocks > INT32_MAX) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nblocks), dim3(threads), kargs, 0, stream);
  return e == hipSuccess ? LPGEMM_SUCCESS : LPGEMM_ERROR_LAUNCH;
}

// B stored K x N row-major runs on the LDS-pipelined kernels with 128-byte
// stage rows: 128 k-rows of B per stage.
bool supports_kxn(int c) {
  return c == CFG_256_S2_R128 || c == CFG_128x64_S6_R128 || c == CFG_128_S4_R128 || c == CFG_256_S2_R128_PIN_KXN;
}

KernelCfg choose_config_kxn(int64_t M, int64_t N, int cu_count) {
  const int f = forced_config();
  if (f >= 0 && supports_kxn(f)) return (KernelCfg)f;
  if (M <= 128) return CFG_128x64_S6_R128;
  if ((int64_t)tiles(M, 256) * tiles(N, 256) >= cu_count) return CFG_256_S2_R128;
  if ((int64_t)tiles(M, 128) * tiles(N, 128) >= cu_count / 2) return CFG_128_S4_R128;
  return CFG_128x64_S6_R128;
}

template <int KIND, bool BKN = false>
lpgemm_status run(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C,
                  const float* rs, const float* cs, hipStream_t stream, int modulus = 0) {
  // K x N B: k-rows of N bytes must start 16-byte aligned and the matrix
  // must fit the 32-bit offsets of its buffer resource (a shape error, so it
  // ranks with the K checks: after negative sizes, before pointers)
  if (BKN && M > 0 && N > 0 && K >= 0 && M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX &&
      (N % 16 != 0 || K * N >= ((int64_t)1 << 31)))
    return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  bool nothing_to_do = false;
  lpgemm_status st = validate((Kind)KIND, M, N, K, A, B, C, rs, cs, nothing_to_do);
  if (st != LPGEMM_SUCCESS || nothing_to_do) return st;
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

  const KernelCfg cfg = BKN ? choose_config_kxn(M, N, dev.cu_count)
                      : (KIND == KIND_I4_E3M2 || KIND == KIND_I8_MOD) ? choose_config_e3m2(M, N, dev.cu_count)
                                             : choose_config(M, N, dev.cu_count, KIND);
  const int64_t stage_bytes = (KIND == KIND_I4 && expands_int4_in_lds(cfg)) ? K : row_bytes;
  (void)is_skinny;
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
    case CFG_SKINNY_PIPE_W4R2:
      return launch<32, 32>((const void*)&gemm_skinny_pipe<KIND, 4, 2>, args, 256, stream);
    case CFG_SKINNY_PIPE_W8R1:
      return launch<32, 32>((const void*)&gemm_skinny_pipe<KIND, 8, 1>, args, 512, stream);
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

}  // namespace
}  // namespace lpgemm

using namespace lpgemm;

namespace {

// fp64 emulation: the moduli, largest first (pairwise coprime)
constexpr int kF64Moduli[kF64MaxModuli] = {256, 255, 253, 251, 247, 241, 239, 233, 229, 227,
                                           223, 217, 211, 199, 197, 193, 191, 181, 179, 173};

struct U192h {
  uint64_t w[3];
};
void u192h_mul_small(U192h& a, uint32_t v) {
  unsigned __int128 carry = 0;
  for (int i = 0; i < 3; ++i) {
    const unsigned __int128 t = (unsigned __int128)a.w[i] * v + carry;
    a.w[i] = (uint64_t)t;
    carry = t >> 64;
  }
}
bool u192h_gt(const U192h& a, const U192h& b) {
  for (int i = 2; i >= 0; --i)
    if (a.w[i] != b.w[i]) return a.w[i] > b.w[i];
  return false;
}
U192h u192h_shl(uint64_t x, int sh) {   // x << sh, sh < 192
  U192h r{{0, 0, 0}};
  const int limb = sh / 64, bit = sh % 64;
  r.w[limb] = x << bit;
  if (bit && limb + 1 < 3) r.w[limb + 1] = x >> (64 - bit);
  return r;
}
int mod_inverse(int a, int m) {   // a^-1 mod m, gcd(a, m) = 1
  int t = 0, nt = 1, r = m, nr = a % m;
  while (nr) {
    const int q = r / nr;
    int x = t - q * nt; t = nt; nt = x;
    x = r - q * nr; r = nr; nr = x;
  }
  return t < 0 ? t + m : t;
}

// Moduli needed so that their product P exceeds 2 K 2^(2 bits); -1 if the
// twenty available are not enough.
int f64emu_moduli(int64_t K, int bits) {
  const U192h bound = u192h_shl((uint64_t)(K > 0 ? K : 1), 2 * bits + 1);
  U192h P{{1, 0, 0}};
  for (int s = 1; s <= kF64MaxModuli; ++s) {
    u192h_mul_small(P, (uint32_t)kF64Moduli[s - 1]);
    if (u192h_gt(P, bound)) return s;
  }
  return -1;
}

// 192-bit value divided by a small integer (long division), and its
// remainder
U192h u192h_div_small(const U192h& a, uint32_t d, uint32_t* rem) {
  U192h q{{0, 0, 0}};
  unsigned __int128 r = 0;
  for (int i = 2; i >= 0; --i) {
    const unsigned __int128 cur = (r << 64) | a.w[i];
    q.w[i] = (uint64_t)(cur / d);
    r = cur % d;
  }
  if (rem) *rem = (uint32_t)r;
  return q;
}

F64EmuConsts f64emu_consts(int s, int bits) {
  F64EmuConsts c{};
  c.s = s;
  c.bits = bits;
  U192h P{{1, 0, 0}};
  for (int l = 0; l < s; ++l) u192h_mul_small(P, (uint32_t)kF64Moduli[l]);
  for (int l = 0; l < s; ++l) {
    const int m = kF64Moduli[l];
    c.m[l] = m;
    c.inv_m[l] = 1.0 / (double)m;
    c.inv_mf[l] = 1.0f / (float)m;
    const U192h Ml = u192h_div_small(P, (uint32_t)m, nullptr);   // exact: m divides P
    for (int i = 0; i < 3; ++i) c.big_m[l][i] = Ml.w[i];
    uint32_t ml_mod = 0;
    u192h_div_small(Ml, (uint32_t)m, &ml_mod);
    c.crt_c[l] = mod_inverse((int)ml_mod, m);
  }
  for (int i = 0; i < 3; ++i) c.p[i] = P.w[i];
  c.p_half[0] = (P.w[0] >> 1) | (P.w[1] << 63);
  c.p_half[1] = (P.w[1] >> 1) | (P.w[2] << 63);
  c.p_half[2] = P.w[2] >> 1;
  return c;
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// the residue and reconstruction kernels, instantiated per modulus count
template <int... S>
struct F64EmuKernels {
  static const void* residues(int s) {
    static const void* const table[] = {(const void*)&f64_residues<S>...};
    return table[s - 1];
  }
  static const void* crt(int s) {
    static const void* const table[] = {(const void*)&f64_crt<S>...};
    return table[s - 1];
  }
};
using F64EmuTable = F64EmuKernels<1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20>;
static_assert(kF64MaxModuli == 20, "one kernel per modulus count");

// Workspace layout: eA (M int), eB (N int), residues of A (s M K int8),
// residues of B (s N K int8), the s reduced products (M N bytes each, every
// one starting 256-byte aligned), each region 256-byte aligned.
struct F64EmuLayout {
  int64_t ea, eb, ra, rb, cl, total;
};
F64EmuLayout f64emu_layout(int64_t M, int64_t N, int64_t K, int s) {
  F64EmuLayout L{};
  L.ea = 0;
  L.eb = L.ea + align256(4 * M);
  L.ra = L.eb + align256(4 * N);
  L.rb = L.ra + align256((int64_t)s * M * K);
  L.cl = L.rb + align256((int64_t)s * N * K);
  L.total = L.cl + (int64_t)s * align256(M * N);
  return L;
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace

extern "C" {

lpgemm_status lpgemm_i8(int64_t M, int64_t N, int64_t K, const int8_t* A, const int8_t* B,
                        int32_t* C, hipStream_t stream) {
  return run<KIND_I8>(M, N, K, A, B, C, nullptr, nullptr, stream);
}

lpgemm_status lpgemm_i4(int64_t M, int64_t N, int64_t K, const uint8_t* A_packed,
                        const uint8_t* B_packed, int32_t* C, hipStream_t stream) {
  return run<KIND_I4>(M, N, K, A_packed, B_packed, C, nullptr, nullptr, stream);
}

int lpgemm_f64_emu_moduli(int64_t K, int bits) {
  if (K < 0 || bits < 1 || bits > 53) return -1;
  return f64emu_moduli(K, bits);
}

int64_t lpgemm_f64_emu_workspace(int64_t M, int64_t N, int64_t K, int bits) {
  if (M < 0 || N < 0 || K < 0 || bits < 1 || bits > 53) return -1;
  const int s = f64emu_moduli(K, bits);
  if (s < 0) return -1;
  return f64emu_layout(M, N, K, s).total;
}

lpgemm_status lpgemm_f64_emu(int64_t M, int64_t N, int64_t K, const double* A, const double* B,
                             double* C, int bits, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX) return LPGEMM_ERROR_INVALID_VALUE;
  if (bits < 1 || bits > 53) return LPGEMM_ERROR_INVALID_VALUE;
  if (K % 16 != 0 || K > LPGEMM_MAX_K_INT) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return LPGEMM_SUCCESS;
  if (!C || !workspace) return LPGEMM_ERROR_INVALID_VALUE;
  if (K > 0 && (!A || !B)) return LPGEMM_ERROR_INVALID_VALUE;
  const int s = f64emu_moduli(K, bits);
  if (s < 0) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  const F64EmuLayout L = f64emu_layout(M, N, K, s);
  if (workspace_bytes < L.total) return LPGEMM_ERROR_INVALID_VALUE;
  if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B))) ||
      ((uintptr_t)workspace & 255) != 0)
    return LPGEMM_ERROR_MISALIGNED;
  DeviceInfo dev;
  lpgemm_status st = current_device(dev);
  if (st != LPGEMM_SUCCESS) return st;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int* eA = reinterpret_cast<int*>(ws + L.ea);
  int* eB = reinterpret_cast<int*>(ws + L.eb);
  int8_t* RA = reinterpret_cast<int8_t*>(ws + L.ra);
  int8_t* RB = reinterpret_cast<int8_t*>(ws + L.rb);
  uint8_t* CR = ws + L.cl;
  const F64EmuConsts c = f64emu_consts(s, bits);
  int k32 = (int)K;
  hipError_t e = hipSuccess;

  // scale / exponent scan of the rows of A and of B (K-contiguous)
  {
    void* a1[] = {&A, &k32, &eA};
    e = hipLaunchKernel((const void*)&f64_row_exponent, dim3((unsigned)M), dim3(256), a1, 0, stream);
    if (e != hipSuccess) return LPGEMM_ERROR_LAUNCH;
    void* a2[] = {&B, &k32, &eB};
    e = hipLaunchKernel((const void*)&f64_row_exponent, dim3((unsigned)N), dim3(256), a2, 0, stream);
    if (e != hipSuccess) return LPGEMM_ERROR_LAUNCH;
  }
  // residue quantisation (eight values per thread)
  if (K > 0) {
    int64_t ta = M * K, tb = N * K;
    F64EmuConsts cc = c;
    void* a1[] = {&A, &eA, &ta, &k32, &RA, &cc};
    e = hipLaunchKernel(F64EmuTable::residues(s), dim3(grid_for(ta / 8)), dim3(256), a1, 0, stream);
    if (e != hipSuccess) return LPGEMM_ERROR_LAUNCH;
    void* a2[] = {&B, &eB, &tb, &k32, &RB, &cc};
    e = hipLaunchKernel(F64EmuTable::residues(s), dim3(grid_for(tb / 8)), dim3(256), a2, 0, stream);
    if (e != hipSuccess) return LPGEMM_ERROR_LAUNCH;
  }
  // one exact int8 GEMM per modulus, its epilogue reducing modulo m
  const int64_t cr_stride = align256(M * N);   // bytes between products
  for (int l = 0; l < s; ++l) {
    st = run<KIND_I8_MOD>(M, N, K, RA + (size_t)l * M * K, RB + (size_t)l * N * K, CR + (size_t)l * cr_stride,
                          nullptr, nullptr, stream, c.m[l]);
    if (st != LPGEMM_SUCCESS) return st;
  }
  // mod reduction, CRT reconstruction, undo scaling, write double
  {
    int64_t mn = M * N;
    int n32 = (int)N;
    F64EmuConsts cc = c;
    int64_t stride = cr_stride;
    void* a[] = {&CR, &stride, &mn, &n32, &eA, &eB, &C, &cc};
    e = hipLaunchKernel(F64EmuTable::crt(s), dim3(grid_for(mn)), dim3(256), a, 0, stream);
    if (e != hipSuccess) return LPGEMM_ERROR_LAUNCH;
  }
  return LPGEMM_SUCCESS;
}

lpgemm_status lpgemm_i8_kxn(int64_t M, int64_t N, int64_t K, const int8_t* A, const int8_t* B_kxn,
                            int32_t* C, hipStream_t stream) {
  return run<KIND_I8, true>(M, N, K, A, B_kxn, C, nullptr, nullptr, stream);
}

lpgemm_status lpgemm_i4_to_e3m2(int64_t rows, int64_t K, const uint8_t* src_packed, uint8_t* dst,
                                hipStream_t stream) {
  if (rows < 0 || K < 0) return LPGEMM_ERROR_INVALID_VALUE;
  if (K % 32 != 0 || K > LPGEMM_MAX_K_INT) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  if (rows == 0 || K == 0) return LPGEMM_SUCCESS;
  if (!src_packed || !dst) return LPGEMM_ERROR_INVALID_VALUE;
  if (!aligned16(src_packed) || !aligned16(dst)) return LPGEMM_ERROR_MISALIGNED;
  DeviceInfo dev;
  lpgemm_status st = current_device(dev);
  if (st != LPGEMM_SUCCESS) return st;
  int64_t groups = rows * (K / 32);   // 32 values: 16 bytes in, 32 bytes out
  const int64_t blocks = (groups + 255) / 256;
  if (blocks > INT32_MAX) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  void* kargs[] = {&src_packed, &dst, &groups};
  hipError_t e = hipLaunchKernel((const void*)&pack_i4_e3m2, dim3((unsigned)blocks), dim3(256), kargs, 0,
                                 stream);
  return e == hipSuccess ? LPGEMM_SUCCESS : LPGEMM_ERROR_LAUNCH;
}

lpgemm_status lpgemm_i4_e3m2(int64_t M, int64_t N, int64_t K, const uint8_t* A_e3m2,
                             const uint8_t* B_e3m2, int32_t* C, hipStream_t stream) {
  return run<KIND_I4_E3M2>(M, N, K, A_e3m2, B_e3m2, C, nullptr, nullptr, stream);
}

lpgemm_status lpgemm_f16(int64_t M, int64_t N, int64_t K, const void* A, const void* B, float* C,
                         hipStream_t stream) {
  return run<KIND_F16>(M, N, K, A, B, C, nullptr, nullptr, stream);
}

lpgemm_status lpgemm_i8_dequant(int64_t M, int64_t N, int64_t K, const int8_t* A,
                                const int8_t* B, const float* row_scale, const float* col_scale,
                                float* C, hipStream_t stream) {
  return run<KIND_I8_DEQUANT>(M, N, K, A, B, C, row_scale, col_scale, stream);
}

lpgemm_status lpgemm_w8a8_fused(int64_t M, int64_t N, int64_t K, const void* X, const int8_t* W,
                                const float* w_scale, float* C, hipStream_t stream) {
  // the dequantising product's checks, with w_scale in both scale slots (the
  // row scales are the kernel's own)
  bool nothing_to_do = false;
  lpgemm_status st = validate(KIND_I8_DEQUANT, M, N, K, X, W, C, w_scale, w_scale, nothing_to_do);
  if (st != LPGEMM_SUCCESS) return st;
  if (M > LPGEMM_W8A8_FUSED_MAX_M) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  if (nothing_to_do) return LPGEMM_SUCCESS;
  DeviceInfo dev;
  st = current_device(dev);
  if (st != LPGEMM_SUCCESS) return st;
  GemmArgs args{};
  args.A = static_cast<const uint8_t*>(X);
  args.B = reinterpret_cast<const uint8_t*>(W);
  args.C = C;
  args.row_scale = nullptr;
  args.col_scale = w_scale;
  args.M = (int)M;
  args.N = (int)N;
  args.row_bytes = (int)K;   // of the int8 operand; the binary16 rows are twice as long
  args.k_stages = (int)((K + 127) / 128);
  return launch<32, 32>((const void*)&gemm_skinny_pipe<KIND_I8_DEQUANT, 4, 1, true>, args, 256, stream);
}

lpgemm_status lpgemm_quantize_rows_f16(int64_t M, int64_t K, const void* X, int8_t* Q,
                                       float* row_scale, hipStream_t stream) {
  if (M < 0 || K < 0 || M > INT32_MAX) return LPGEMM_ERROR_INVALID_VALUE;
  if (K % 8 != 0 || K > LPGEMM_MAX_K_QUANT) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  if (M == 0) return LPGEMM_SUCCESS;
  if (!row_scale) return LPGEMM_ERROR_INVALID_VALUE;
  if (K > 0 && (!X || !Q)) return LPGEMM_ERROR_INVALID_VALUE;
  if (!aligned4(row_scale)) return LPGEMM_ERROR_MISALIGNED;
  if (K > 0 && (!aligned16(X) || !aligned16(Q))) return LPGEMM_ERROR_MISALIGNED;
  DeviceInfo dev;
  lpgemm_status st = current_device(dev);
  if (st != LPGEMM_SUCCESS) return st;
  const uint8_t* x = static_cast<const uint8_t*>(X);
  int m = (int)M, k = (int)K;
  hipError_t e;
  if (K > 0 && K <= 8192) {
    // rows held in registers: a whole workgroup per row while there are
    // fewer rows than SIMDs, one wavefront per row beyond that
    const bool wide = M < 4 * (int64_t)dev.cu_count;
    const int per_lane = (int)((K / 8 + (wide ? 255 : 63)) / (wide ? 256 : 64));
    const void* fn;
    if (wide) {
      fn = per_lane <= 1 ? (const void*)&quantize_rows_f16_regs<4, 1>
         : per_lane <= 2 ? (const void*)&quantize_rows_f16_regs<4, 2>
                         : (const void*)&quantize_rows_f16_regs<4, 4>;
    } else {
      fn = per_lane <= 1 ? (const void*)&quantize_rows_f16_regs<1, 1>
         : per_lane <= 2 ? (const void*)&quantize_rows_f16_regs<1, 2>
         : per_lane <= 4 ? (const void*)&quantize_rows_f16_regs<1, 4>
         : per_lane <= 8 ? (const void*)&quantize_rows_f16_regs<1, 8>
                         : (const void*)&quantize_rows_f16_regs<1, 16>;
    }
    void* kargs[] = {&x, &Q, &row_scale, &m, &k};
    const unsigned grid = wide ? (unsigned)M : (unsigned)((M + 3) / 4);
    e = hipLaunchKernel(fn, dim3(grid), dim3(256), kargs, 0, stream);
  } else {
    // longer rows (and K = 0): one workgroup per row, two passes over it
    void* kargs[] = {&x, &Q, &row_scale, &k};
    e = hipLaunchKernel((const void*)&quantize_rows_f16, dim3((unsigned)M), dim3(256), kargs, 0,
                        stream);
  }
  return e == hipSuccess ? LPGEMM_SUCCESS : LPGEMM_ERROR_LAUNCH;
}

const char* lpgemm_status_string(lpgemm_status status) {
  switch (status) {
    case LPGEMM_SUCCESS: return "success";
    case LPGEMM_ERROR_INVALID_VALUE: return "invalid value (null pointer or bad size)";
    case LPGEMM_ERROR_MISALIGNED: return "pointer not 16-byte aligned";
    case LPGEMM_ERROR_UNSUPPORTED_SHAPE: return "unsupported K (divisibility or range)";
    case LPGEMM_ERROR_ARCH: return "current device is not gfx950";
    case LPGEMM_ERROR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int lpgemm_version(void) { return 100; }

}  // extern "C"
