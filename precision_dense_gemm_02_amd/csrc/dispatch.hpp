// Host-side dispatch shared by the translation units of liblpgemm: argument
// checks, the kernel configurations and their choice per shape, and the
// launch of one GEMM kernel (run<KIND, BKN>).
//
// run<> is defined here and instantiated once per operand kind in its own
// translation unit (run_*.hip), so that the library's kernel instantiations
// compile in parallel; lpgemm.hip, which holds the C entry points, sees only
// the declarations.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/lpgemm.h"
#include "gemm_kernels.hpp"

namespace lpgemm {

struct DeviceInfo {
  bool probed = false;
  bool is_gfx950 = false;
  int cu_count = 0;
};

// Current device's properties, read once per device (lpgemm.hip).
lpgemm_status current_device(DeviceInfo& out);

// The configuration pinned by lpgemm_force_config (or LPGEMM_FORCE_CONFIG at
// load time), -1 for automatic selection (lpgemm.hip).
extern std::atomic<int> g_forced_config;
inline int forced_config() { return g_forced_config.load(std::memory_order_relaxed); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Host-only argument checks, in the order the header documents.  Sets
// `nothing_to_do` when the product is empty (M or N is zero).
inline lpgemm_status validate(Kind kind, int64_t M, int64_t N, int64_t K, const void* A, const void* B,
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
  CFG_256_S2_R128_PERSIST = 47,  // configuration 0 as a persistent grid of at most one workgroup per CU
  // int4 ablations (the same kernels as the base configuration for the other kinds)
  CFG_128_S2_R256_W4 = 48,       // configuration 36, int4 fragments read 32 packed bytes at a time
  CFG_256_S2_R128_SX = 49,       // configuration 0, int4 expanded by sign extension (no x16 scaling)
  CFG_256_S2_R128_W4 = 50,       // configuration 0, int4 fragments read 32 packed bytes at a time
  CFG_128_S2_R256_SX = 51,       // configuration 36, int4 expanded by sign extension
  CFG_256_S2_R128_PERSIST_SX = 52,  // configuration 47, int4 too, expanded by sign extension
  CFG_256_S2_R128_PIN_SX = 53,   // configuration 0 with pinned loads, int4 too, expanded by sign extension
  CFG_REF = 54,                  // the reference kernel: one unswizzled LDS stage, nothing tuned (gemm_ref)
  CFG_STREAM_128x64 = 55,        // short M: 128 x 64 tiles, A (3 stages) and B (10 stages) in separate rings
  CFG_STREAM_128x64_B14 = 56,    // ... B in 14 stages (A in 2)
  CFG_STREAM_64x64 = 57,         // ... 64 x 64 tiles, A 3 stages, B 14 stages
  CFG_256_S2_R128_EARLY = 58,    // configuration 0 with half of each stage's loads issued one K-step earlier
  CFG_128_S2_R256_BIAS = 59,     // configuration 36, int4 expanded biased (u = v + 8) with sum corrections
  CFG_128_S2_R256_SPLITK = 60,   // configuration 36 (int4: 48) with K split over workgroups (needs a workspace)
  CFG_256x224_S2_R128 = 61,      // configuration 0 with 256 x 224 tiles (four waves of 64 x 224)
  CFG_256x224_S2_R128_PERSIST = 62,  // configuration 61 as a persistent grid (int4: 61)
  CFG_SKINNY_PIPE_W4R2_N2 = 63,  // configuration 14 with two 32-row B blocks per workgroup (up to 64 columns)
  CFG_256x128_S3_R128 = 64,      // 4 waves, 256 x 128, 3 stages of 128-byte rows
  CFG_128x256_S3_R128 = 65,      // 4 waves, 128 x 256, 3 stages of 128-byte rows
  CFG_COUNT = 66
};

// Row bytes of one LDS K-stage for a configuration (the register-staged
// kernels expand int4 to int8 on the way into LDS, 128 values per stage).
inline int stage_row_bytes(KernelCfg c) {
  return (c == CFG_256_S4_R64 || c == CFG_256_S3_R64 || c == CFG_128_S4_R64 || c == CFG_PP_R64 ||
          c == CFG_128x64_S4_R64 || c == CFG_256x128_S4_R64 || c == CFG_128x64_S8_R64 ||
          c == CFG_256_S5_R64_NT || c == CFG_256_S4_R64_NT)
             ? 64
             : ((c == CFG_128x64_S3_R256 || c == CFG_128_S2_R256 || c == CFG_128_S2_R256_W4 ||
                 c == CFG_128_S2_R256_SX || c == CFG_128_S2_R256_BIAS || c == CFG_128_S2_R256_SPLITK)
                    ? 256
                    : 128);
}
inline bool expands_int4_in_lds(KernelCfg c) { return c >= CFG_V1_256x256 && c <= CFG_V1_64x64; }

inline int tiles(int64_t x, int t) { return (int)((x + t - 1) / t); }

// The E3M2 kind runs only on the LDS-pipelined kernels with 128-byte stage
// rows (two 64-value MFMA steps per stage); the reduced int8 kind of the
// fp64 emulation uses the same three.
inline bool supports_e3m2(int c) {
  return c == CFG_256_S2_R128 || c == CFG_128x64_S6_R128 || c == CFG_128_S4_R128 || c == CFG_256_S2_R128_PIN_E3M2;
}

inline KernelCfg choose_config_e3m2(int64_t M, int64_t N, int cu_count) {
  const int f = forced_config();
  if (f >= 0 && supports_e3m2(f)) return (KernelCfg)f;
  if (M <= 128) return CFG_128x64_S6_R128;
  // 256 x 256 tiles once they fill more than half the CUs, as for the other
  // kinds (graph-timed, one MI355X, 3072^3: E3M2 1060 against 1011 TOP/s,
  // K x N B 1325 against 1162 on 128 x 128 tiles)
  if (2 * (int64_t)tiles(M, 256) * tiles(N, 256) > cu_count) return CFG_256_S2_R128;
  if ((int64_t)tiles(M, 128) * tiles(N, 128) >= cu_count / 2) return CFG_128_S4_R128;
  return CFG_128x64_S6_R128;
}

// Columns of C per workgroup for the skinny kernel at M <= 32 with `nb`
// 32-row B blocks per workgroup (configs 14 and 63): a multiple of 4 that
// spreads the N columns evenly over the workgroups the CUs hold at once
// (two per CU of one block, one of two blocks) or a few times as many, when
// that leaves the busiest CU fewer columns than 32-column tiles do; 0
// otherwise.  At least 24 columns: below that each workgroup's copy of the
// A rows outweighs its share of B.  N = 14336 on 256 CUs: 28 columns with
// one block (512 workgroups, 56 columns per CU against two 32-column tiles
// on 192 CUs); N = 8192 and 16384 already spread evenly.
inline int skinny_columns(int64_t N, int cu_count, int nb) {
  if (cu_count <= 0 || N <= 0) return 0;
  const int per_cu = nb == 1 ? 2 : 1;
  const int64_t plain = ((int64_t)tiles(N, 32) + cu_count - 1) / cu_count * 32;
  for (int64_t k = 1; k <= 4; ++k) {
    const int64_t groups = (int64_t)cu_count * per_cu * k;
    const int64_t w = ((N + groups - 1) / groups + 3) / 4 * 4;
    if (w <= 32 * nb) return w >= 24 && per_cu * k * w < plain ? (int)w : 0;
  }
  return 0;
}

// The automatic choice for the i8, i4, f16 and dequant kinds (no forced
// configuration, no split-K workspace).
inline KernelCfg auto_config(int64_t M, int64_t N, int64_t K, int cu_count, int kind) {
  // few rows against many columns: stream B with split-K workgroups, each
  // owning an equal share of the columns where that helps (skinny_columns);
  // int4, whose expansion adds ALU work per byte, with eight waves of one
  // K-block per round (graph-timed, one MI355X: int4 16 x 14336 x 4096 333
  // against 301 TOP/s with four waves of two, 32 x 14336 x 4096 522 against
  // 490, 16 x 4096 x 4096 141 against 127)
  // The other kinds take eight waves too when the 32-column tiles number at
  // most half the CUs: more waves per CU then stream B (graph-timed, one
  // MI355X: int8 32 x 4096 x 4096 6.98 against 7.59 us, dequant
  // 16 x 4096 x 14336 13.77 against 14.45, fp16 16 x 4096 x 4096 8.72
  // against 8.89, dequant 32 x 2048 x 8192 10.92 against 11.19; at N = 8192
  // four waves stay ahead, int8 32 x 8192 x 8192 14.04 against 15.41).
  const bool few_columns = (int64_t)tiles(N, 32) <= cu_count / 2;
  if (M <= 32)
    return kind == KIND_I4 || few_columns ? CFG_SKINNY_PIPE_W8R1 : CFG_SKINNY_PIPE_W4R2;
  // int4 keeps that kernel up to three 32-row bands (graph-timed, one
  // MI355X: M = 48, 64, 96 at N = 14336, K = 4096: 532, 625, 684 TOP/s
  // against 485, 589, 636 with four waves and 325, 424, 604 for the band
  // kernel below; M = 128 782 against 842 for the band kernel)
  if (kind == KIND_I4 && M <= 96) return CFG_SKINNY_PIPE_W8R1;
  // 33-64 rows: the 128-row band kernel below once its 64-column tiles
  // number more than half the CUs, else the skinny kernel over two 32-row
  // bands (graph-timed at K = 4096, one
  // MI355X: dequant M = 64, N = 14336 512 TOP/s against 317 skinny and 242
  // for the earlier choice, the split-K kernel of 64-row tiles; fp16 there
  // 329 against 176 TFLOP/s; N = 8192 (128 tiles) 317 against 343 skinny)
  // (and there, as above, eight waves at few columns: int8 64 x 4096 x 4096
  // 7.05 against 7.47 us, dequant 64 x 4096 x 14336 18.67 against 19.02)
  if (M <= 64)
    return (int64_t)tiles(N, 64) > cu_count / 2 ? CFG_128x64_S3_R256
           : few_columns                         ? CFG_SKINNY_PIPE_W8R1
                                                 : CFG_SKINNY_PIPE_W4R2;
  // a 128-row band: 128 x 64 tiles double the workgroups of 128 x 128, and
  // B streams in 256-byte pieces per stage (graph-timed, one MI355X, against
  // six 128-byte stages: dequant M = 128, K = 4096, N = 14336 19.2 against
  // 20.4 us; fp16 there 555 against 524-541 TFLOP/s, fp16 128 x 8192 x 8192
  // 444 against 364; int4 128 x 14336 x 4096 846 against 804 TOP/s)
  if (M <= 128) return CFG_128x64_S3_R256;
  const int64_t big = (int64_t)tiles(M, 256) * tiles(N, 256);
  // N a multiple of 224 (the LLM projection's 14336 = 64 x 224): 256 x 224
  // tiles once they fill more than half the CUs and their rounds of one tile
  // per CU, each 7/8 of a 256 x 256 round's work, add up to less (M = 2048:
  // 512 tiles in two full rounds against 448 in 1.75), on the persistent
  // grid when they fill two or more whole rounds (int4: the plain grid).  Graph-timed,
  // K = 4096, one MI355X: dequant M = 1024 1959 TOP/s against 1950 with
  // 256 x 256 tiles and 1329 with 128 x 128; M = 768 1808 against 1752 and
  // 1332; M = 512 (128 tiles, half the CUs) takes the half-size tiles below;
  // M = 1536 (1.5 rounds) 1725 plain against 1568 persistent; int8
  // M = 4096 2156 against 2064 on the persistent 256 x 256 grid (3.5
  // rounds); the persistent 224 grid 2-3.5% ahead of the plain one at
  // M = 2048, 4096, 5120, 6144 (whole rounds) and 4-8% behind it at
  // M = 2560 and 3584 (2.5 and 3.5 rounds).
  if (N % 224 == 0) {
    const int64_t t224 = (int64_t)tiles(M, 256) * (N / 224);
    const int64_t r256 = (big + cu_count - 1) / cu_count;
    const int64_t r224 = (t224 + cu_count - 1) / cu_count;
    if (2 * t224 > cu_count && 7 * r224 < 8 * r256)
      return t224 >= 2 * (int64_t)cu_count && t224 % cu_count == 0 ? CFG_256x224_S2_R128_PERSIST
                                                                    : CFG_256x224_S2_R128;
  }
  // 256 x 256 tiles once they fill more than half the CUs: on this
  // power-limited board fewer busy CUs run at a higher clock, and the large
  // tile moves half the bytes per MAC of a 128 x 128 one (graph-timed, one
  // MI355X: int8 3072^2 x 4096, 144 tiles, 1696 TOP/s against 1367 for the
  // best 128 x 128 kernel; dequant 512 x 16384 x 4096, 128 tiles, 1495
  // against 1569).  Two or more whole rounds: the persistent grid, whose
  // workgroups load a tile's first stage while they store the previous
  // tile's C (8192^3: int8 +3.0%, fp16 +1.6%; 6144 x 8192 x 4096, three
  // rounds, +2.8%); int4 stays on configuration 0, whose registers leave no
  // room for the persistent state.  With a partial last round the plain
  // grid, whose workgroups start wherever a CU frees up, was ahead (LLM
  // M = 2048, 1.75 rounds: 1919 against 1757 TOP/s; 5120 x 8192 x 4096, 2.5
  // rounds: 2041 against 1939; 7168 x 8192 x 4096, 3.5: 2114 against 2065).
  if (2 * big > cu_count) {
    if (big >= 2 * (int64_t)cu_count && big % cu_count == 0 && kind != KIND_I4) return CFG_256_S2_R128_PERSIST;
    return CFG_256_S2_R128;
  }
  // half-size large tiles, 128 x 256 (int4: 256 x 128) with three 128-byte
  // stages, when they make more than half a round and at most one, at
  // K >= 2048 (graph-timed, one MI355X, against the earlier choice: int8 2048 x 4096
  // x 4096 1716 against 1480 TOP/s, 1536 x 4096 x 4096 1517 against 1319,
  // 1280 x 4096 x 4096 1442 against 1211, 2048 x 4096 x 2048 1487 against
  // 1200; dequant 512 x 14336 x 4096 1626 against 1458 on 256 x 224 tiles
  // (128 of them), 768 x 8192 x 4096 1570 against 1352; fp16 1536 x 4096 x
  // 4096 887 against 786 TFLOP/s; int4 2048 x 4096 x 4096 2037 against
  // 1739; a full round and more lost: int8 1536 x 6144 x 2048, 288 tiles,
  // 1026 against 1383 for 256 x 256 tiles, and half a round: 2048^3 1000
  // against 1086)
  {
    const bool i4 = kind == KIND_I4;
    const int64_t t_half = i4 ? (int64_t)tiles(M, 256) * tiles(N, 128) : (int64_t)tiles(M, 128) * tiles(N, 256);
    if (K >= 2048 && 2 * t_half > cu_count && t_half <= cu_count) return i4 ? CFG_256x128_S3_R128 : CFG_128x256_S3_R128;
  }
  // 128 x 64 tiles with three 256-byte stages (the 128-row band kernel)
  // when they make between a quarter of a round and one round, at K >=
  // 2048, except for int4 (graph-timed, one MI355X, against the earlier
  // 128 x 128 or 64 x 64 choice: int8 1024 x 1024 x 8192 798 against 506
  // TOP/s, 1024 x 2048 x 2048 956 against 889, 512 x 4096 x 4096 1168
  // against 1012, 256 x 8192 x 4096 1138 against 1019, 768 x 768 x 4096 401
  // against 379; fp16 1024 x 1024 x 4096 396 against 253 TFLOP/s; dequant
  // 256 x 4096 x 4096 672 against 604; at 1024^3 it lost, 382 against 404,
  // and at 1536^3, 288 tiles, 567 against 784)
  const int64_t t_band = (int64_t)tiles(M, 128) * tiles(N, 64);
  if (kind != KIND_I4 && K >= 2048 && 4 * t_band >= cu_count && t_band <= cu_count) return CFG_128x64_S3_R256;
  // 128 x 128 tiles: fp16 four 128-byte stages (2048^3: 23.1 against 25.4
  // us with four 64-byte stages); int4 two 256-byte stages with 32-byte
  // fragment reads, which remove the bank conflicts of 8-byte reads on
  // 256-byte rows (2048^3: 1290 against 1248 TOP/s); int8 and dequant four
  // 128-byte stages, or two 256-byte stages for one round of tiles at
  // K <= 2048 (graph-timed, one MI355X: 2048^2 x 4096 1524 against 1430
  // TOP/s, 1280 x 4096 x 4096 1234 against 1054, 1536 x 4096 x 8192 1582
  // against 1445, dequant 512 x 14336 x 2048 (448 tiles) 1248 against
  // 1190; 2048^3 1247 against 1201 the other way)
  const int64_t mid = (int64_t)tiles(M, 128) * tiles(N, 128);
  if (mid >= cu_count / 2) {
    if (kind == KIND_F16) return CFG_128_S4_R128;
    if (kind == KIND_I4) return CFG_128_S2_R256_W4;
    return mid <= cu_count && K <= 2048 ? CFG_128_S2_R256 : CFG_128_S4_R128;
  }
  // at most half as many 64 x 64 tiles as CUs: 32 x 32 tiles whose eight
  // waves split K, four times the workgroups (graph-timed, one MI355X: int8 512^3
  // 2.89 against 3.53 us, int4 2.87 against 3.79, fp16 3.43 against 4.70;
  // int8 512 x 512 x 16384 21.7 against 63.8 us; 768^3, with 144 tiles,
  // stays faster on 64 x 64: 4.23 against 5.26 us)
  // int4 from K = 4096 on too, whose band choice is this (graph-timed, one
  // MI355X: int4 1024 x 1024 x 4096 720 against 600 TOP/s on 64 x 64 tiles,
  // 768 x 768 x 8192 609 against 377, 1024 x 1024 x 16384 870 against 578;
  // 1024^3 350 against 371 the other way)
  if ((int64_t)tiles(M, 64) * tiles(N, 64) <= cu_count / 2 || (kind == KIND_I4 && K >= 4096))
    return CFG_SKINNY_PIPE_W8R1;
  return CFG_V1_64x64;
}

inline KernelCfg choose_config(int64_t M, int64_t N, int64_t K, int cu_count, int kind) {
  const int f = forced_config();
  // configurations 45 and 46 differ from 0 only for the E3M2 kind and for
  // K x N B
  if (f == CFG_256_S2_R128_PIN_E3M2 || f == CFG_256_S2_R128_PIN_KXN) return CFG_256_S2_R128;
  if (f >= 0) return (KernelCfg)f;
  return auto_config(M, N, K, cu_count, kind);
}

// Split-K over 128 x 128 tiles (configuration 60) for products with few
// tiles and a long K: each tile's K-stages are split over up to four
// workgroups, which write raw partial sums to a caller-provided workspace;
// the last one of a tile to finish adds them and runs the epilogue, so the
// result is the unsplit kernel's bit for bit for the integer kinds.  The
// hand-over (the parts written through to the device's coherence point, an
// arrival counter, the parts read back) costs a few microseconds per tile,
// so the automatic choice splits only products whose 128 x 128 tiles fill
// at most a quarter of the CUs (see splitk_auto_shape), four ways, and only
// when K spans at least 32 K-stages of 256 bytes (8 per part); below 64
// stages only where the unsplit choice, the band kernel's 128 x 64 tiles,
// fills less than half the CUs, or for int4, which keeps 64 x 64 tiles.
// Measured (graph replay, one MI355X) against the unsplit choice: int8
// 512 x 2048 x 32768 1486 against 938 TOP/s, 256 x 4096 x 16384 1163
// against 891, 1024 x 1024 x 16384 1088 against 877, 600 x 1000 x 8208 (80
// band tiles) 458 against 405; fp16 1024 x 1024 x 8192 (64 stages of 256
// bytes) 543 against 442 TFLOP/s; int4 1024 x 1024 x 16384 1276 against
// 576; unsplit as fast or faster at 32 stages with 128 band tiles: int8
// 1024 x 1024 x 8192 797 against 775, dequant 256 x 4096 x 8192 775
// against 794.  Two parts of 8 stages lost: int8 1024 x 1024 x 4096 16.4
// against 12.8 us, the LLM projection at M = 128, K = 4096 (112 tiles) 23
// against 18 us.
//
// Workspace layout, the same for every shape so that one workspace serves
// products of any size in turn: 4 KiB of 32-bit arrival counters (tile t
// uses counter t; all are zero between calls), then tiles x splits slots of
// 128 x 128 32-bit partial sums.  Products of more than 1024 tiles do not
// split.
constexpr int64_t kSplitTile = 128;
constexpr int64_t kSplitSlotBytes = kSplitTile * kSplitTile * 4;
constexpr int kMaxSplits = 4;
constexpr int kMinStagesPerSplit = 8;
constexpr int64_t kSplitCounterBytes = 4096;
constexpr int64_t kMaxSplitTiles = kSplitCounterBytes / 4;

inline int64_t splitk_bytes(int64_t ntiles, int splits) {
  return splits > 1 ? kSplitCounterBytes + ntiles * splits * kSplitSlotBytes : 0;
}

// Whether the automatic choice splits an M x N product on `cu_count` CUs
// at all (any K): above 64 rows (below that the skinny kernels split K
// inside a workgroup) and when the 128 x 128 tiles fill at most a quarter
// of the CUs, but not above 128 rows with at most a quarter of the CUs'
// worth of 64 x 64 tiles, where the unsplit choice (32 x 32 tiles whose
// waves split K) was as fast or faster (int8 512 x 512 x 16384: 21.7
// against 23.4 us split; 300 x 520 x 8208: 16.6 against 18.4 us).  Such a
// product may use up to kMaxSplits parts.
inline bool splitk_auto_shape(int64_t M, int64_t N, int cu_count) {
  if (M <= 64 || (int64_t)tiles(M, kSplitTile) * tiles(N, kSplitTile) > cu_count / 4) return false;
  return M <= 128 || (int64_t)tiles(M, 64) * tiles(N, 64) > cu_count / 4;
}

// Parts for the automatic choice with `nks` 256-byte K-stages (1: no split).
inline int splitk_auto_splits(int64_t M, int64_t N, int nks, int cu_count, int kind) {
  if (!splitk_auto_shape(M, N, cu_count) || nks < kMaxSplits * kMinStagesPerSplit) return 1;
  if (nks < 2 * kMaxSplits * kMinStagesPerSplit && kind != KIND_I4 &&
      2 * (int64_t)tiles(M, 128) * tiles(N, 64) >= cu_count)
    return 1;
  return kMaxSplits;
}

// Parts for a launch of configuration 60 with `nks` K-stages and a
// workspace of `ws_bytes`: the automatic count (when forced: at least 2,
// at most one part per K-stage and as many as fill the CUs once), and 1 when
// the workspace is missing or too small.
inline int splitk_launch_splits(int64_t M, int64_t N, int nks, int cu_count, int kind, const void* ws,
                                int64_t ws_bytes) {
  if (!ws) return 1;
  const int64_t t = (int64_t)tiles(M, kSplitTile) * tiles(N, kSplitTile);
  if (t > kMaxSplitTiles) return 1;
  int s = splitk_auto_splits(M, N, nks, cu_count, kind);
  if (s < 2) {
    const int64_t fill = cu_count / t;
    s = fill > kMaxSplits ? kMaxSplits : (fill < 2 ? 2 : (int)fill);
  }
  if (s > nks) s = nks;
  if (s < 2 || ws_bytes < splitk_bytes(t, s)) return 1;
  return s;
}

// B stored K x N row-major runs on the LDS-pipelined kernels with 128-byte
// stage rows: 128 k-rows of B per stage.
inline bool supports_kxn(int c) {
  return c == CFG_256_S2_R128 || c == CFG_128x64_S6_R128 || c == CFG_128_S4_R128 || c == CFG_256_S2_R128_PIN_KXN;
}

inline KernelCfg choose_config_kxn(int64_t M, int64_t N, int cu_count) {
  const int f = forced_config();
  if (f >= 0 && supports_kxn(f)) return (KernelCfg)f;
  if (M <= 128) return CFG_128x64_S6_R128;
  // 256 x 256 tiles once they fill more than half the CUs, as for the other
  // kinds (graph-timed, one MI355X, 3072^3: E3M2 1060 against 1011 TOP/s,
  // K x N B 1325 against 1162 on 128 x 128 tiles)
  if (2 * (int64_t)tiles(M, 256) * tiles(N, 256) > cu_count) return CFG_256_S2_R128;
  if ((int64_t)tiles(M, 128) * tiles(N, 128) >= cu_count / 2) return CFG_128_S4_R128;
  return CFG_128x64_S6_R128;
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

// A launch of the skinny pipelined kernel with `w` columns per workgroup
// (at most its 32 NB B rows).
inline lpgemm_status launch_skinny(const void* fn, GemmArgs args, int threads, hipStream_t stream, int w) {
  args.tile_w = w;
  args.tiles_m = tiles(args.M, 32);
  args.tiles_n = tiles(args.N, w);
  args.group_m = 8;
  const int64_t nblocks = (int64_t)args.tiles_m * args.tiles_n;
  if (nblocks > INT32_MAX) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nblocks), dim3(threads), kargs, 0, stream);
  return e == hipSuccess ? LPGEMM_SUCCESS : LPGEMM_ERROR_LAUNCH;
}

// A persistent launch: at most `max_groups` workgroups (one per CU), each
// walking its tiles round by round (gemm_v3<..., PERSIST = true>).
template <int BM, int BN>
lpgemm_status launch_persistent(const void* fn, GemmArgs args, int threads, hipStream_t stream, int max_groups) {
  args.tiles_m = tiles(args.M, BM);
  args.tiles_n = tiles(args.N, BN);
  args.group_m = 8;
  const int64_t ntiles = (int64_t)args.tiles_m * args.tiles_n;
  if (ntiles > INT32_MAX - (int64_t)max_groups) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  const int64_t groups = ntiles < max_groups ? ntiles : max_groups;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(groups > 0 ? groups : 1)), dim3(threads), kargs, 0, stream);
  return e == hipSuccess ? LPGEMM_SUCCESS : LPGEMM_ERROR_LAUNCH;
}

// A split-K launch: a grid of tiles x splits workgroups (gemm_v3<..., SPK =
// true>), with the workspace's counters and slots in the arguments.
template <int BM, int BN>
lpgemm_status launch_split(const void* fn, GemmArgs args, int threads, hipStream_t stream, int splits, void* ws) {
  args.tiles_m = tiles(args.M, BM);
  args.tiles_n = tiles(args.N, BN);
  args.group_m = 8;
  const int64_t nblocks = (int64_t)args.tiles_m * args.tiles_n;
  if (nblocks > INT32_MAX) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  args.splits = splits;
  args.split_count = static_cast<uint32_t*>(ws);
  args.split_part = splits > 1 ? reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + kSplitCounterBytes) : nullptr;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nblocks, (unsigned)splits), dim3(threads), kargs, 0, stream);
  return e == hipSuccess ? LPGEMM_SUCCESS : LPGEMM_ERROR_LAUNCH;
}

// One GEMM of the given kind (BKN: B stored K x N) on `stream`: validation,
// the configuration for the shape, and the kernel launch.  `ws` (may be
// null) is a split-K workspace of `ws_bytes`; with one, short products may
// run split (configuration 60).  Defined in run_kernels.hpp; instantiated in
// run_*.hip.
template <int KIND, bool BKN = false>
lpgemm_status run(int64_t M, int64_t N, int64_t K, const void* A, const void* B, void* C, const float* rs,
                  const float* cs, hipStream_t stream, int modulus = 0, void* ws = nullptr,
                  int64_t ws_bytes = 0);

extern template lpgemm_status run<KIND_I8, false>(int64_t, int64_t, int64_t, const void*, const void*, void*,
                                                  const float*, const float*, hipStream_t, int, void*, int64_t);
extern template lpgemm_status run<KIND_I4, false>(int64_t, int64_t, int64_t, const void*, const void*, void*,
                                                  const float*, const float*, hipStream_t, int, void*, int64_t);
extern template lpgemm_status run<KIND_F16, false>(int64_t, int64_t, int64_t, const void*, const void*, void*,
                                                   const float*, const float*, hipStream_t, int, void*, int64_t);
extern template lpgemm_status run<KIND_I8_DEQUANT, false>(int64_t, int64_t, int64_t, const void*, const void*,
                                                          void*, const float*, const float*, hipStream_t, int, void*, int64_t);
extern template lpgemm_status run<KIND_I4_E3M2, false>(int64_t, int64_t, int64_t, const void*, const void*,
                                                       void*, const float*, const float*, hipStream_t, int, void*, int64_t);
extern template lpgemm_status run<KIND_I8_MOD, false>(int64_t, int64_t, int64_t, const void*, const void*,
                                                      void*, const float*, const float*, hipStream_t, int, void*, int64_t);
extern template lpgemm_status run<KIND_I8, true>(int64_t, int64_t, int64_t, const void*, const void*, void*,
                                                 const float*, const float*, hipStream_t, int, void*, int64_t);

}  // namespace lpgemm
