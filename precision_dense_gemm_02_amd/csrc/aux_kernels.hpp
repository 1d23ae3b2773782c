// Kernels around the GEMMs: the int4 -> FP6 E3M2 operand re-encoding and the
// per-row int8 quantiser of fp16 activations.  Only the translation unit
// with the C entry points includes this header (its kernels are not
// templates, so a second inclusion would define them twice).
#pragma once

#include "gemm_kernels.hpp"

namespace lpgemm {

// ---------------------------------------------------------------------------
// Packed int4 -> FP6 E3M2 operand rows for the E3M2 MFMA.
//
// Every int4 value v in [-8, 7] is exact in E3M2 (1 sign, 3 exponent bits
// with bias 3, 2 mantissa bits): 1 = 1.0 x 2^0, 3 = 1.5 x 2^1, 5 = 1.25 x 2^2,
// 7 = 1.75 x 2^2, 8 = 1.0 x 2^3, and so on.  A group of 32 values of one row
// (16 packed bytes) becomes 32 bytes: 32 six-bit codes packed little-endian
// into 24 bytes, then 8 zero bytes, so a row of K values takes K bytes and
// a group is two 16-byte chunks (the layout the LDS swizzle works in).
//
// Within a group the codes are stored in the order k = 0, 2, 4, 6, 1, 3, 5,
// 7, 8, 10, ...: even and odd nibbles of each packed dword are looked up
// separately.  The MFMA pairs slot i of A with slot i of B, and both
// operands use this order, so the sum over k is unchanged.
//
// Code lookup, four nibbles at a time: v_perm_b32 picks bytes from an
// eight-byte table, one table for nibbles 0..7 (v = 0..7) and one for
// 8..15 (v = -8..-1); the nibble's bit 3 selects between them.
__device__ __forceinline__ uint32_t e3m2_codes(uint32_t nib4) {
  // table bytes: codes of v = 0..7 and of v = -8..-1
  constexpr uint32_t kPosLo = 0x12100C00u, kPosHi = 0x17161514u;
  constexpr uint32_t kNegLo = 0x35363738u, kNegHi = 0x2C303234u;
  const uint32_t idx = nib4 & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(kPosHi, kPosLo, idx);
  const uint32_t neg = __builtin_amdgcn_perm(kNegHi, kNegLo, idx);
  const uint32_t mask = ((nib4 >> 3) & 0x01010101u) * 0xFFu;   // 0xFF where v < 0
  return (neg & mask) | (pos & ~mask);
}
// four six-bit codes (one per byte) -> 24 contiguous bits
__device__ __forceinline__ uint32_t pack4_6bit(uint32_t c) {
  return (c & 0x3Fu) | ((c >> 2) & 0xFC0u) | ((c >> 4) & 0x3F000u) | ((c >> 6) & 0xFC0000u);
}

__global__ __launch_bounds__(256) void pack_i4_e3m2(const uint8_t* __restrict__ src,
                                                    uint8_t* __restrict__ dst, int64_t groups) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= groups) return;
  const i32x4 x = ((const i32x4*)src)[g];
  uint32_t q[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w = (uint32_t)x[d];
    q[2 * d] = pack4_6bit(e3m2_codes(w & 0x0F0F0F0Fu));          // k = 8d, 8d+2, 8d+4, 8d+6
    q[2 * d + 1] = pack4_6bit(e3m2_codes((w >> 4) & 0x0F0F0F0Fu)); // k = 8d+1, ..., 8d+7
  }
  // eight 24-bit pieces -> six dwords
  const i32x4 lo = {(int)(q[0] | (q[1] << 24)), (int)((q[1] >> 8) | (q[2] << 16)),
                    (int)((q[2] >> 16) | (q[3] << 8)), (int)(q[4] | (q[5] << 24))};
  const i32x4 hi = {(int)((q[5] >> 8) | (q[6] << 16)), (int)((q[6] >> 16) | (q[7] << 8)), 0, 0};
  ((i32x4*)dst)[2 * g] = lo;
  ((i32x4*)dst)[2 * g + 1] = hi;
}


// Rows of at most 512 * WPR * NC halves, held in registers: WPR wavefronts
// share a row (a workgroup of four waves takes 4 / WPR rows) and each lane
// keeps its NC 16-byte chunks (chunk li + 64 WPR c, li the lane's index
// within the row), so the row is read once for both passes.  Chunks past the
// row end load as zero through the buffer resource, which leaves the absmax
// unchanged.  WPR = 4 spreads a row over 256 lanes for short M (the rounding
// pass is ALU latency there); WPR = 1 needs no LDS and no barrier.
template <int WPR, int NC>
__global__ __launch_bounds__(256) void quantize_rows_f16_regs(const uint8_t* __restrict__ X,
                                                              int8_t* __restrict__ Q,
                                                              float* __restrict__ scale, int M,
                                                              int K) {
  static_assert(WPR == 1 || WPR == 4, "a row takes one wave or the whole workgroup");
  constexpr int kRowLanes = 64 * WPR;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * (4 / WPR) + wave / WPR;
  const int li = threadIdx.x - (wave / WPR) * kRowLanes;
  if (WPR == 1 && row >= M) return;   // with WPR = 4 the grid has exactly M workgroups
  const int chunks = K >> 3;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + (size_t)row * K * 2), 0, K * 2, kBufferWord3);
  i32x4 v[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    v[c] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)(li + kRowLanes * c) * 16u, 0, 0);
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) amax = absmax8(__builtin_bit_cast(f16x8, v[c]), amax);
  amax = wave_max(amax);
  if constexpr (WPR > 1) {
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  }
  const float s = __fdiv_rn(amax, 127.0f);
  if (li == 0) scale[row] = s;
  const float r = __fdiv_rn(1.0f, s);
  uint64_t* qrow = (uint64_t*)(Q + (size_t)row * K);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = li + kRowLanes * c;
    if (idx < chunks) qrow[idx] = s != 0.f ? quantize8(__builtin_bit_cast(f16x8, v[c]), s, r) : 0;
  }
}

// Longer rows (and K = 0): one workgroup per row and two passes over it, the
// second re-reading the row (mostly from L2).
__global__ __launch_bounds__(256) void quantize_rows_f16(const uint8_t* __restrict__ X,
                                                         int8_t* __restrict__ Q,
                                                         float* __restrict__ scale, int K) {
  const int row = blockIdx.x;
  const int chunks = K / 8;   // 16-byte chunks of 8 halves
  const i32x4* xrow = (const i32x4*)(X + (size_t)row * K * 2);
  float amax = 0.f;
  for (int c = threadIdx.x; c < chunks; c += 256)
    amax = absmax8(__builtin_bit_cast(f16x8, xrow[c]), amax);
  amax = wave_max(amax);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float s = __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) scale[row] = s;
  const float r = __fdiv_rn(1.0f, s);
  uint64_t* qrow = (uint64_t*)(Q + (size_t)row * K);
  for (int c = threadIdx.x; c < chunks; c += 256)
    qrow[c] = s != 0.f ? quantize8(__builtin_bit_cast(f16x8, xrow[c]), s, r) : 0;
}

}  // namespace lpgemm
