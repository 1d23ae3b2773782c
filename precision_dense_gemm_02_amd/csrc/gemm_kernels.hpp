// Tiled MFMA GEMM kernels for gfx950 (CDNA4).
//
// One template serves the four entry points.  A workgroup computes a BM x BN
// tile of C.  Both operands are K-contiguous, so a K-stage of a tile is a
// block of rows of 128 LDS bytes each (128 int8, 64 fp16, or 128 int4 values
// once unpacked to int8):
//
//   global  --16-byte buffer loads (out-of-range reads return 0)-->  VGPRs
//   VGPRs   --ds_write_b128, XOR-swizzled 16-byte chunks-->          LDS stage
//   LDS     --ds_read_b128 fragments-->                              MFMA 32x32
//
// Two LDS stages: while the waves contract stage s, the next K-stage is
// already in flight from global memory into registers, and is written to the
// other stage after the MFMAs; one barrier per K-stage separates the phases.
//
// The pages' kernels (the PTX-vs-WMMA summary page; the async Tensor Core
// article, sections on the synchronous data path, cp.async, multi-stage
// buffering and swizzle) move tiles global -> shared -> registers -> mma with
// cp.async pipelining and swizzled shared memory.  On CDNA4 the MFMA reads its
// operands from VGPRs, so the same three-level path is built from buffer
// loads, LDS and ds_read_b128; there is no TMA or mbarrier to port.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lpgemm {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum Kind : int { KIND_I8 = 0, KIND_I4 = 1, KIND_F16 = 2, KIND_I8_DEQUANT = 3 };

// LDS bytes of one operand row per K-stage, and 16-byte chunks per such row.
constexpr int kStageRowBytes = 128;
constexpr int kChunksPerRow = kStageRowBytes / 16;

// Word 3 of a gfx9 buffer resource for raw (unformatted, stride-0) access.
constexpr int kBufferWord3 = 0x00020000;
// A buffer offset at or beyond the resource's size reads as zero.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct GemmArgs {
  const uint8_t* A;     // operand rows of `row_bytes` bytes, M rows
  const uint8_t* B;     // operand rows of `row_bytes` bytes, N rows
  void* C;              // M x N, int32 or fp32
  const float* row_scale;
  const float* col_scale;
  int M, N;
  int row_bytes;        // global bytes per operand row (K, 2K or K/2)
  int k_stages;         // number of 128-byte LDS K-stages
  int tiles_m, tiles_n;
  int group_m;          // tile rows per raster group
};

// Position of 16-byte chunk `c` of LDS row `r` within that row.  XOR with a
// 3-bit function of the row so that the eight rows read together by
// consecutive lanes (a fragment read takes one chunk from each of 32
// consecutive rows) fall on distinct chunk positions: conflict-free for a
// 32-bank (128 B) LDS across 8 consecutive rows, and for a 64-bank (256 B)
// LDS across 16 consecutive rows, since rows r and r+1 then start half a
// bank set apart and bit 2 of the swizzle alternates with the row parity.
__device__ __forceinline__ int swizzle_chunk(int r, int c) {
  int f = (((r & 1) ^ ((r >> 3) & 1)) << 2) | ((r >> 1) & 3);
  return c ^ f;
}

__device__ __forceinline__ int lds_offset(int r, int c) {
  return r * kStageRowBytes + (swizzle_chunk(r, c) << 4);
}

// Map the linear workgroup id to a (tile_m, tile_n) pair.  Workgroups are
// dealt round-robin to the 8 XCDs (each with its own L2), so first give every
// XCD a contiguous range of logical tile ids, then walk those ids in groups
// of `group_m` tile rows so that workgroups resident together on one XCD
// share A row panels and B column panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& tm, int& tn) {
  const int nb = gridDim.x;
  const int w = blockIdx.x;
  const int xcd = w & 7;
  const int q = nb >> 3, rem = nb & 7;
  const int logical = xcd * q + (xcd < rem ? xcd : rem) + (w >> 3);
  const int per_group = p.group_m * p.tiles_n;
  const int group = logical / per_group;
  const int first_m = group * p.group_m;
  const int gm = min(p.tiles_m - first_m, p.group_m);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// INT4 expansion: 8 nibbles of a dword become 8 int8 bytes, each
// holding 16 * v (the nibble moved to the byte's high half keeps its two's
// complement sign).  Even-k nibbles go to `lo`, odd-k nibbles to `hi`.  The
// same byte permutation of k is applied to A and B, so the sum over k is
// unchanged; every product carries a factor 256 that the epilogue removes.
__device__ __forceinline__ void expand_int4(uint32_t x, uint32_t& lo, uint32_t& hi) {
  lo = (x << 4) & 0xF0F0F0F0u;
  hi = x & 0xF0F0F0F0u;
}

template <int KIND>
struct KindTraits;
template <>
struct KindTraits<KIND_I8> {
  static constexpr int global_chunks = kChunksPerRow;  // 128 B of a row per stage
  using Acc = i32x16;
};
template <>
struct KindTraits<KIND_I8_DEQUANT> {
  static constexpr int global_chunks = kChunksPerRow;
  using Acc = i32x16;
};
template <>
struct KindTraits<KIND_I4> {
  static constexpr int global_chunks = kChunksPerRow / 2;  // 64 packed B -> 128 LDS B
  using Acc = i32x16;
};
template <>
struct KindTraits<KIND_F16> {
  static constexpr int global_chunks = kChunksPerRow;
  using Acc = f32x16;
};

template <int KIND>
__device__ __forceinline__ typename KindTraits<KIND>::Acc mfma(const i32x4& a, const i32x4& b,
                                                               const typename KindTraits<KIND>::Acc& c) {
  if constexpr (KIND == KIND_F16) {
    // 32 x 32 x 16 fp16 -> fp32: 8 halves (16 bytes) of K per lane
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    // 32 x 32 x 32 int8 -> int32: 16 bytes of K per lane
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
}

// BM x BN workgroup tile, WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) sub-tile made of 32 x 32 MFMA blocks.
template <int KIND, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void gemm_tiled(GemmArgs p) {
  using Traits = KindTraits<KIND>;
  using Acc = typename Traits::Acc;
  constexpr int kThreads = WM * WN * 64;
  constexpr int GCH = Traits::global_chunks;        // global 16-byte chunks per row per stage
  constexpr int kStageBytesGlobal = GCH * 16;
  constexpr int kLoadsA = BM * GCH / kThreads;      // chunk loads per thread per stage
  constexpr int kLoadsB = BN * GCH / kThreads;
  static_assert(BM * GCH % kThreads == 0 && BN * GCH % kThreads == 0, "tile/thread mismatch");
  static_assert(kLoadsA >= 1 && kLoadsB >= 1, "too many threads for the tile");
  constexpr int WTM = BM / WM, WTN = BN / WN;       // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;       // 32x32 MFMA blocks per wave
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  constexpr int kStageA = BM * kStageRowBytes;
  constexpr int kStageB = BN * kStageRowBytes;
  constexpr int kStage = kStageA + kStageB;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  int tm, tn;
  tile_coords(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Buffer resources over this tile's A and B row panels: rows past M (N)
  // and chunks past the row end read as zero.
  const int rows_a = min(BM, p.M - m0);
  const int rows_b = min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + (size_t)m0 * p.row_bytes), 0, rows_a * p.row_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + (size_t)n0 * p.row_bytes), 0, rows_b * p.row_bytes, kBufferWord3);

  // Per-thread load slots: slot i covers chunk c = tid + i * kThreads of the
  // stage, i.e. row c / GCH, chunk c % GCH (consecutive lanes walk along a row).
  uint32_t a_row_off[kLoadsA], b_row_off[kLoadsB];
  int a_col[kLoadsA], b_col[kLoadsB];
  int a_lds[kLoadsA], b_lds[kLoadsB];
#pragma unroll
  for (int i = 0; i < kLoadsA; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / GCH, col = c % GCH;
    a_row_off[i] = r * p.row_bytes + col * 16;
    a_col[i] = col * 16;
    a_lds[i] = (KIND == KIND_I4) ? lds_offset(r, 2 * col) : lds_offset(r, col);
  }
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / GCH, col = c % GCH;
    b_row_off[i] = r * p.row_bytes + col * 16;
    b_col[i] = col * 16;
    b_lds[i] = kStageA + ((KIND == KIND_I4) ? lds_offset(r, 2 * col) : lds_offset(r, col));
  }

  i32x4 ra[kLoadsA], rb[kLoadsB];

  auto load_stage = [&](int ks) {
    const int kbyte = ks * kStageBytesGlobal;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
      const bool in_row = kbyte + a_col[i] < p.row_bytes;
      const uint32_t off = in_row ? a_row_off[i] + kbyte : kOutOfRange;
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) {
      const bool in_row = kbyte + b_col[i] < p.row_bytes;
      const uint32_t off = in_row ? b_row_off[i] + kbyte : kOutOfRange;
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, off, 0, 0);
    }
  };

  auto store_chunk = [&](uint8_t* base, int lds_off, const i32x4& v) {
    if constexpr (KIND == KIND_I4) {
      // 32 packed nibbles -> two 16-byte chunks of int8 (16 * value each).
      // lds_off addresses chunk 2g; chunk 2g+1 sits at swizzle(r, 2g+1),
      // which differs from swizzle(r, 2g) only in bit 0: XOR 16 bytes.
      uint32_t lo0, hi0, lo1, hi1, lo2, hi2, lo3, hi3;
      expand_int4((uint32_t)v.x, lo0, hi0);
      expand_int4((uint32_t)v.y, lo1, hi1);
      expand_int4((uint32_t)v.z, lo2, hi2);
      expand_int4((uint32_t)v.w, lo3, hi3);
      const i32x4 c0 = {(int)lo0, (int)hi0, (int)lo1, (int)hi1};
      const i32x4 c1 = {(int)lo2, (int)hi2, (int)lo3, (int)hi3};
      *(i32x4*)(base + lds_off) = c0;
      *(i32x4*)(base + (lds_off ^ 16)) = c1;
    } else {
      *(i32x4*)(base + lds_off) = v;
    }
  };

  auto store_stage = [&](int buf) {
    uint8_t* base = smem + buf * kStage;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) store_chunk(base, a_lds[i], ra[i]);
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) store_chunk(base, b_lds[i], rb[i]);
  };

  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Fragment addressing: lane l reads row (l & 31) of a 32-row block, chunk
  // 2*kk + (l >> 5) of the stage row, for K-step kk (32 LDS bytes).
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  const int a_frag_base = (wm * WTM + frag_row) * kStageRowBytes;
  const int b_frag_base = kStageA + (wn * WTN + frag_row) * kStageRowBytes;

  auto compute_stage = [&](int buf) {
    const uint8_t* base = smem + buf * kStage;
#pragma unroll
    for (int kk = 0; kk < kChunksPerRow / 2; ++kk) {
      // the row within a 32-row block decides the swizzle; blocks start at
      // multiples of 32 rows, so the block offset does not change it
      const int chunk_pos = swizzle_chunk(frag_row, 2 * kk + frag_half) << 4;
      i32x4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *(const i32x4*)(base + a_frag_base + i * 32 * kStageRowBytes + chunk_pos);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *(const i32x4*)(base + b_frag_base + j * 32 * kStageRowBytes + chunk_pos);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma<KIND>(fa[i], fb[j], acc[i][j]);
    }
  };

  const int nks = p.k_stages;   // 0 when K = 0: C is written as zeros
  if (nks > 0) {
    load_stage(0);
    store_stage(0);
    __syncthreads();
  }
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) load_stage(ks + 1);
    compute_stage(cur);
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element e of lane l in a 32x32 block holds
  // row 8*(e/4) + 4*(l/32) + e%4, column l%32.
  const int col_in_block = lane & 31;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + col_in_block;
      const bool col_ok = col < p.N;
      float cs = 0.f;
      if constexpr (KIND == KIND_I8_DEQUANT) cs = col_ok ? p.col_scale[col] : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * frag_half + (e & 3);
        if (col_ok && row < p.M) {
          const size_t idx = (size_t)row * p.N + col;
          if constexpr (KIND == KIND_F16) {
            ((float*)p.C)[idx] = acc[i][j][e];
          } else if constexpr (KIND == KIND_I4) {
            ((int32_t*)p.C)[idx] = acc[i][j][e] >> 8;   // undo the 16 x 16 scaling
          } else if constexpr (KIND == KIND_I8_DEQUANT) {
            float t = (float)acc[i][j][e];
            t = t * p.row_scale[row];
            t = t * cs;
            ((float*)p.C)[idx] = t;
          } else {
            ((int32_t*)p.C)[idx] = acc[i][j][e];
          }
        }
      }
    }
  }
}

}  // namespace lpgemm
