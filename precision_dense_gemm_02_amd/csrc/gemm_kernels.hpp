// Tiled MFMA GEMM kernels for gfx950 (CDNA4).
//
// Template families serve the entry points; each workgroup computes a tile
// of C.  Both operands are K-contiguous (one gemm_v3 variant also takes B as
// K x N), so a K-stage of a tile is a block of operand rows:
//
//   gemm_v3 (the default above a few hundred rows): 16-byte direct-to-LDS
//     buffer loads put each stage's rows straight into an XOR-swizzled LDS
//     ring (2-8 stages), ds_read_b128 fragments feed 32x32 MFMAs, and one
//     barrier per stage rotates the ring.  Knobs select the tile, the ring,
//     the load schedule, the C stores, a persistent grid that walks its
//     tiles round by round, and split-K over a caller's workspace.
//   gemm_tiled (the first kernel, kept for small grids): loads into VGPRs,
//     ds_write_b128 into LDS, then the same fragment reads.
//   gemm_skinny* (short M, and small products): the waves of a workgroup
//     split K, B goes through LDS, and the partial sums meet in LDS.
//   gemm_ref: one unswizzled stage, nothing pipelined, the depth-1
//     reference the tuned kernels are checked against.
//   gemm_pingpong, gemm_stream: measured alternatives (two wave groups
//     alternating memory and MFMA phases; a loader wave with a deep B ring).
//
// The pages' kernels (the PTX-vs-WMMA summary page; the async Tensor Core
// article, sections on the synchronous data path, cp.async, multi-stage
// buffering and swizzle) move tiles global -> shared -> registers -> mma with
// cp.async pipelining and swizzled shared memory.  On CDNA4 the MFMA reads its
// operands from VGPRs, so the same three-level path is built from buffer
// loads (direct to LDS), LDS and ds_read_b128; there is no TMA or mbarrier to
// port.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lpgemm {

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum Kind : int {
  KIND_I8 = 0,
  KIND_I4 = 1,
  KIND_F16 = 2,
  KIND_I8_DEQUANT = 3,
  KIND_I4_E3M2 = 4,
  KIND_I8_MOD = 5   // int8 product reduced modulo GemmArgs::modulus, one byte per element
};

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
  int modulus;          // KIND_I8_MOD: C[i][j] = (A.B)[i][j] mod modulus (0 < modulus <= 256), uint8
  double inv_modulus;   // KIND_I8_MOD: RN(1 / modulus)
  // split-K (gemm_v3<..., SPK = true>): K-stages split `splits` ways over
  // gridDim.y; per tile one arrival counter (zero between launches) and
  // `splits` slots of raw 32-bit partial accumulators
  int splits;
  uint32_t* split_count;
  uint32_t* split_part;
  // gemm_skinny_pipe: columns of C per workgroup (at most its 32 NB B rows;
  // 0: all of them)
  int tile_w;
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
// The logical id of workgroup w in a grid of nb workgroups.
__device__ __forceinline__ int xcd_logical(int w, int nb) {
  const int xcd = w & 7;
  const int q = nb >> 3, rem = nb & 7;
  return xcd * q + (xcd < rem ? xcd : rem) + (w >> 3);
}

// (tile_m, tile_n) of a logical tile id.
__device__ __forceinline__ void tile_of(const GemmArgs& p, int logical, int& tm, int& tn) {
  const int per_group = p.group_m * p.tiles_n;
  const int group = logical / per_group;
  const int first_m = group * p.group_m;
  const int gm = min(p.tiles_m - first_m, p.group_m);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& tm, int& tn) {
  const int nb = gridDim.x;
  const int w = blockIdx.x;
  const int logical = xcd_logical(w, nb);
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

// The sign-extending INT4 expansion (the same byte order, each byte holding
// v itself, so no scaling is left for the epilogue): with c = n XOR 8 the
// nibble's value plus 8, the byte c + 0x78 stays below 0x100 (no carry into
// the next byte) and XOR 0x80 turns it into c - 8 modulo 256, the two's
// complement byte of v.  Eight operations per eight nibbles against three.
__device__ __forceinline__ void expand_int4_sx(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const uint32_t t = x ^ 0x88888888u;
  lo = ((t & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
  hi = (((t >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
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
struct KindTraits<KIND_I8_MOD> {
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
// int4 values re-encoded as FP6 E3M2, one byte per value (see
// pack_i4_e3m2): products and their sums are integers below 2^24, exact in
// the fp32 accumulator
template <>
struct KindTraits<KIND_I4_E3M2> {
  static constexpr int global_chunks = kChunksPerRow;
  using Acc = f32x16;
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32 x 32 x 64 MFMA on FP6 E3M2 operands (format 3 of the f8f6f4 family),
// both block scales 2^0 (E8M0 127).  Each lane supplies 32 values of K in
// the low six dwords.
__device__ __forceinline__ f32x16 mfma_e3m2(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 3, 3, 0, 127, 0, 127);
}

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



// ---------------------------------------------------------------------------
// Direct-to-LDS loads, counter waits and barriers written out explicitly.
//
// The compiler's __syncthreads() carries a workgroup fence that waits for
// every outstanding vector-memory load (vmcnt(0)), which would drain the
// whole multi-stage load pipeline at each barrier.  The pipelined kernels
// therefore issue their direct-to-LDS loads, their vmcnt(N) waits and their
// barriers themselves: the "memory" clobbers keep the compiler from moving
// LDS accesses across them, and the counts are derived in each kernel.

// Raw buffer resource (gfx9 V#) over [base, base + bytes); offsets at or past
// `bytes` read as zero.  All fields are made wave-uniform.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu));   // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = kBufferWord3;
  return r;
}

// Each lane loads 16 bytes at buffer offset `voff`; lane l's bytes land at
// LDS byte address lds_addr + 16 l.  M0 carries the LDS address for the
// load and is restored afterwards; one wait state separates the M0 write
// from its use.
// Cache policy of the operand loads (the gfx950 cache-policy bits, written
// before `lds`): 0 default, 1 nt (non-temporal: stream, evict first),
// 2 sc0, 3 sc1, 4 sc0 sc1 (widest coherence scope).
template <int CPOL = 0>
__device__ __forceinline__ void lds_dma_16(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  uint32_t saved;
#define LPGEMM_LDS_DMA(MODS)                                              \
  asm volatile(                                                           \
      "s_mov_b32 %0, m0\n\t"                                              \
      "s_mov_b32 m0, %1\n\t"                                              \
      "s_nop 0\n\t"                                                       \
      "buffer_load_dwordx4 %2, %3, 0 offen " MODS "lds\n\t"              \
      "s_mov_b32 m0, %0"                                                  \
      : "=&s"(saved)                                                      \
      : "s"(lds_addr), "v"(voff), "s"(rsrc)                               \
      : "memory")
  if constexpr (CPOL == 1) LPGEMM_LDS_DMA("nt ");
  else if constexpr (CPOL == 2) LPGEMM_LDS_DMA("sc0 ");
  else if constexpr (CPOL == 3) LPGEMM_LDS_DMA("sc1 ");
  else if constexpr (CPOL == 4) LPGEMM_LDS_DMA("sc0 sc1 ");
  else LPGEMM_LDS_DMA("");
#undef LPGEMM_LDS_DMA
}

// The same transfer at 4 bytes per lane (lane l's word lands at lds_addr +
// 4 l).  Used to pull operand lines into the L2 ahead of their real loads:
// the words land in an LDS area nobody reads, so there is no register result
// to track and nothing for the compiler to drop.
__device__ __forceinline__ void lds_dma_4(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)p);
}

// Four accumulator elements summed over split-K slots: int32 adds (exact,
// wrapping like the MFMA's own accumulation) or binary32 adds in the order
// the slots are given.
template <typename AccT>
struct Acc_elem4 {
  using E = typename std::conditional<std::is_same<AccT, f32x16>::value, float, int>::type;
  E v[4];
  __device__ __forceinline__ void add(i32x4 x, bool first) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int xk = x[k];   // a vector element is not an object: copy it first
      const E e = __builtin_bit_cast(E, xk);
      if constexpr (std::is_same<E, float>::value) v[k] = first ? e : v[k] + e;
      else v[k] = first ? e : (E)((uint32_t)v[k] + (uint32_t)e);
    }
  }
  __device__ __forceinline__ E get(int k) const { return v[k]; }
};

// ---------------------------------------------------------------------------
// Four-wave kernel with direct-to-LDS loads and an LDS-staged epilogue.
//
// A workgroup of 4 waves (one per SIMD) computes a BM x BN tile; each wave
// owns a (BM/2) x (BN/2) quadrant made of 32 x 32 MFMA blocks, so that at
// BM = BN = 256 every wave keeps 16 independent accumulator chains in flight
// (a 32 x 32 MFMA needs about 8 per SIMD to run at full rate) and reads half
// as many LDS bytes per MAC as an 8-wave 128 x 64 split.  A tile 224
// columns wide (seven 32-column blocks, for N a multiple of 224 such as
// 14336) cannot be halved into 32-column blocks, so there each wave owns a
// band of BM/4 rows by all 224 columns (2 x 7 blocks, 14 chains); its
// epilogue stores a 224-column row with 56 lanes and leaves 8 idle.
//
// Operand rows stay K-contiguous in LDS, ROWB (64 or 128) bytes per row per
// K-stage: int8 or fp16 values, or packed int4 (int4 stays packed in LDS and
// is expanded to int8 in registers after the fragment read).  Global data
// goes straight into LDS with 16-byte buffer loads (lane l writes 16 bytes at
// base + 16 l), so the swizzle is applied by choosing which global chunk each
// lane fetches.  STAGES buffers form a ring: the loads of stage s+STAGES-1 are
// issued during stage s, so STAGES-1 stages of latency are hidden; the
// barrier that publishes stage s+1 sits in the middle of stage s's last
// K-step, and the first fragments of stage s+1 are read while the remaining
// MFMAs of stage s execute.
//
// Epilogue: each wave transposes its accumulators through LDS (64 rows at a
// time) so that every lane stores 16 contiguous bytes and a store
// instruction covers two 512-byte row segments.
template <int ROWB>
struct RowLayout;

// 128-byte rows: 8 chunks; the chunk position XORs a 3-bit function of the
// row, conflict-free for fragment reads that take one chunk from each of 16
// consecutive rows (64 banks) or 8 consecutive rows (32 banks).
template <>
struct RowLayout<128> {
  static constexpr int kChunks = 8;
  __device__ static int off(int r, int c) { return r * 128 + (swizzle_chunk(r, c) << 4); }
  __device__ static int pos(int r, int c) { return swizzle_chunk(r, c); }
};

// 256-byte rows: 16 chunks; the chunk position XORs the row's low 4 bits,
// so the 16 consecutive rows one 16-lane group of a fragment read touches
// (one chunk each) sit on distinct chunk positions: conflict-free at 64
// banks, and at 32 banks for every 8 consecutive rows.  Longer rows let one
// stage take 256 contiguous bytes of each operand row from HBM.
template <>
struct RowLayout<256> {
  static constexpr int kChunks = 16;
  __device__ static int off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
  __device__ static int pos(int r, int c) { return c ^ (r & 15); }
};

// 64-byte rows: 4 chunks; pairs of rows share a 128-byte line.  The chunk
// position XORs a 2-bit function of the line chosen so that rows m, m+4,
// m+8, m+12 (which share banks at 64 banks) and rows of one parity among 8
// consecutive rows (at 32 banks) all land on distinct chunk positions.
template <>
struct RowLayout<64> {
  static constexpr int kChunks = 4;
  __device__ static int f(int r) {
    const int L = r >> 1;
    return ((((L >> 1) ^ (L >> 2)) & 1) << 1) | ((L ^ (L >> 1)) & 1);
  }
  __device__ static int off(int r, int c) { return r * 64 + ((c ^ f(r)) << 4); }
  __device__ static int pos(int r, int c) { return c ^ f(r); }
};

// CPOL: cache policy of the operand loads (see lds_dma_16; 5: A default, B
// non-temporal).  SPLIT: waves 0 and 1 load only A, waves 2 and 3 only B
// (needs BM == BN); by default every wave loads its share of both.  These
// two are ablation knobs.
//
// BKN: B is stored K x N row-major (N contiguous, int8) instead of
// K-contiguous.  A stage then holds ROWB k-rows of the tile's BN columns of
// B, copied with the same coalesced 1 KiB direct-to-LDS loads (16 lanes per
// 256-byte k-row), and the MFMA's B fragments are read back transposed with
// ds_read_b64_tr_b8.  Within each group of 16 lanes that instruction gives
// lane 8h + c byte c of the eight 8-byte rows addressed by lanes 2b + h
// (b = 0..7); so lane l, addressing k-row 16 (l/32) + b (+8 for the second
// read) at columns (l/16 % 2) 16 + 8h, receives 8 consecutive k of column
// l % 32, in the k order of the A fragment.  16-byte chunks of k-row k are
// XOR-swizzled by 2k, which puts the eight rows one read touches on
// distinct banks.
//
// LSTEPS: the number of K-steps at the start of a stage over which the next
// stage's loads are issued (0: all but the last K-step).  NTC: C is written
// with non-temporal stores.  BSPLIT: MFMAs of the last K-step issued before
// the stage barrier (0: half).
//
// HIL: in a K-step that issues loads, pin one MFMA in front of each load
// (the scheduler does not see the inline-asm loads as memory reads, so left
// alone it issues a K-step's loads back to back ahead of its MFMAs).  int4
// then expands a K-step's operands once, before the pinned MFMAs.
//
// PF: during stage s, after the loads of stage s + STAGES - 1, touch one word
// of every operand row's stage s + STAGES chunk (one 64-row load per 64 rows,
// into a 256-byte LDS sink), so that the chunk's lines are on their way to
// the L2 one stage before the real loads ask for them.
//
// I4MODE (int4 only): bit 0, wide fragment reads: one ds_read_b128 takes 32
// packed bytes (two MFMA K-steps) of a row, which feed two MFMAs per
// accumulator block, instead of one ds_read_b64 per K-step; bit 1, the
// sign-extending expansion (expand_int4_sx) instead of the x16-scaled one;
// bit 2, the biased expansion: XOR 0x8 turns every nibble into u = v + 8 in
// [0, 15], which needs no sign handling (lo = t & 0x0F0F0F0F, hi = (t >> 4)
// & 0x0F0F0F0F), and the MFMA sums u_a u_b; since (u_a - 8)(u_b - 8) =
// u_a u_b - 8 u_a - 8 u_b + 64, the epilogue subtracts 8 times each row's
// and each column's sum of u (kept per lane with v_dot8_u32_u4 against
// 0x11111111 as the fragments pass) and adds 64 per k summed.  Zero padding
// past K reads as v = 0, u = 8, and contributes 64 - 64 - 64 + 64 = 0.
//
// EARLY (with pinned loads, two stages): the first half of stage s + 2's
// loads go out in stage s's last K-step, right after the barrier that frees
// stage s's buffer, one behind each MFMA left in that K-step; the second
// half in stage s + 1's first K-step.  The loads then leave about a K-step
// earlier than with LSTEPS = 2.
//
// PERSIST: a persistent grid (at most one workgroup per CU, launched with
// the number of workgroups in gridDim.x) in which each workgroup walks its
// tiles round by round, tile r·G + (its logical id) in round r, so that a
// round covers the same tiles, on the same XCDs, as one wave of a
// one-tile-per-workgroup launch.  The stage after a tile's last one is the
// next tile's first: its loads go out during the last stage like any other,
// so the next tile's operands are on their way while this tile's C is
// staged and stored, and the next tile's first fragments are read before
// the epilogue.  The epilogue therefore stages 32 rows per wave at a time
// and keeps clear of the LDS stage those loads fill.  Two stages only.
//
// SPK: split-K.  Workgroup (x, y) of a grid of tiles x p.splits sums the
// y-th of p.splits contiguous runs of the tile's K-stages.  Every workgroup
// writes its raw accumulators to its own slot of p.split_part (each lane its
// registers, in register order, so no layout is involved), publishes them
// with a device-scope release and counts itself in at the tile's counter;
// the one that arrives last (an acquire, no waiting) resets the counter to
// zero for the next launch, adds the slots in split order (fp16: a fixed
// order, so the result does not depend on which workgroup came last) and
// runs the epilogue on the sum.  Nothing waits for another workgroup, so no
// workgroup can be held up by one that is not resident.  p.splits = 1 is
// the plain kernel.
template <int KIND, int BM, int BN, int STAGES, int ROWB, int CPOL = 0, bool SPLIT = false,
          bool BKN = false, int LSTEPS = 0, bool NTC = false, int BSPLIT = 0, bool PF = false,
          bool HIL = false, bool PERSIST = false, int I4MODE = 0, bool EARLY = false, bool SPK = false>
__global__ __launch_bounds__(256) void gemm_v3(GemmArgs p) {
  using Acc = typename KindTraits<KIND>::Acc;
  using Layout = RowLayout<ROWB>;
  constexpr bool I4 = KIND == KIND_I4;
  constexpr bool E3M2 = KIND == KIND_I4_E3M2;
  constexpr bool W4 = I4 && (I4MODE & 1) != 0;   // wide int4 fragment reads
  constexpr bool SX = I4 && (I4MODE & 2) != 0;   // sign-extending int4 expansion
  constexpr bool BIAS = I4 && (I4MODE & 4) != 0; // biased int4 expansion with sum corrections
  static_assert(I4MODE == 0 || I4, "int4 knobs");
  static_assert(!BIAS || (!SX && !PERSIST && !HIL), "one expansion; the biased one on the plain kernel");
  static_assert(!W4 || !HIL, "wide int4 reads keep the compiler's load placement");
  // MFMAs per accumulator block per K-step
  constexpr int kSub = W4 ? 2 : 1;
  // row bytes one K-step consumes: 32 packed int4 (16 B) expand to one int8
  // MFMA step (wide reads: 32 B, two MFMA steps); an E3M2 step is 64 values
  // in two 32-byte groups
  constexpr int kStepBytes = I4 ? (W4 ? 32 : 16) : (E3M2 ? 64 : 32);
  constexpr int KSTEPS = ROWB / kStepBytes;
  // the two fragment buffers alternate per K-step and the next stage's first
  // step reads into buffer 0 again, so a stage needs an even number of steps
  static_assert(KSTEPS % 2 == 0, "K-steps per stage must be even");
  static_assert(!BKN || KIND == KIND_I8 || KIND == KIND_I8_DEQUANT, "K x N storage of B is int8 only");
  static_assert(!BKN || !SPLIT, "one ablation at a time");
  // int4 with pinned loads expands a K-step's operands once, ahead of the
  // pinned MFMAs, so that they are not rebuilt between scheduling barriers
  constexpr bool kOnce = HIL && I4;
  // wave layout: 2 x 2 quadrants, or, for tiles whose width is an odd
  // multiple of 32 columns (224: N = 64 x 224 = 14336), four row bands of
  // the full width
  constexpr int kWavesN = BN % 64 == 0 ? 2 : 1;
  constexpr int WTM = BM / (4 / kWavesN), WTN = BN / kWavesN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM % 2 == 0 && TN >= 1 && BM % 128 == 0 && BN % 32 == 0, "tile");
  constexpr int kRows = BM + BN;
  constexpr int kStage = kRows * ROWB;
  constexpr int kRowsPerLoad = 1024 / ROWB;          // rows one 1 KiB wave load fills
  constexpr int kLoads = kRows / kRowsPerLoad;       // 1 KiB loads per stage
  static_assert(kLoads % 4 == 0 && (BM / kRowsPerLoad) % 4 == 0, "loads per wave");
  constexpr int kSlots = kLoads / 4;                 // per wave per stage
  constexpr int kSlotsA = BM / kRowsPerLoad / 4;
  static_assert((STAGES - 2) * kSlots <= 63, "vmcnt range");
  constexpr int kMainLds = STAGES * kStage;
  // epilogue staging: per wave 64 rows (32 when persistent; half as many for
  // 224-column rows) of WTN 4-byte values plus 32 B padding
  constexpr int kEpiPitch = WTN * 4 + 32;
  constexpr int kEpiRows = (PERSIST ? 32 : 64) / (WTN > 128 ? 2 : 1);
  constexpr int kEpiWave = kEpiRows * kEpiPitch;
  constexpr int kEpiLds = 4 * kEpiWave;
  static_assert(!PERSIST || (STAGES == 2 && !PF && !BKN && !SPLIT && KIND != KIND_I8_MOD), "persistent variant");
  static_assert(!SPK || (!PERSIST && !BIAS && !BKN && !PF && KIND != KIND_I8_MOD && KIND != KIND_I4_E3M2),
                "split-K variant");
  // persistent: the epilogue avoids the stage the next tile's first loads
  // fill.  Stage 0 in flight: the four waves stage in [kStage, kStage +
  // kEpiLds).  Stage 1 in flight: waves 0-2 stage in stage 0's space, wave 3
  // past the ring.
  static_assert(!PERSIST || (3 * kEpiWave <= kStage && kStage + kEpiLds <= kMainLds + kEpiWave), "staging");
  constexpr int kLds0 = PERSIST ? kMainLds + kEpiWave : (kMainLds > kEpiLds ? kMainLds : kEpiLds);
  // prefetch: 64-row touches per wave per stage, and their LDS sink
  static_assert(!PF || (!BKN && BM % 64 == 0 && (BM + BN) % 256 == 0), "prefetch rows");
  constexpr int kPf = PF ? (BM + BN) / 256 : 0;
  constexpr int kLds = kLds0 + (PF ? 256 : 0);
  static_assert(kLds <= 160 * 1024, "LDS");
  static_assert((STAGES - 2) * kSlots + kPf <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;

  // this workgroup's (first) tile; persistent: round r takes logical tile
  // r G + xcd_logical(workgroup)
  const int ntiles = p.tiles_m * p.tiles_n;
  int logical = PERSIST ? xcd_logical(blockIdx.x, gridDim.x) : 0;
  int tm, tn;
  if constexpr (PERSIST) tile_of(p, logical, tm, tn);
  else tile_coords(p, tm, tn);
  int m0 = tm * BM, n0 = tn * BN;
  // split-K: this workgroup's run of K-stages [kb, kb + nks)
  const int split = SPK ? (int)blockIdx.y : 0;
  const int kb = SPK ? (int)(((int64_t)split * p.k_stages) / p.splits) : 0;
  const int nks = SPK ? (int)(((int64_t)(split + 1) * p.k_stages) / p.splits) - kb
                      : p.k_stages;   // 0 when K = 0: C is written as zeros
  // buffer resources over a tile's A and B row panels
  auto panel_a = [&](int mm0) -> i32x4 {
    return make_rsrc(p.A + (size_t)mm0 * p.row_bytes, min(BM, p.M - mm0) * p.row_bytes);
  };
  auto panel_b = [&](int nn0) -> i32x4 {
    return make_rsrc(p.B + (size_t)nn0 * p.row_bytes, min(BN, p.N - nn0) * p.row_bytes);
  };
  i32x4 rsrc_a = panel_a(m0);
  // K-contiguous B: this tile's BN rows; K x N B: the whole matrix (K rows of
  // N bytes, below 2^31 bytes), columns selected per lane
  i32x4 rsrc_b = BKN ? make_rsrc(p.B, (uint32_t)p.row_bytes * (uint32_t)p.N) : panel_b(n0);
  // persistent: the next tile's panels (empty resources, which read as
  // zero, after the last tile)
  int logical_next = logical + (int)gridDim.x;
  i32x4 rsrc_a_next = rsrc_a, rsrc_b_next = rsrc_b;
  auto set_next = [&]() {
    if (logical_next < ntiles) {
      int tm2, tn2;
      tile_of(p, logical_next, tm2, tn2);
      rsrc_a_next = panel_a(tm2 * BM);
      rsrc_b_next = panel_b(tn2 * BN);
    } else {
      rsrc_a_next = make_rsrc(p.A, 0);
      rsrc_b_next = make_rsrc(p.B, 0);
    }
  };
  if constexpr (PERSIST) set_next();
  // parity of the LDS stage holding a tile's first K-stage (persistent: the
  // stages run on across tiles)
  int gbase = 0;
  const uint32_t smem_lds = lds_address(smem);

  // Load slot t of this wave fills stage rows kRowsPerLoad*g .. (g = 4t +
  // wave): lane l writes row kRowsPerLoad*g + l / kChunks at chunk position
  // l % kChunks, so it fetches the global chunk whose swizzled position that is.
  static_assert(!SPLIT || BM == BN, "a split loader gives A and B the same number of waves");
  // slot t of this wave loads row group g (kRowsPerLoad rows; A's groups
  // come first); interleaved: g = 4t + wave, split: waves 0-1 walk A's
  // groups, waves 2-3 B's
  auto group_of = [&](int t) -> int {
    if constexpr (SPLIT) return wave < 2 ? 2 * t + wave : BM / kRowsPerLoad + 2 * t + (wave - 2);
    else return 4 * t + wave;
  };
  auto is_a = [&](int t) -> bool {
    if constexpr (SPLIT) return wave < 2;
    else return t < kSlotsA;
  };
  // K x N B: 16-byte chunks per k-row of the tile, and the chunk swizzle
  constexpr int kBChunks = BN / 16;
  auto b_swz = [](int krow) -> int { return (2 * krow) & (kBChunks - 1); };
  uint32_t slot_off[kSlots];
  uint32_t slot_col[kSlots];   // K-contiguous rows: byte column; K x N B: k-row in the stage
  bool slot_ok[kSlots];        // K x N B: the chunk's columns lie inside N
#pragma unroll
  for (int t = 0; t < kSlots; ++t) {
    const int g = group_of(t);
    if (BKN && !is_a(t)) {
      const int krow = (g - BM / kRowsPerLoad) * (1024 / BN) + lane / kBChunks;
      const int c = (lane % kBChunks) ^ b_swz(krow);
      const int col = n0 + c * 16;
      slot_off[t] = (uint32_t)krow * (uint32_t)p.N + col;
      slot_col[t] = krow;
      slot_ok[t] = col < p.N;
    } else {
      const int lrow = kRowsPerLoad * g + lane / Layout::kChunks;
      const int c = Layout::pos(lrow, lane % Layout::kChunks);   // XOR swizzle is an involution
      const int grow = is_a(t) ? lrow : lrow - BM;
      slot_off[t] = grow * p.row_bytes + c * 16;
      slot_col[t] = c * 16;
      slot_ok[t] = true;
    }
  }

  // stage s of this tile (persistent: s = nks is the next tile's stage 0)
  auto issue_load = [&](int t, int s) {
    const bool next = PERSIST && s >= p.k_stages;
    const uint32_t kbyte = next ? 0u : (uint32_t)(kb + s) * ROWB;
    const int g = group_of(t);
    uint32_t off;
    if (BKN && !is_a(t)) {
      // k-row s*ROWB + krow of B, when inside K
      const bool ok = slot_ok[t] && kbyte + slot_col[t] < (uint32_t)p.row_bytes;
      off = ok ? slot_off[t] + kbyte * (uint32_t)p.N : kOutOfRange;
    } else {
      const bool in_row = kbyte + slot_col[t] < (uint32_t)p.row_bytes;
      off = in_row ? slot_off[t] + kbyte : kOutOfRange;
    }
    const i32x4 ra = next ? rsrc_a_next : rsrc_a;
    const i32x4 rb = next ? rsrc_b_next : rsrc_b;
    // CPOL 5: A with the default policy, B non-temporal
    constexpr int kCpolA = CPOL == 5 ? 0 : CPOL, kCpolB = CPOL == 5 ? 1 : CPOL;
    if (is_a(t)) lds_dma_16<kCpolA>(ra, smem_lds + ((gbase + s) % STAGES) * kStage + g * 1024, off);
    else lds_dma_16<kCpolB>(rb, smem_lds + ((gbase + s) % STAGES) * kStage + g * 1024, off);
  };

  // prefetch touch t of this wave covers operand rows 64 (kPf wave + t) ..
  // + 63 (A's rows first), one row per lane, at the row's first word of the
  // stage's chunk
  auto issue_prefetch = [&](int s) {
    const uint32_t kbyte = (uint32_t)s * ROWB;
#pragma unroll
    for (int t = 0; t < kPf; ++t) {
      const int r = 64 * (kPf * wave + t) + lane;
      const bool a_rows = 64 * (kPf * wave + t) < BM;
      const uint32_t off = kbyte < (uint32_t)p.row_bytes
                               ? (uint32_t)(a_rows ? r : r - BM) * (uint32_t)p.row_bytes + kbyte
                               : kOutOfRange;
      lds_dma_4(a_rows ? rsrc_a : rsrc_b, smem_lds + kLds0, off);
    }
  };

  // Fragment addressing: lane l reads row (l & 31) of a 32-row block; blocks
  // start at multiples of 32 rows, which leaves the swizzle unchanged.
  const int fr = lane & 31, fh = lane >> 5;
  const int a_row_base = (wm * WTM) * ROWB;
  const int b_row_base = (BM + wn * WTN) * ROWB;
  auto frag_off = [&](int kk) -> int {
    if constexpr (I4 && !W4) return Layout::off(fr, kk) + fh * 8;   // 8 packed bytes
    else if constexpr (E3M2) return Layout::off(fr, 4 * kk + 2 * fh);   // group, first chunk
    else return Layout::off(fr, 2 * kk + fh);                     // 16 bytes
  };
  // E3M2: the group's second chunk holds codes in its first 8 bytes (the
  // other 8 are padding and are not read)
  auto frag_off2 = [&](int kk) -> int { return Layout::off(fr, 4 * kk + 2 * fh + 1); };

  // E3M2 fragments are read straight into the eight-dword MFMA operand (of
  // which the FP6 format uses the low six)
  using Raw = typename std::conditional<I4 && !W4, i32x2_t,
                                        typename std::conditional<E3M2, i32x8, i32x4>::type>::type;
  using Op = typename std::conditional<E3M2, i32x8, i32x4>::type;
  auto e3m2_frag = [](const uint8_t* p0, const uint8_t* p1) -> i32x8 {
    const i32x4 lo = *(const i32x4*)p0;
    const i32x2_t hi = *(const i32x2_t*)p1;
    return __builtin_shufflevector(lo, __builtin_shufflevector(hi, hi, 0, 1, -1, -1), 0, 1, 2, 3, 4, 5, 6, 7);
  };
  Raw fa[2][TM], fb[2][TN];

  // K x N B: this lane's transposed-read addresses within the B region, per
  // K-step and n-block (the two reads are 8 k-rows apart; the swizzle of
  // k-row k and k + 8 is the same)
  const int tr_b = (lane % 16) / 2, tr_h = lane % 2, tr_g = lane / 16;
  auto b_tr_off = [&](int kk, int j) -> int {
    const int krow = 32 * kk + 16 * (tr_g / 2) + tr_b;
    const int ncol = wn * WTN + 32 * j + (16 * tr_g + 8 * tr_h) % 32;
    return krow * BN + (((ncol / 16) ^ b_swz(krow)) << 4) + (ncol % 16);
  };

  auto read_frags = [&](int s, int kk, int dst) {
    const uint8_t* base = smem + ((gbase + s) % STAGES) * kStage;
    const int off = frag_off(kk);
    if constexpr (BKN) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[dst][i] = *(const Raw*)(base + a_row_base + i * 32 * ROWB + off);
      typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint8_t* pb = base + BM * ROWB + b_tr_off(kk, j);
        const i32x2_t lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_address(pb)));
        const i32x2_t hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_address(pb + 8 * BN)));
        fb[dst][j] = i32x4{lo.x, lo.y, hi.x, hi.y};
      }
    } else if constexpr (E3M2) {
      const int off2 = frag_off2(kk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[dst][i] = e3m2_frag(base + a_row_base + i * 32 * ROWB + off, base + a_row_base + i * 32 * ROWB + off2);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[dst][j] = e3m2_frag(base + b_row_base + j * 32 * ROWB + off, base + b_row_base + j * 32 * ROWB + off2);
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[dst][i] = *(const Raw*)(base + a_row_base + i * 32 * ROWB + off);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[dst][j] = *(const Raw*)(base + b_row_base + j * 32 * ROWB + off);
    }
  };

  // MFMA operand h (0 .. kSub-1) of a raw fragment
  auto operand = [&](const Raw& r, int h = 0) -> Op {
    if constexpr (I4) {
      uint32_t lo0, hi0, lo1, hi1;
      const uint32_t d0 = (uint32_t)r[2 * h], d1 = (uint32_t)r[2 * h + 1];
      if constexpr (SX) {
        expand_int4_sx(d0, lo0, hi0);
        expand_int4_sx(d1, lo1, hi1);
      } else if constexpr (BIAS) {
        const uint32_t t0 = d0 ^ 0x88888888u, t1 = d1 ^ 0x88888888u;
        lo0 = t0 & 0x0F0F0F0Fu;
        hi0 = (t0 >> 4) & 0x0F0F0F0Fu;
        lo1 = t1 & 0x0F0F0F0Fu;
        hi1 = (t1 >> 4) & 0x0F0F0F0Fu;
      } else {
        expand_int4(d0, lo0, hi0);
        expand_int4(d1, lo1, hi1);
      }
      return i32x4{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
    } else {
      return r;
    }
  };

  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // biased int4: per lane, the running sum of u over its row (A) or column
  // (B) of each block and its half of every K-step
  uint32_t usum_a[TM], usum_b[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) usum_a[i] = 0;
#pragma unroll
  for (int j = 0; j < TN; ++j) usum_b[j] = 0;
  auto add_usums = [&](int src) {
    if constexpr (BIAS) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int d = 0; d < 2; ++d)
          usum_a[i] = __builtin_amdgcn_udot8((uint32_t)fa[src][i][d] ^ 0x88888888u, 0x11111111u, usum_a[i], false);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int d = 0; d < 2; ++d)
          usum_b[j] = __builtin_amdgcn_udot8((uint32_t)fb[src][j][d] ^ 0x88888888u, 0x11111111u, usum_b[j], false);
    }
  };

  // MFMAs first .. last-1 of a K-step on operands already in MFMA form
  auto compute_ops = [&](const Op (&a)[TM], const Op (&b)[TN], int first, int last) {
#pragma unroll
    for (int x = 0; x < TM * TN; ++x) {
      if (x < first || x >= last) continue;
      const int i = x / TN, j = x % TN;
      if constexpr (E3M2) acc[i][j] = mfma_e3m2(a[i], b[j], acc[i][j]);
      else acc[i][j] = mfma<KIND>(a[i], b[j], acc[i][j]);
    }
  };
  // ... on fragment buffer src, converted here (int4: expanded to int8; wide
  // int4 reads: both halves of each fragment, one MFMA each)
  auto compute = [&](int src, int first, int last) {
#pragma unroll
    for (int h = 0; h < kSub; ++h) {
      Op a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = operand(fa[src][i], h);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = operand(fb[src][j], h);
      compute_ops(a, b, first, last);
    }
  };

  constexpr int kMfma = TM * TN;
  constexpr int kSplit = BSPLIT > 0 ? BSPLIT : kMfma / 2;
  static_assert(kSplit > 0 && kSplit < kMfma, "barrier split");
  constexpr int kReads = (E3M2 ? 2 : 1) * (TM + TN);   // DS read instructions per K-step
  // loads of one stage are spread over K-steps 0 .. kLoadSteps-1
  constexpr int kLoadSteps = LSTEPS > 0 ? LSTEPS : (KSTEPS > 1 ? KSTEPS - 1 : 1);
  static_assert(kLoadSteps < KSTEPS || KSTEPS == 1, "loads end before the stage's last K-step");
  constexpr int kLoadsPerStep = (kSlots + kLoadSteps - 1) / kLoadSteps;
  static_assert(!EARLY || (STAGES == 2 && HIL && !kOnce && !PERSIST && !PF && !BKN && !SPLIT), "early loads");
  // early loads: slots t < kHead of a stage go out in the stage two before
  // it (after its barrier), the others in the stage before it (K-step 0)
  constexpr int kHead = EARLY ? kSlots / 2 : 0;
  static_assert(!EARLY || kHead <= kMfma - kSplit, "one MFMA in front of each early load");
  auto interleave = [&](int mfmas, int reads, int loads) {
#pragma unroll
    for (int x = 0; x < kMfma; ++x) {
      if (x >= mfmas) break;
      __builtin_amdgcn_sched_group_barrier(0x008, kSub, 0);               // MFMA
      if (x < reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      if (x < loads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
    }
  };

  // the prefetch of stage s + STAGES is issued in this K-step of stage s,
  // after the stage's own loads
  constexpr int kPfStep = kLoadSteps < KSTEPS - 1 ? kLoadSteps : KSTEPS - 1;
  if (nks > 0) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
#pragma unroll
      for (int t = 0; t < kSlots; ++t) issue_load(t, s);
    if constexpr (PF) issue_prefetch(STAGES - 1);
    if constexpr (EARLY) {
#pragma unroll
      for (int t = 0; t < kHead; ++t) issue_load(t, 1);   // stage 1's early half
    }
    wait_vmcnt<(STAGES - 2) * kSlots + kPf + kHead>();   // own loads of stage 0
    block_barrier();                             // everyone's
    read_frags(0, 0, 0);
  }
  for (;;) {   // tiles: one pass, or every round's tile of a persistent workgroup
  for (int s = 0; s < nks; ++s) {
    // loads for stage s + STAGES - 1 (past the last stage they only write
    // zeros that nobody reads, or, persistent, fill the next tile's stage 0)
    const int sl = s + STAGES - 1;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int src = kk & 1, dst = src ^ 1;
      add_usums(src);
      Op ea[TM], eb[TN];
      if constexpr (kOnce) {
#pragma unroll
        for (int i = 0; i < TM; ++i) ea[i] = operand(fa[src][i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) eb[j] = operand(fb[src][j]);
      }
      auto mm = [&](int first, int last) {
        if constexpr (kOnce) compute_ops(ea, eb, first, last);
        else compute(src, first, last);
      };
      int nl = 0;
      int pre = 0;   // MFMAs already issued in front of this K-step's loads
      if (EARLY ? kk == 0 : kk < kLoadSteps) {
#pragma unroll
        for (int t = 0; t < kSlots; ++t) {
          if (EARLY ? t < kHead : t / kLoadsPerStep != kk) continue;
          if constexpr (HIL) {
            if (pre < (kk + 1 < KSTEPS ? kMfma : kSplit)) {
              mm(pre, pre + 1);
              ++pre;
              __builtin_amdgcn_sched_barrier(0);
            }
            issue_load(t, sl);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            issue_load(t, sl);
            ++nl;
          }
        }
      }
      if constexpr (PF) {
        if (kk == kPfStep) {
          issue_prefetch(s + STAGES);
          nl += kPf;
        }
      }
      if (kk + 1 < KSTEPS) {
        read_frags(s, kk + 1, dst);
        mm(pre, kMfma);
        interleave(kMfma - pre, kReads, nl);
      } else {
        mm(pre, kSplit);
        interleave(kSplit - pre, 0, nl);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(STAGES - 2) * kSlots + kPf>();   // own loads of stage s+1 landed
        wait_lgkmcnt0();                       // own reads of stage s done
        block_barrier();                       // ... everyone's
        read_frags(s + 1, 0, dst);
        if constexpr (EARLY) {
          // stage s's buffer is free: the early half of stage s + 2, one
          // load behind each of the K-step's remaining MFMAs
#pragma unroll
          for (int t = 0; t < kHead; ++t) {
            mm(kSplit + t, kSplit + t + 1);
            __builtin_amdgcn_sched_barrier(0);
            issue_load(t, s + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        mm(kSplit + kHead, kMfma);
        // (early loads: the next stage's first fragment reads went out before
        // the pinned loads)
        interleave(kMfma - kSplit - kHead, EARLY ? 0 : kReads, 0);
      }
    }
  }

  // ------------------------------------------------------------------ epilogue
  // Element e of lane l in a 32x32 block is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32 of the block.
  // biased int4: each row's and column's whole sum of u (lanes l and l + 32
  // summed the two halves of every K-step)
  int usum_tot_a[TM], usum_tot_b[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) usum_tot_a[i] = BIAS ? (int)usum_a[i] + __shfl_xor((int)usum_a[i], 32) : 0;
#pragma unroll
  for (int j = 0; j < TN; ++j) usum_tot_b[j] = BIAS ? (int)usum_b[j] + __shfl_xor((int)usum_b[j], 32) : 0;
  // The value a lane stages for accumulator element e of block (i, j); the
  // dequant kind stages the raw sum and scales it when storing
  auto value = [&](int i, int j, int e) -> uint32_t {
    if constexpr (KIND == KIND_F16) {
      return __builtin_bit_cast(uint32_t, (float)acc[i][j][e]);
    } else if constexpr (E3M2) {
      return (uint32_t)(int32_t)acc[i][j][e];   // an integer below 2^24: exact
    } else if constexpr (BIAS) {
      // sum of (u_a - 8)(u_b - 8) over every k summed (nks stages of 2 ROWB
      // values)
      const int r = 8 * (e >> 2) + 4 * fh + (e & 3);   // row within block i
      const int row_sum = __shfl(usum_tot_a[i], r);
      return (uint32_t)(acc[i][j][e] - 8 * row_sum - 8 * (int)usum_tot_b[j] + 64 * 2 * ROWB * nks);
    } else if constexpr (KIND == KIND_I4 && !SX) {
      return (uint32_t)(acc[i][j][e] >> 8);   // undo the 16 x 16 scaling
    } else {
      return (uint32_t)acc[i][j][e];
    }
  };

  // Outstanding loads (all past the last stage) must land before LDS is
  // reused; the barrier then also covers every wave's fragment reads.
  // Persistent: the last K-step already waited for every load (the next
  // tile's stage 0) and its barrier followed every wave's last reads of the
  // stage the staging reuses; the staging keeps clear of the next tile's
  // stage 0, which the fragment reads of its first K-step are reading.
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  if constexpr (SPK) {
    if (p.splits > 1) {
      // The tile's slots, split sp at sp * kSlotBytes: 4 waves x TM*TN
      // blocks x 4 quads x 64 lanes of 16 bytes; a lane's quad q of block b
      // is its accumulator elements 4q .. 4q + 3.
      //
      // Publishing without cache flushes: the slots are written and read
      // with device-scope (sc1) accesses, the form device-scope relaxed
      // atomics take on this chip, which write through to the device's
      // coherence point and read from it.  A workgroup waits until its
      // stores are acknowledged (vmcnt 0) before it counts itself in with a
      // device-scope atomic, and the last arrival reads the slots only after
      // that atomic has returned, so every slot it reads is complete.  (A
      // device-scope release/acquire pair would write back and invalidate
      // the whole L2 around each arrival, which costs far more than the
      // split saves.)
      constexpr int kSlotBytes = 4 * TM * TN * 16 * 64 * 4;
      constexpr int kSc1 = 16;   // cache-policy bits: device scope
      const int tile = (int)blockIdx.x;
      const __amdgpu_buffer_rsrc_t slots = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.split_part + (size_t)tile * p.splits * (kSlotBytes / 4)), 0, p.splits * kSlotBytes,
          kBufferWord3);
      auto slot_off = [&](int sp, int i, int j, int q) -> int {
        return sp * kSlotBytes + (((wave * TM + i) * TN + j) * 4 + q) * 1024 + lane * 16;
      };
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            i32x4 v;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              // (a vector element is not an object: copy it before the bit cast)
              const auto e = acc[i][j][4 * q + x];
              v[x] = __builtin_bit_cast(int, e);
            }
            __builtin_amdgcn_raw_buffer_store_b128(v, slots, slot_off(split, i, j, q), 0, kSc1);
          }
      __shared__ uint32_t arrived;
      wait_vmcnt<0>();   // this wave's slot stores acknowledged
      block_barrier();   // ... every wave's
      if (tid == 0) arrived = __hip_atomic_fetch_add(p.split_count + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_lgkmcnt0();
      block_barrier();
      if (arrived != (uint32_t)(p.splits - 1)) return;
      // the last arrival: the counter back to zero for the next launch, then
      // the sum in split order, this workgroup's own part from its registers
      if (tid == 0) __hip_atomic_store(p.split_count + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // one batch of loads per other split (a single wait for each), added
      // into the running sum in split order
      Acc_elem4<Acc> sum[TM][TN][4];
      for (int sp = 0; sp < p.splits; ++sp) {
        i32x4 part[TM][TN][4];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (sp == split) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                  const auto e = acc[i][j][4 * q + x];
                  part[i][j][q][x] = __builtin_bit_cast(int, e);
                }
              } else {
                part[i][j][q] = __builtin_amdgcn_raw_buffer_load_b128(slots, slot_off(sp, i, j, q), 0, kSc1);
              }
            }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) sum[i][j][q].add(part[i][j][q], sp == 0);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[i][j][4 * q + x] = sum[i][j][q].get(x);
    }
  }
  if constexpr (KIND != KIND_I8_MOD) {
    // Every kind but the reduced one goes through LDS: each wave transposes
    // kEpiRows rows of its quadrant at a time so that a lane holds 4
    // consecutive columns of one row.  A tile inside C whose rows start
    // 16-byte aligned (N % 4 == 0) writes them with 16-byte stores; an edge
    // tile writes each value inside C with its own 4-byte store.
    const bool full = m0 + BM <= p.M && n0 + BN <= p.N && (p.N & 3) == 0;
    int stage_off = wave * kEpiWave;
    if constexpr (PERSIST) {
      const bool next_in_0 = (gbase + nks) % STAGES == 0;
      stage_off = next_in_0 ? kStage + wave * kEpiWave : (wave < 3 ? wave * kEpiWave : 2 * kStage);
    } else {
      block_barrier();   // every wave is done with the operand stages
    }
    uint8_t* stage_out = smem + stage_off;
    const int row0 = m0 + wm * WTM;
    const int col0 = n0 + wn * WTN;
    // each lane stores 16 bytes; lanes 0..WTN/4-1 cover one row (a row of
    // 224 columns: lanes 0-55 store, 56-63 read row 0 and store nothing)
    constexpr int kLanesPerRow = WTN / 4;
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    constexpr bool kAllLanes = 64 % kLanesPerRow == 0;
    const bool lane_on = kAllLanes || lane < kRowsPerStore * kLanesPerRow;
    const int lane_row = lane_on ? lane / kLanesPerRow : 0;
    const int c_lane = (lane % kLanesPerRow) * 4;
    // dequant: the column scales of this lane's four output columns (the
    // same in every row it stores; zero outside C)
    float cs4[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KIND == KIND_I8_DEQUANT) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (col0 + c_lane + x < p.N) cs4[x] = p.col_scale[col0 + c_lane + x];
    }
    static_assert(WTM % kEpiRows == 0 && kEpiRows % 8 == 0, "epilogue passes");
#pragma unroll
    for (int half = 0; half < WTM / kEpiRows; ++half) {
      // pass `half` stages the wave's rows half*kEpiRows .. + kEpiRows - 1:
      // the accumulator elements whose 8-row group (block i, element e / 4)
      // falls there
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rg = i * 32 + 8 * (e >> 2);
            if (rg / kEpiRows != half) continue;
            const int r = rg - half * kEpiRows + 4 * fh + (e & 3);
            const int c = j * 32 + fr;
            // dequant: the raw sums go through LDS; the scales are applied
            // as the rows are stored
            *(uint32_t*)(stage_out + r * kEpiPitch + c * 4) =
                KIND == KIND_I8_DEQUANT ? (uint32_t)acc[i][j][e] : value(i, j, e);
          }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes done
      // dequant: lane l holds the scale of row l of these kEpiRows (zero
      // outside C); each store's rows take theirs by lane index
      float rs_half = 0.f;
      if constexpr (KIND == KIND_I8_DEQUANT) {
        const int rl = row0 + half * kEpiRows + lane;
        if (lane < kEpiRows && rl < p.M) rs_half = p.row_scale[rl];
      }
      // the staged rows of this pass, kRowsPerStore per read: a group of
      // reads is issued back to back and only then stored, so that the
      // reads' LDS latency is paid once per group rather than once per row
      constexpr int kReadsPerPass = kEpiRows / kRowsPerStore;
      constexpr int kGroup = kReadsPerPass < 16 ? kReadsPerPass : 16;
      static_assert(kReadsPerPass % kGroup == 0, "read groups");
      const int gcol = col0 + c_lane;
      auto scaled = [&](i32x4 v, int r0) -> i32x4 {
        if constexpr (KIND == KIND_I8_DEQUANT) {
          // ((float)acc * row_scale) * col_scale, each product rounded once
          float rs = 0.f;
#pragma unroll
          for (int q = 0; q < kRowsPerStore; ++q) {
            const float sq = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs_half), r0 + q));
            if (lane_row == q) rs = sq;
          }
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            float t = (float)v[x];
            t = t * rs;
            t = t * cs4[x];
            v[x] = __builtin_bit_cast(int, t);
          }
        }
        return v;
      };
      if constexpr (I4) {
        // int4: one row at a time (its main loop already holds 256 VGPRs)
#pragma unroll
        for (int r0 = 0; r0 < kEpiRows; r0 += kRowsPerStore) {
          const int r = r0 + lane_row;
          i32x4 v = *(const i32x4*)(stage_out + r * kEpiPitch + c_lane * 4);
          const int grow = row0 + half * kEpiRows + r;
          uint32_t* dst = (uint32_t*)p.C + (size_t)grow * p.N + gcol;
          if (!lane_on) {
          } else if (full) {
            if constexpr (NTC) __builtin_nontemporal_store(v, (i32x4*)dst);
            else *(i32x4*)dst = v;
          } else if (grow < p.M) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
              if (gcol + x < p.N) dst[x] = (uint32_t)v[x];
          }
        }
      } else if (full) {
#pragma unroll
        for (int g = 0; g < kReadsPerPass; g += kGroup) {
          i32x4 v[kGroup];
#pragma unroll
          for (int q = 0; q < kGroup; ++q) {
            const int r = (g + q) * kRowsPerStore + lane_row;
            v[q] = *(const i32x4*)(stage_out + r * kEpiPitch + c_lane * 4);
          }
#pragma unroll
          for (int q = 0; q < kGroup; ++q) {
            const int r0 = (g + q) * kRowsPerStore;
            const i32x4 w = scaled(v[q], r0);
            const int grow = row0 + half * kEpiRows + r0 + lane_row;
            i32x4* dst = (i32x4*)((uint32_t*)p.C + (size_t)grow * p.N + gcol);
            if (lane_on) {
              if constexpr (NTC) __builtin_nontemporal_store(w, dst);
              else *dst = w;
            }
          }
        }
      } else {
#pragma unroll
        for (int r0 = 0; r0 < kEpiRows; r0 += kRowsPerStore) {
          const int r = r0 + lane_row;
          const i32x4 v = scaled(*(const i32x4*)(stage_out + r * kEpiPitch + c_lane * 4), r0);
          const int grow = row0 + half * kEpiRows + r;
          uint32_t* dst = (uint32_t*)p.C + (size_t)grow * p.N + gcol;
          if (lane_on && grow < p.M) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
              if (gcol + x < p.N) dst[x] = (uint32_t)v[x];
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the next half overwrites
    }
  } else {
    // the reduced kind: one byte per value, straight from the accumulators
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WTN + j * 32 + fr;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
          if (col < p.N && row < p.M) {
            {
              // the non-negative residue: |acc| < 2^31 is exact in double, q
              // from the rounded reciprocal is within one of floor(acc / m),
              // fma(-q, m, acc) is exact, and one correction each way ends it
              const double x = (double)(int32_t)acc[i][j][e], m = (double)p.modulus;
              double r = fma(-floor(x * p.inv_modulus), m, x);
              if (r < 0.0) r += m;
              if (r >= m) r -= m;
              ((uint8_t*)p.C)[(size_t)row * p.N + col] = (uint8_t)(int)r;
            }
          }
        }
      }
    }
  }
  if constexpr (!PERSIST) {
    break;
  } else {
    if (logical_next >= ntiles) break;
    // every wave's staging reads are done before the next tile's stage-1
    // loads refill that space
    block_barrier();
    logical = logical_next;
    logical_next += (int)gridDim.x;
    tile_of(p, logical, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    rsrc_a = rsrc_a_next;
    rsrc_b = rsrc_b_next;
    set_next();
    gbase = (gbase + nks) % STAGES;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
  }
  }   // tiles
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel for short M (the LLM projection's 128-token band).
//
// With M <= BM the whole of A is a few hundred KiB that every workgroup
// needs, while each workgroup streams its own BN rows of B from HBM, once.
// How fast B arrives is set by how many of its bytes each CU keeps in
// flight: a ring whose stages hold A and B together (the tiled kernels)
// spends two thirds of the LDS on A, which comes from L2 at short latency,
// and leaves B two stages (32 KiB) in flight.  Here A and B get rings of
// their own, of different depths, filled by different waves: the vector
// memory counter retires a wave's loads in issue order, so one wave cannot
// wait for a near A stage without also waiting for the far B stages issued
// before it.  Wave 4 loads A (SA stages of BM rows); waves 0-3 load B (SB
// stages of BN rows) and compute, a 2 x 2 arrangement of (BM/2) x (BN/2)
// quadrants.  One barrier per stage: every wave first waits for its own
// loads of the next stage and for its fragment reads of this one, so past
// the barrier the next stage is whole and this one's buffers are free.  The
// accumulators are stored straight to C (4-byte stores, masked at the
// edges): the tile is small next to the B panel it streams.
template <int KIND, int BM, int BN, int SA, int SB>
__global__ __launch_bounds__(320) void gemm_stream(GemmArgs p) {
  using Acc = typename KindTraits<KIND>::Acc;
  static_assert(KIND == KIND_I8 || KIND == KIND_I8_DEQUANT || KIND == KIND_F16 || KIND == KIND_I4, "kinds");
  constexpr bool I4 = KIND == KIND_I4;
  using Layout = RowLayout<128>;
  // a K-step: 32 row bytes (int4: 16 packed bytes, expanded to one int8 step)
  constexpr int ROWB = 128, KSTEPS = ROWB / (I4 ? 16 : 32);
  constexpr int WTM = BM / 2, WTN = BN / 2, TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "quadrants");
  constexpr int kStageA = BM * ROWB, kStageB = BN * ROWB;
  constexpr int kLoadsA = BM / 8;          // 1 KiB loads of an A stage, all by wave 4
  constexpr int kLoadsB = BN / 8 / 4;      // ... of a B stage, per compute wave
  static_assert(kLoadsB >= 1 && (BN / 8) % 4 == 0, "B loads per wave");
  static_assert((SA - 2) * kLoadsA <= 63 && (SB - 2) * kLoadsB <= 63 && SA >= 2 && SB >= 2, "vmcnt range");
  constexpr int kBaseB = SA * kStageA;
  static_assert(kBaseB + SB * kStageB <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBaseB + SB * kStageB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_coords(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const i32x4 rsrc_a = make_rsrc(p.A + (size_t)m0 * p.row_bytes, min(BM, p.M - m0) * p.row_bytes);
  const i32x4 rsrc_b = make_rsrc(p.B + (size_t)n0 * p.row_bytes, min(BN, p.N - n0) * p.row_bytes);
  const uint32_t smem_lds = lds_address(smem);
  const int nks = p.k_stages;
  const bool loader = wave == 4;

  // load g of a stage fills rows 8g .. 8g + 7: lane l writes row 8g + l / 8
  // at chunk position l % 8, so it fetches the global chunk whose swizzled
  // position that is
  auto chunk_of = [&](int g, uint32_t& off, uint32_t& col) {
    const int row = 8 * g + lane / 8;
    const int c = Layout::pos(row, lane % 8);
    off = (uint32_t)row * (uint32_t)p.row_bytes + c * 16;
    col = c * 16;
  };
  auto issue = [&](int s) {
    const uint32_t kbyte = (uint32_t)s * ROWB;
    if (loader) {
#pragma unroll
      for (int g = 0; g < kLoadsA; ++g) {
        uint32_t off, col;
        chunk_of(g, off, col);
        lds_dma_16(rsrc_a, smem_lds + (s % SA) * kStageA + g * 1024,
                   kbyte + col < (uint32_t)p.row_bytes ? off + kbyte : kOutOfRange);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kLoadsB; ++t) {
        const int g = wave * kLoadsB + t;
        uint32_t off, col;
        chunk_of(g, off, col);
        lds_dma_16(rsrc_b, smem_lds + kBaseB + (s % SB) * kStageB + g * 1024,
                   kbyte + col < (uint32_t)p.row_bytes ? off + kbyte : kOutOfRange);
      }
    }
  };
  // each wave waits for its own loads of stage s + 1 (the loads of the
  // stages after it stay in flight), then for its fragment reads, then meets
  // the others
  auto stage_end = [&]() {
    if (loader) wait_vmcnt<(SA - 2) * kLoadsA>();
    else wait_vmcnt<(SB - 2) * kLoadsB>();
    wait_lgkmcnt0();
    block_barrier();
  };

  const int wm = (wave >> 1) & 1, wn = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;
  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  if (nks > 0) {
    const int pre = loader ? SA - 1 : SB - 1;
    for (int s = 0; s < pre; ++s) issue(s);
    if (loader) wait_vmcnt<(SA - 2) * kLoadsA>();
    else wait_vmcnt<(SB - 2) * kLoadsB>();
    block_barrier();   // stage 0 of A and B has landed
  }
  for (int s = 0; s < nks; ++s) {
    // the stage that reuses the buffers stage s - 1 released at the last barrier
    issue(s + (loader ? SA : SB) - 1);
    if (!loader) {
      const uint8_t* a_base = smem + (s % SA) * kStageA + (wm * WTM) * ROWB;
      const uint8_t* b_base = smem + kBaseB + (s % SB) * kStageB + (wn * WTN) * ROWB;
      auto frag = [&](const uint8_t* p0) -> i32x4 {
        if constexpr (I4) {
          const i32x2_t x = *(const i32x2_t*)p0;
          uint32_t lo0, hi0, lo1, hi1;
          expand_int4((uint32_t)x.x, lo0, hi0);
          expand_int4((uint32_t)x.y, lo1, hi1);
          return i32x4{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
        } else {
          return *(const i32x4*)p0;
        }
      };
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int off = I4 ? Layout::off(fr, kk) + 8 * fh : Layout::off(fr, 2 * kk + fh);
        i32x4 fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = frag(a_base + i * 32 * ROWB + off);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = frag(b_base + j * 32 * ROWB + off);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma<KIND>(fa[i], fb[j], acc[i][j]);
      }
    }
    stage_end();
  }
  wait_vmcnt<0>();   // loads past the last stage (zeros nobody reads)
  if (loader) return;

  // element e of lane l in a 32 x 32 block: row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column l % 32
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + fr;
      float cs = 0.f;
      if constexpr (KIND == KIND_I8_DEQUANT) cs = col < p.N ? p.col_scale[col] : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
        if (row >= p.M || col >= p.N) continue;
        const size_t idx = (size_t)row * p.N + col;
        if constexpr (KIND == KIND_F16) {
          ((float*)p.C)[idx] = acc[i][j][e];
        } else if constexpr (KIND == KIND_I8_DEQUANT) {
          float t = (float)acc[i][j][e];
          t = t * p.row_scale[row];
          t = t * cs;
          ((float*)p.C)[idx] = t;
        } else if constexpr (I4) {
          ((int32_t*)p.C)[idx] = acc[i][j][e] >> 8;   // undo the 16 x 16 scaling
        } else {
          ((int32_t*)p.C)[idx] = acc[i][j][e];
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Reference kernel: the same contraction with nothing tuned.  One LDS stage
// (load, barrier, contract, barrier), operand rows stored unswizzled, plain
// per-lane global loads and 4-byte stores, a 128 x 128 tile of four 64 x 64
// wave quadrants.  It feeds each accumulator the same K-steps, in the same
// order and with the same lane-to-k assignment as the pipelined kernels
// (lane l: row l % 32 of a 32-row block, bytes 16 (l / 32) .. + 15 of a
// 32-byte K-step; packed int4: bytes 8 (l / 32) .. + 7 of a 16-byte step), so
// for fp16 its result must equal theirs bit for bit: the bring-up version
// against which the swizzled, multi-stage kernels are checked.
template <int KIND>
__global__ __launch_bounds__(256) void gemm_ref(GemmArgs p) {
  using Acc = typename KindTraits<KIND>::Acc;
  static_assert(KIND == KIND_I8 || KIND == KIND_I4 || KIND == KIND_F16 || KIND == KIND_I8_DEQUANT, "kinds");
  constexpr bool I4 = KIND == KIND_I4;
  constexpr int BM = 128, BN = 128, ROWB = 128;      // LDS bytes per operand row
  constexpr int kStep = I4 ? 16 : 32;                // row bytes one MFMA K-step consumes
  constexpr int TM = 2, TN = 2;                      // 32 x 32 blocks per wave
  __shared__ __attribute__((aligned(16))) uint8_t sa[BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sb[BN * ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int fr = lane & 31, fh = lane >> 5;

  Acc acc[TM][TN];
  for (int i = 0; i < TM; ++i)
    for (int j = 0; j < TN; ++j)
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  for (int ks = 0; ks < p.k_stages; ++ks) {
    const int kb0 = ks * ROWB;
    __syncthreads();   // every wave is done with the previous stage
    // 128 rows x 8 chunks of 16 bytes per operand: four chunks per thread
    for (int c = tid; c < BM * (ROWB / 16); c += 256) {
      const int r = c / (ROWB / 16), col = (c % (ROWB / 16)) * 16;
      i32x4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
      if (m0 + r < p.M && kb0 + col < p.row_bytes)
        va = *(const i32x4*)(p.A + (size_t)(m0 + r) * p.row_bytes + kb0 + col);
      if (n0 + r < p.N && kb0 + col < p.row_bytes)
        vb = *(const i32x4*)(p.B + (size_t)(n0 + r) * p.row_bytes + kb0 + col);
      *(i32x4*)(sa + r * ROWB + col) = va;
      *(i32x4*)(sb + r * ROWB + col) = vb;
    }
    __syncthreads();
    for (int kk = 0; kk < ROWB / kStep; ++kk) {
      i32x4 fa[TM], fb[TN];
      for (int i = 0; i < TM; ++i) {
        const uint8_t* ra = sa + (wm * 64 + i * 32 + fr) * ROWB + kk * kStep;
        if constexpr (I4) {
          uint32_t lo0, hi0, lo1, hi1;
          const i32x2_t x = *(const i32x2_t*)(ra + 8 * fh);
          expand_int4((uint32_t)x.x, lo0, hi0);
          expand_int4((uint32_t)x.y, lo1, hi1);
          fa[i] = i32x4{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
        } else {
          fa[i] = *(const i32x4*)(ra + 16 * fh);
        }
      }
      for (int j = 0; j < TN; ++j) {
        const uint8_t* rb = sb + (wn * 64 + j * 32 + fr) * ROWB + kk * kStep;
        if constexpr (I4) {
          uint32_t lo0, hi0, lo1, hi1;
          const i32x2_t x = *(const i32x2_t*)(rb + 8 * fh);
          expand_int4((uint32_t)x.x, lo0, hi0);
          expand_int4((uint32_t)x.y, lo1, hi1);
          fb[j] = i32x4{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
        } else {
          fb[j] = *(const i32x4*)(rb + 16 * fh);
        }
      }
      for (int i = 0; i < TM; ++i)
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma<KIND>(fa[i], fb[j], acc[i][j]);
    }
  }

  // element e of lane l in a 32 x 32 block: row 8 (e / 4) + 4 (l / 32) + e % 4,
  // column l % 32
  for (int i = 0; i < TM; ++i)
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * 64 + j * 32 + fr;
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
        if (row >= p.M || col >= p.N) continue;
        const size_t idx = (size_t)row * p.N + col;
        const auto v = acc[i][j][e];
        if constexpr (KIND == KIND_F16) {
          ((float*)p.C)[idx] = v;
        } else if constexpr (I4) {
          ((int32_t*)p.C)[idx] = v >> 8;   // undo the 16 x 16 scaling
        } else if constexpr (KIND == KIND_I8_DEQUANT) {
          float t = (float)v;
          t = t * p.row_scale[row];
          t = t * p.col_scale[col];
          ((float*)p.C)[idx] = t;
        } else {
          ((int32_t*)p.C)[idx] = v;
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Eight-wave ping-pong kernel.
//
// A 256 x 256 tile is split into eight 128 x 64 wave tiles; waves w and w+4
// share SIMD w % 4.  The two groups of four waves alternate between a memory
// phase (read this stage's operand fragments from LDS into registers, issue
// the direct-to-LDS loads of a later stage) and a compute phase (only MFMAs,
// on operands already in registers), separated by workgroup barriers and
// offset by one barrier, so that on every SIMD one wave keeps the matrix
// core busy while the other one waits on memory.  A single wave that mixes
// both kinds of instructions stalls its own MFMA issue whenever a memory
// instruction or a wait on one blocks.
//
// Barrier schedule (group A = waves 0-3, group B = waves 4-7; b_n = n-th
// barrier after the prologue):
//   A: MEM(0) b1 COMP(0) b2 MEM(1) b3 COMP(1) b4 ...   MEM(s) in (b_2s, b_2s+1)
//   B: b1 MEM(0) b2 COMP(0) b3 MEM(1) b4 ...           MEM(s) in (b_2s+1, b_2s+2)
// In MEM(s) a wave reads stage s, issues its loads for stage s+3 into buffer
// (s+3) % 4 = (s-1) % 4, and waits for its own loads of stage s+1.  Hence
// every load of stage s has landed before b_2s (A's wait in MEM(s-1) precedes
// b_2s-1, B's precedes b_2s), and every read of stage s-1 has finished
// before b_2s, after which both groups first overwrite buffer (s-1) % 4.
template <int KIND, int ROWB>
__global__ __launch_bounds__(512) void gemm_pingpong(GemmArgs p) {
  using Acc = typename KindTraits<KIND>::Acc;
  using Layout = RowLayout<ROWB>;
  constexpr bool I4 = KIND == KIND_I4;
  constexpr int BM = 256, BN = 256, STAGES = 4;
  constexpr int kStepBytes = I4 ? 16 : 32;
  constexpr int KSTEPS = ROWB / kStepBytes;
  constexpr int WTM = 128, WTN = 64;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int kRows = BM + BN;
  constexpr int kStage = kRows * ROWB;
  constexpr int kRowsPerLoad = 1024 / ROWB;
  constexpr int kLoads = kRows / kRowsPerLoad;      // 1 KiB loads per stage
  constexpr int kSlots = kLoads / 8;                // per wave per stage
  constexpr int kLoadsA = BM / kRowsPerLoad;
  static_assert(kLoads % 8 == 0 && kLoadsA % 8 == 0, "loads per wave");
  static_assert(2 * kSlots <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;          // 0: A, 1: B
  const int wm = group, wn = wave & 3;  // group A owns rows 0..127 of the tile

  int tm, tn;
  tile_coords(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = min(BM, p.M - m0);
  const int rows_b = min(BN, p.N - n0);
  const i32x4 rsrc_a = make_rsrc(p.A + (size_t)m0 * p.row_bytes, rows_a * p.row_bytes);
  const i32x4 rsrc_b = make_rsrc(p.B + (size_t)n0 * p.row_bytes, rows_b * p.row_bytes);
  const uint32_t smem_lds = lds_address(smem);

  // slot t of this wave: the (8t + wave)-th 1 KiB piece of the stage
  uint32_t slot_off[kSlots];
  uint32_t slot_col[kSlots];
#pragma unroll
  for (int t = 0; t < kSlots; ++t) {
    const int g = 8 * t + wave;
    const int lrow = kRowsPerLoad * g + lane / Layout::kChunks;
    const int c = Layout::pos(lrow, lane % Layout::kChunks);
    const int grow = g < kLoadsA ? lrow : lrow - BM;
    slot_off[t] = grow * p.row_bytes + c * 16;
    slot_col[t] = c * 16;
  }
  auto issue_load = [&](int t, int s) {
    const uint32_t kbyte = (uint32_t)s * ROWB;
    const int g = 8 * t + wave;
    const bool in_row = kbyte + slot_col[t] < (uint32_t)p.row_bytes;
    const uint32_t off = in_row ? slot_off[t] + kbyte : kOutOfRange;
    lds_dma_16(g < kLoadsA ? rsrc_a : rsrc_b, smem_lds + (s % STAGES) * kStage + g * 1024, off);
  };

  const int fr = lane & 31, fh = lane >> 5;
  const int a_row_base = (wm * WTM) * ROWB;
  const int b_row_base = (BM + wn * WTN) * ROWB;
  auto frag_off = [&](int kk) -> int {
    if constexpr (I4) return Layout::off(fr, kk) + fh * 8;
    else return Layout::off(fr, 2 * kk + fh);
  };

  using Raw = typename std::conditional<I4, i32x2_t, i32x4>::type;
  Raw fa[KSTEPS][TM], fb[KSTEPS][TN];

  auto read_stage = [&](int s) {
    const uint8_t* base = smem + (s % STAGES) * kStage;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int off = frag_off(kk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[kk][i] = *(const Raw*)(base + a_row_base + i * 32 * ROWB + off);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[kk][j] = *(const Raw*)(base + b_row_base + j * 32 * ROWB + off);
    }
  };

  auto operand = [&](const Raw& r) -> i32x4 {
    if constexpr (I4) {
      uint32_t lo0, hi0, lo1, hi1;
      expand_int4((uint32_t)r.x, lo0, hi0);
      expand_int4((uint32_t)r.y, lo1, hi1);
      return i32x4{(int)lo0, (int)hi0, (int)lo1, (int)hi1};
    } else {
      return r;
    }
  };

  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  auto compute_stage = [&]() {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      i32x4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = operand(fa[kk][i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = operand(fb[kk][j]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma<KIND>(a[i], b[j], acc[i][j]);
    }
  };

  const int nks = p.k_stages;   // 0 when K = 0: C is written as zeros
  if (nks > 0) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
#pragma unroll
      for (int t = 0; t < kSlots; ++t) issue_load(t, s);
    wait_vmcnt<2 * kSlots>();            // own loads of stage 0
    block_barrier();                     // everyone's
    if (group == 1) block_barrier();     // B runs one barrier behind
    for (int s = 0; s < nks; ++s) {
      // memory phase
      read_stage(s);
#pragma unroll
      for (int t = 0; t < kSlots; ++t) issue_load(t, s + STAGES - 1);
      wait_vmcnt<2 * kSlots>();          // own loads of stage s+1
      wait_lgkmcnt0();                   // own fragment reads of stage s
      block_barrier();
      // compute phase
      __builtin_amdgcn_s_setprio(1);
      compute_stage();
      __builtin_amdgcn_s_setprio(0);
      block_barrier();
    }
    if (group == 0) block_barrier();     // same barrier count for both groups
  }
  wait_vmcnt<0>();                       // loads past the last stage

  // Epilogue: element e of lane l in a 32x32 block is row 8*(e/4) + 4*(l/32)
  // + e%4, column l%32.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + j * 32 + fr;
      const bool col_ok = col < p.N;
      float cs = 0.f;
      if constexpr (KIND == KIND_I8_DEQUANT) cs = col_ok ? p.col_scale[col] : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
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

// ---------------------------------------------------------------------------
// Skinny-M kernel: weight streaming with in-workgroup split-K.
//
// For a few rows of A against many rows of B (the quantised LLM projection
// at 16 tokens) the time goes into streaming B from HBM once; the MFMA work
// is small.  A workgroup owns 32*MB rows x 32 columns of C and its WAVES
// waves split K: wave w sums the 128-byte K-blocks [w*n/WAVES, (w+1)*n/WAVES).
// Operands go straight from global memory into MFMA-shaped registers
// (16-byte buffer loads; out-of-range rows, the K tail and blocks past the
// wave's share read as zero without touching memory).  A wave issues the
// loads of CHUNK blocks at once and then contracts them, so that a whole
// share costs one memory round trip rather than one per block.  Lane l holds
// row l % 32 and reads bytes 64*(l/32) .. +63 of each 128-byte block of that
// row, four 16-byte pieces that serve four MFMA K-steps (eight 8-byte pieces
// for packed int4); A and B use the same byte-to-step assignment, so the sum
// over k is unchanged, and the two half-waves cover each 128-byte row
// segment.  The partial sums are combined through LDS in a fixed wave order
// and the epilogue is applied once per output element.
// One 128-byte K-block of the skinny kernels: a[mb][q] and b[q] are the
// 16-byte fragments of step q (lane l: row l % 32 of its 32-row block, bytes
// 64 (l / 32) + 16 q of the block; A and B use the same assignment, so the
// sum over k is unchanged).  Packed int4 gives two int8 steps per fragment.
template <int KIND, int MB>
__device__ __forceinline__ void skinny_block(typename KindTraits<KIND>::Acc (&acc)[MB],
                                             const i32x4 (&a)[MB][4], const i32x4 (&b)[4]) {
  if constexpr (KIND == KIND_I4) {
    // 64 packed bytes = 8 K-steps of 8 bytes (16 nibbles) each
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t blo, bhi, blo1, bhi1;
        expand_int4((uint32_t)b[q][2 * half], blo, bhi);
        expand_int4((uint32_t)b[q][2 * half + 1], blo1, bhi1);
        const i32x4 bv = {(int)blo, (int)bhi, (int)blo1, (int)bhi1};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          uint32_t alo, ahi, alo1, ahi1;
          expand_int4((uint32_t)a[mb][q][2 * half], alo, ahi);
          expand_int4((uint32_t)a[mb][q][2 * half + 1], alo1, ahi1);
          const i32x4 av = {(int)alo, (int)ahi, (int)alo1, (int)ahi1};
          acc[mb] = mfma<KIND>(av, bv, acc[mb]);
        }
      }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma<KIND>(a[mb][q], b[q], acc[mb]);
  }
}

// Split-K epilogue of the skinny kernels: every wave has written its partial
// 32*MB x 32 tile to red (rows of kPitch words, wave w's tile starting at
// word w * kWaveWords); the
// partials are summed in wave order (a fixed order, so the result does not
// depend on timing) and the epilogue of the kind is applied once per element.
template <int KIND, int MT, int NT, int WAVES, int kPitch, int kWaveWords>
__device__ __forceinline__ void skinny_reduce_store_strided(const GemmArgs& p, const uint32_t* red,
                                                            int m0, int n0,
                                                            const float* rs_local = nullptr,
                                                            int ncols = NT) {
  for (int idx = threadIdx.x; idx < MT * NT; idx += WAVES * 64) {
    const int rr = idx / NT, cc = idx % NT;
    const int row = m0 + rr, col = n0 + cc;
    if (row >= p.M || col >= p.N || cc >= ncols) continue;
    if constexpr (KIND == KIND_F16) {
      float sum = 0.f;
      for (int w = 0; w < WAVES; ++w) sum += __builtin_bit_cast(float, red[w * kWaveWords + rr * kPitch + cc]);
      ((float*)p.C)[(size_t)row * p.N + col] = sum;
    } else {
      int32_t sum = 0;
      for (int w = 0; w < WAVES; ++w) sum += (int32_t)red[w * kWaveWords + rr * kPitch + cc];
      if constexpr (KIND == KIND_I4) {
        ((int32_t*)p.C)[(size_t)row * p.N + col] = sum >> 8;   // undo the 16 x 16 scaling
      } else if constexpr (KIND == KIND_I8_DEQUANT) {
        float t = (float)sum;
        t = t * (rs_local ? rs_local[rr] : p.row_scale[row]);   // the tile's scales, when local
        t = t * p.col_scale[col];
        ((float*)p.C)[(size_t)row * p.N + col] = t;
      } else {
        ((int32_t*)p.C)[(size_t)row * p.N + col] = sum;
      }
    }
  }
}

// Partial sums of one wave -> its slice of red (element e of lane l: row
// 8*(e/4) + 4*(l/32) + e%4, column l%32 of a 32x32 block).
template <int KIND, int MB, int kPitch>
__device__ __forceinline__ void skinny_store_partials(const typename KindTraits<KIND>::Acc (&acc)[MB],
                                                      uint32_t* mine, int lane) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = mb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      // copy the element out first: bit-casting a vector-element lvalue
      // directly reads the vector's first element
      const auto v = acc[mb][e];
      mine[rr * kPitch + r] = __builtin_bit_cast(uint32_t, v);
    }
}

template <int KIND, int MB, int WAVES, int CHUNK>
__global__ __launch_bounds__(WAVES * 64) void gemm_skinny(GemmArgs p) {
  using Acc = typename KindTraits<KIND>::Acc;
  constexpr int kBlock = 128;
  constexpr int MT = 32 * MB, NT = 32;
  constexpr int kPitch = NT + 1;   // 32-bit words per reduction row

  __shared__ __attribute__((aligned(16))) uint32_t red[WAVES * MT * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
  const int m0 = tm * MT, n0 = tn * NT;
  const int rows_a = min(MT, p.M - m0);
  const int rows_b = min(NT, p.N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + (size_t)m0 * p.row_bytes), 0, rows_a * p.row_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + (size_t)n0 * p.row_bytes), 0, rows_b * p.row_bytes, kBufferWord3);

  const int r = lane & 31, h = lane >> 5;
  const int nblk = p.k_stages;
  const int b0 = (int)(((long long)nblk * wave) / WAVES);
  const int b1 = (int)(((long long)nblk * (wave + 1)) / WAVES);

  // Row offsets are fixed per lane; the K position only adds to them, and
  // the range check is a select, so no branches surround the loads.
  uint32_t a_row[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) a_row[mb] = (uint32_t)(mb * 32 + r) * (uint32_t)p.row_bytes;
  const uint32_t b_row = (uint32_t)r * (uint32_t)p.row_bytes;
  const uint32_t row_bytes = (uint32_t)p.row_bytes;

  i32x4 fa[CHUNK][MB][4], fb[CHUNK][4];
  auto load_block = [&](int blk, i32x4 (&a)[MB][4], i32x4 (&b)[4]) {
    const uint32_t col0 = (uint32_t)blk * kBlock + (uint32_t)h * 64;
    const bool in_range = blk < b1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t col = col0 + q * 16;
      const bool ok = in_range && col < row_bytes;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb][q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, ok ? a_row[mb] + col : kOutOfRange, 0, 0);
      b[q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, ok ? b_row + col : kOutOfRange, 0, 0);
    }
  };

  Acc acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0;

  for (int c = b0; c < b1; c += CHUNK) {
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) load_block(c + j, fa[j], fb[j]);
    // keep every load of the chunk ahead of the MFMAs (the scheduler would
    // otherwise trade memory parallelism for registers)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < CHUNK; ++j) skinny_block<KIND, MB>(acc, fa[j], fb[j]);
  }

  skinny_store_partials<KIND, MB, kPitch>(acc, red + wave * MT * kPitch, lane);
  __syncthreads();
  skinny_reduce_store_strided<KIND, MT, NT, WAVES, kPitch, MT * kPitch>(p, red, m0, n0);
}

// Skinny-M kernel with B staged through LDS (M <= 32).  Loading B fragments
// straight into MFMA registers makes every 16-byte-per-lane load touch 32
// rows; together with the A loads that request count, not HBM, limits the
// weight stream.  Here each wave copies R 128-byte K-blocks of the 32 B rows
// into its own LDS region with direct-to-LDS loads in which lanes 8j .. 8j+7
// cover one row's whole 128-byte line, then reads the fragments back with
// ds_read_b128 (the XOR swizzle of the main kernels keeps those reads free of
// bank conflicts).  A, a few rows shared by every workgroup and mostly L2
// hits, is still loaded straight into fragments.  Each wave only reads what
// it loaded itself, so a round needs no barrier: vmcnt(0) covers the copies,
// and lgkmcnt(0) before the next round's copies makes sure the previous
// round's fragment reads have completed.  The wave's LDS region then holds
// its partial sums for the split-K epilogue.
template <int KIND, int WAVES, int R>
__global__ __launch_bounds__(WAVES * 64) void gemm_skinny_lds(GemmArgs p) {
  using Acc = typename KindTraits<KIND>::Acc;
  constexpr int kBlock = 128;
  constexpr int MT = 32, NT = 32;
  constexpr int kPitch = NT + 1;
  constexpr int kBlockLds = NT * kBlock;      // one K-block of the NT B rows (4 KiB per 32)
  constexpr int kWaveLds = R * kBlockLds;
  static_assert(kWaveLds >= MT * kPitch * 4, "the partial sums reuse the wave's region");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[WAVES * kWaveLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
  const int m0 = tm * MT, n0 = tn * NT;
  const int rows_a = min(MT, p.M - m0);
  const int rows_b = min(NT, p.N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + (size_t)m0 * p.row_bytes), 0, rows_a * p.row_bytes, kBufferWord3);
  const i32x4 rsrc_b = make_rsrc(p.B + (size_t)n0 * p.row_bytes, rows_b * p.row_bytes);
  uint8_t* const my_smem = smem + wave * kWaveLds;
  const uint32_t my_lds = lds_address(my_smem);

  const int r = lane & 31, h = lane >> 5;
  const uint32_t row_bytes = (uint32_t)p.row_bytes;
  const int nblk = p.k_stages;
  const int b0 = (int)(((long long)nblk * wave) / WAVES);
  const int b1 = (int)(((long long)nblk * (wave + 1)) / WAVES);

  // Copy slot t of a K-block fills LDS rows 8t .. 8t+7: lane l writes row
  // 8t + l/8 at chunk position l%8, so it fetches the global chunk whose
  // swizzled position that is (the XOR swizzle is an involution).
  uint32_t dma_off[4], dma_col[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 8 * t + (lane >> 3);
    const int c = swizzle_chunk(row, lane & 7);
    dma_off[t] = (uint32_t)row * row_bytes + c * 16;
    dma_col[t] = c * 16;
  }
  const uint32_t a_row = (uint32_t)r * row_bytes;
  // fragment q of a block: row r, global chunk 4h + q, at its swizzled place
  int frag_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) frag_off[q] = r * kBlock + (swizzle_chunk(r, 4 * h + q) << 4);

  // one accumulator per K-block of a round: independent MFMA chains, summed
  // (in a fixed order) before the epilogue
  Acc acc[R][1];
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][0][e] = 0;

  i32x4 fa[R][1][4], fb[R][4];
  for (int c = b0; c < b1; c += R) {
    wait_lgkmcnt0();   // the previous round's fragment reads are done with the region
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int blk = c + j;
      const uint32_t kbyte = (uint32_t)blk * kBlock;
      const bool in_range = blk < b1;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool ok = in_range && kbyte + dma_col[t] < row_bytes;
        lds_dma_16(rsrc_b, my_lds + j * kBlockLds + t * 1024, ok ? dma_off[t] + kbyte : kOutOfRange);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t col = kbyte + (uint32_t)h * 64 + q * 16;
        const bool ok = in_range && col < row_bytes;
        fa[j][0][q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, ok ? a_row + col : kOutOfRange, 0, 0);
      }
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        fb[j][q] = *(const i32x4*)(my_smem + j * kBlockLds + frag_off[q]);
#pragma unroll
    for (int j = 0; j < R; ++j) skinny_block<KIND, 1>(acc[j], fa[j], fb[j]);
  }
#pragma unroll
  for (int j = 1; j < R; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[0][0][e] += acc[j][0][e];

  wait_lgkmcnt0();
  uint32_t* const red = (uint32_t*)smem;
  skinny_store_partials<KIND, 1, kPitch>(acc[0], (uint32_t*)my_smem, lane);
  __syncthreads();
  // wave w's partials start at w * kWaveLds bytes, kWaveLds / 4 words apart
  skinny_reduce_store_strided<KIND, MT, NT, WAVES, kPitch, kWaveLds / 4>(p, red, m0, n0);
}


// ---------------------------------------------------------------------------
// Per-row int8 quantisation of fp16 activations (the step in front of a W8A8
// projection): scale s = absmax / 127 and q = the nearest-even integer to the
// binary32 quotient x / s, clamped to [-127, 127]; an all-zero row gets
// s = 0 and q = 0.  The max is exact, so the order of the absmax reduction
// does not matter.  HBM-bound: 2K bytes read and K + 4 bytes written per row.
//
// The quotient.  s is always RN(a / 127) for a finite fp16 a, so only about
// 31.7 thousand scales occur.  For every one of them and every finite fp16 x
// the sequence  r = RN(1 / s) (once per row), q0 = RN(x r),
// e = fma(-q0, s, x), q = RN(e r + q0)  gives exactly RN(x / s) (checked
// exhaustively on the CPU, over all 2.0e9 pairs); this is the residual
// correction step of Markstein's division, and it costs three instructions
// per element where a full IEEE division costs about ten.

// Eight fp16 values to eight int8 codes, packed little-endian.  s must be
// nonzero and r = RN(1 / s).
__device__ __forceinline__ uint64_t quantize8(f16x8 h, float s, float r) {
  uint64_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = (float)h[e];
    const float q0 = __fmul_rn(x, r);
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
    const float c = fminf(fmaxf(rintf(q), -127.f), 127.f);
    packed |= (uint64_t)(uint8_t)(int8_t)(int)c << (8 * e);
  }
  return packed;
}

__device__ __forceinline__ float absmax8(f16x8 h, float amax) {
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)h[e]));
  return amax;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Skinny-M kernel, B through LDS as in gemm_skinny_lds, with the rounds of
// each wave double-buffered: the copies and A loads of round i+1 are in
// flight while round i is read back and contracted, so the weight stream
// does not stop at every round.  Two LDS regions of R K-blocks per wave for
// B (direct-to-LDS copies, counted only by the explicit waits); A's
// fragments come through the compiler-tracked register load, two rounds
// ahead in three register sets (one round ahead in two for the eight-wave
// int4 kernel and three-block rounds), in an issue order under which the
// compiler's own waits for them never hold back the next round's copies.
//
// QA: A holds fp16 activations (M x K binary16) that the kernel quantises
// per row itself, the W8A8 step in one launch (KIND_I8_DEQUANT only).  Each
// workgroup first scans the whole of its (at most 32) rows for their absmax
// and derives the row scale s = absmax / 127 and r = 1 / s exactly as the
// separate quantiser does; in the loop every A fragment is loaded as 16
// halves (two 16-byte loads) and rounded to int8 with the same operations,
// and the epilogue multiplies by the tile's scales from LDS.  The result
// equals the separate quantiser followed by the dequantising GEMM bit for
// bit.  The scan is repeated by every workgroup of a row band (the cost the
// Day-12 page ascribes to a quantisation prologue inside the GEMM).
//
// BCPOL: cache policy of the B copies (see lds_dma_16).  The four-wave
// kernel the automatic choice takes at many columns streams B
// non-temporally: the weights of a skinny product are read once per call,
// and from HBM (graph-timed, one MI355X, weights cold: LLM M = 16 12.88
// against 14.03 us, fp16 16 x 14336 x 4096 21.75 against 23.93, int8
// 32 x 8192 x 8192 16.31 against 17.35); re-read from the Infinity Cache
// call after call they gain or lose a few percent (-9% to +6%).  The fused
// W8A8 kernel streams them non-temporally too (31.3 against 34.8 us cold,
// 29.9 against 32.0 warm).  The eight-wave kernel keeps the default: warm,
// it lost 11-25% with them.
//
// NB, p.tile_w: a workgroup holds NB 32-row blocks of B and owns p.tile_w
// (at most 32 NB) columns of C from column p.tile_w * (its tile column) on;
// B rows past its columns read as zero without touching memory and their
// columns are not stored.  Every workgroup then streams the same number of
// B rows, so a column width that divides N into as many workgroups as
// there are CUs (N = 14336 on 256 CUs: 56 columns, NB = 2) loads every CU
// equally, where 32-column tiles (448) give some CUs two and others one.
template <int KIND, int WAVES, int R, bool QA = false, int NB = 1, int BCPOL = 0>
__global__ __launch_bounds__(WAVES * 64) void gemm_skinny_pipe(GemmArgs p) {
  using Acc = typename KindTraits<KIND>::Acc;
  static_assert(!QA || KIND == KIND_I8_DEQUANT, "on-the-fly quantisation feeds the dequantising product");
  static_assert(NB == 1 || NB == 2, "B blocks per workgroup");
  constexpr int kBlock = 128;
  constexpr int MT = 32, NT = 32 * NB;
  constexpr int kPitch = NT + 1;
  constexpr int kBlockLds = NT * kBlock;      // one K-block of the NT B rows (4 KiB per 32)
  constexpr int kRoundLds = R * kBlockLds;
  constexpr int kWaveLds = 2 * kRoundLds;
  constexpr int kAParts = QA ? 2 : 1;         // 16-byte loads per A fragment
  constexpr int kLoadsB = 4 * NB * R;          // B copies per round (4 per 32 rows and block)
  constexpr int kLoadsA = 4 * kAParts * R;     // A fragment loads per round
  static_assert(kWaveLds >= MT * kPitch * 4, "the partial sums reuse the wave's region");
  // at most three rounds of A and two of B are outstanding at once; the
  // vector-memory counter holds at most 63, and a wait on a counter that
  // has overflowed passes too early
  static_assert(3 * kLoadsA + 2 * kLoadsB <= 63, "the loads in flight must fit the vmcnt counter");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[WAVES * kWaveLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
  const int tile_w = p.tile_w > 0 ? p.tile_w : NT;
  const int m0 = tm * MT, n0 = tn * tile_w;
  const int rows_a = min(MT, p.M - m0);
  const int rows_b = min(tile_w, p.N - n0);
  // bytes per row of A: K (int8) or 2K (binary16)
  const uint32_t a_stride = (uint32_t)p.row_bytes * kAParts;
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + (size_t)m0 * a_stride), 0, rows_a * a_stride, kBufferWord3);
  const i32x4 rsrc_b = make_rsrc(p.B + (size_t)n0 * p.row_bytes, rows_b * p.row_bytes);
  uint8_t* const my_smem = smem + wave * kWaveLds;
  const uint32_t my_lds = lds_address(my_smem);

  const int r = lane & 31, h = lane >> 5;
  const uint32_t row_bytes = (uint32_t)p.row_bytes;

  // QA: the row scale s and its reciprocal r of this lane's row r
  __shared__ float row_amax[QA ? MT : 1];
  __shared__ float row_s[QA ? MT : 1];
  float qs = 0.f, qr = 0.f;
  if constexpr (QA) {
    for (int rr = wave; rr < MT; rr += WAVES) {
      float amax = 0.f;
      if (rr < rows_a) {
        const uint8_t* xrow = p.A + (size_t)(m0 + rr) * a_stride;
        for (uint32_t c = lane; c < row_bytes / 8; c += 64)
          amax = absmax8(*(const f16x8*)(xrow + 16 * (size_t)c), amax);
      }
      amax = wave_max(amax);
      if (lane == 0) row_amax[rr] = amax;
    }
    __syncthreads();
    qs = __fdiv_rn(row_amax[r], 127.0f);
    qr = __fdiv_rn(1.0f, qs);
    if (wave == 0 && lane < MT) row_s[lane] = qs;   // for the epilogue, after its barrier
  }
  const int nblk = p.k_stages;
  const int b0 = (int)(((long long)nblk * wave) / WAVES);
  const int b1 = (int)(((long long)nblk * (wave + 1)) / WAVES);
  const int rounds = (b1 - b0 + R - 1) / R;

  uint32_t dma_off[4 * NB], dma_col[4 * NB];
#pragma unroll
  for (int t = 0; t < 4 * NB; ++t) {
    const int row = 8 * t + (lane >> 3);
    const int c = swizzle_chunk(row, lane & 7);
    dma_off[t] = (uint32_t)row * row_bytes + c * 16;
    dma_col[t] = c * 16;
  }
  const uint32_t a_row = (uint32_t)r * a_stride;
  int frag_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) frag_off[q] = r * kBlock + (swizzle_chunk(r, 4 * h + q) << 4);

  Acc acc[R][NB][1];
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][nb][0][e] = 0;

  // A's fragments go straight into registers through the compiler-tracked
  // load; B's blocks go into LDS through direct copies, one round ahead, in
  // two regions (round x in region x % 2).  The compiler does not count the
  // copies, so before A(i)'s first use it waits until no more A loads are
  // outstanding than it issued after A(i); the issue order below makes that
  // wait no stricter than the explicit one for B(i) (with no more B copies
  // than A loads per round, one B block), so the next copies stay in flight.
  //
  // kAhead = 2 (three A register sets, round x in set x % 3): the step for
  // round i issues B(i + 1), then A(i + 2), waits until only A(i + 1),
  // B(i + 1) and A(i + 2) may be outstanding (B(i) has landed; the compiler
  // adds A(i + 1), issued right after B(i)), and contracts round i.  No load
  // is issued past the last round, as such a load moves no data but costs
  // the CU's load path as much as one that does: the last rounds are
  // straight-line code with the issue pattern fixed at compile time (a
  // branch around an A load would leave the compiler unsure whether it is
  // in flight, and it would then wait for everything before the next use).
  //
  // kAhead = 1 (two sets: for the eight-wave int4 kernel, whose registers
  // must stay within 128 for two workgroups per CU, and for three blocks
  // per round, where three sets would spill): the step issues
  // A(i + 1), then B(i + 1) while rounds remain (the compiler does not
  // track the copies, so their branch costs nothing), waits for B(i), and
  // contracts round i; the compiler adds A(i + 1).  Its A loads run one
  // round past the end (outside A, no data moves) and are consumed at the
  // end.
  //
  // Either way every A load issued is used later, so the compiler drops
  // none and the explicit counts hold.
  constexpr int kAhead = ((KIND == KIND_I4 && WAVES == 8) || R >= 3) ? 1 : 2;
  i32x4 fa[kAhead + 1][R][1][4 * kAParts];

  auto issue_a = [&](int i, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int blk = b0 + R * i + j;
      const uint32_t kbyte = (uint32_t)blk * kBlock;
      const bool in_range = blk < b1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t col = kbyte + (uint32_t)h * 64 + q * 16;
        const bool ok = in_range && col < row_bytes;
#pragma unroll
        for (int part = 0; part < kAParts; ++part)
          fa[buf][j][0][kAParts * q + part] = __builtin_amdgcn_raw_buffer_load_b128(
              rsrc_a, ok ? a_row + kAParts * col + 16 * part : kOutOfRange, 0, 0);
      }
    }
  };
  auto issue_b = [&](int i) __attribute__((always_inline)) {
    const uint32_t region = my_lds + (uint32_t)(i & 1) * kRoundLds;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int blk = b0 + R * i + j;
      const uint32_t kbyte = (uint32_t)blk * kBlock;
      const bool in_range = blk < b1;
#pragma unroll
      for (int t = 0; t < 4 * NB; ++t) {
        const bool ok = in_range && kbyte + dma_col[t] < row_bytes;
        lds_dma_16<BCPOL>(rsrc_b, region + j * kBlockLds + t * 1024, ok ? dma_off[t] + kbyte : kOutOfRange);
      }
    }
  };
  // contract round i from A set `set` and B region i % 2
  auto contract = [&](int i, auto set_c) __attribute__((always_inline)) {
    constexpr int set = decltype(set_c)::value;
    const uint8_t* const region = my_smem + (i & 1) * kRoundLds;
    i32x4 fb[R][NB][4];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        // block nb's rows start 32 rows on, which leaves the swizzle unchanged
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          fb[j][nb][q] = *(const i32x4*)(region + j * kBlockLds + nb * 32 * kBlock + frag_off[q]);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if constexpr (QA) {
        // 16 halves per fragment -> 16 int8 codes (an all-zero row: s = 0, codes 0)
        i32x4 qa[1][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint64_t lo = qs != 0.f ? quantize8(__builtin_bit_cast(f16x8, fa[set][j][0][2 * q]), qs, qr) : 0;
          const uint64_t hi = qs != 0.f ? quantize8(__builtin_bit_cast(f16x8, fa[set][j][0][2 * q + 1]), qs, qr) : 0;
          qa[0][q] = i32x4{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi, (int)(uint32_t)(hi >> 32)};
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) skinny_block<KIND, 1>(acc[j][nb], qa, fb[j][nb]);
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) skinny_block<KIND, 1>(acc[j][nb], fa[set][j], fb[j][nb]);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  if constexpr (kAhead == 2) {
    // kFull: issue B(i + 1) and A(i + 2); kSecondLast: only B(i + 1);
    // kLast: nothing
    constexpr int kFull = 0, kSecondLast = 1, kLast = 2;
    auto step = [&](int i, auto set_c, auto mode_c) __attribute__((always_inline)) {
      constexpr int set = decltype(set_c)::value;
      constexpr int mode = decltype(mode_c)::value;
      __builtin_amdgcn_sched_barrier(0);   // steps do not interleave (fewer live registers)
      if constexpr (mode == kFull) {
        wait_lgkmcnt0();   // the other region's fragment reads (round i - 1) are complete
        issue_b(i + 1);
        issue_a(i + 2, std::integral_constant<int, (set + 2) % 3>());
        wait_vmcnt<2 * kLoadsA + kLoadsB>();   // all but A(i + 1), B(i + 1), A(i + 2)
      } else if constexpr (mode == kSecondLast) {
        wait_lgkmcnt0();
        issue_b(i + 1);
        wait_vmcnt<kLoadsA + kLoadsB>();       // all but A(i + 1), B(i + 1)
      } else {
        wait_vmcnt<0>();
      }
      contract(i, set_c);
    };
    using Full = std::integral_constant<int, kFull>;
    using SecondLast = std::integral_constant<int, kSecondLast>;
    using Last = std::integral_constant<int, kLast>;
    if (rounds > 0) {
      issue_a(0, I0());
      issue_b(0);
      issue_a(1, I1());   // (a single round: outside A, no data moves)
      // whole groups of three full steps while two more rounds follow them;
      // the loop's back edge comes only from a whole group, so the
      // compiler's view of the loads in flight is the same at every loop head
      int i = 0;
      for (; i + 5 <= rounds; i += 3) {
        step(i, I0(), Full());
        step(i + 1, I1(), Full());
        step(i + 2, I2(), Full());
      }
      // the last one to four rounds, each case straight-line
      switch (rounds - i) {
        case 4:
          step(i, I0(), Full());
          step(i + 1, I1(), Full());
          step(i + 2, I2(), SecondLast());
          step(i + 3, I0(), Last());
          break;
        case 3:
          step(i, I0(), Full());
          step(i + 1, I1(), SecondLast());
          step(i + 2, I2(), Last());
          break;
        case 2:
          step(i, I0(), SecondLast());
          step(i + 1, I1(), Last());
          break;
        default:
          step(i, I0(), Last());
          break;
      }
    }
  } else {
    auto step = [&](int i, auto set_c) __attribute__((always_inline)) {
      constexpr int set = decltype(set_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkmcnt0();   // the other region's fragment reads (round i - 1) are complete
      issue_a(i + 1, std::integral_constant<int, 1 - set>());
      if (i + 1 < rounds) {
        issue_b(i + 1);
        wait_vmcnt<kLoadsA + kLoadsB>();   // all but A(i + 1), B(i + 1)
      } else {
        wait_vmcnt<kLoadsA>();
      }
      contract(i, set_c);
    };
    if (rounds > 0) {
      issue_a(0, I0());
      issue_b(0);
      // whole pairs, then the rest; the loop's back edge comes only from a
      // whole pair
      int i = 0;
      for (; i + 2 <= rounds; i += 2) {
        step(i, I0());
        step(i + 1, I1());
      }
      if (i < rounds) step(i, I0());
      wait_vmcnt<0>();
#pragma unroll
      for (int set = 0; set < 2; ++set)
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
          for (int q = 0; q < 4 * kAParts; ++q) asm volatile("" ::"v"(fa[set][j][0][q]));
    }
  }
#pragma unroll
  for (int j = 1; j < R; ++j)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[0][nb][0][e] += acc[j][nb][0][e];

  wait_lgkmcnt0();
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    skinny_store_partials<KIND, 1, kPitch>(acc[0][nb], (uint32_t*)my_smem + 32 * nb, lane);
  __syncthreads();
  skinny_reduce_store_strided<KIND, MT, NT, WAVES, kPitch, kWaveLds / 4>(p, (const uint32_t*)smem, m0, n0,
                                                                          QA ? row_s : nullptr, tile_w);
}

}  // namespace lpgemm
