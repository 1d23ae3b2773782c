// fp64 GEMM emulated with exact int8 GEMMs (device code).
//
// The stages follow the FP64-emulation page of the series (day 12): scale /
// exponent scan, residue quantisation, INT8 GEMM, mod reduction, CRT
// reconstruction, undo scaling, write double.  Readings where the page is
// silent:
//   * scaling: each row of A (each column of B, a row of the K-contiguous
//     B) is multiplied by 2^(t - e), e the binary exponent of its largest
//     magnitude (max = f 2^e, 0.5 <= f < 1), and rounded to the nearest
//     integer, ties to even, so |a'| <= 2^t (t = target bits, 1..53);
//   * moduli: the largest pairwise coprime integers up to 256 (256, 255,
//     253, 251, 247, 241, ...), as many as make their product P exceed
//     2 K 2^(2t), so the exact integer product X = A'.B' (|X| <= K 2^(2t))
//     is the unique balanced residue class modulo P;
//   * residues are stored balanced in int8 ([-128, 127] for 256,
//     [-(m-1)/2, (m-1)/2] for odd m), so each modulus is one exact int8
//     GEMM with int32 sums (|sum| <= K 2^14), whose epilogue reduces each
//     sum modulo m and stores the byte (mod reduction);
//   * reconstruction: with M_l = P / m_l and t_l = r_l (M_l^-1 mod m_l)
//     mod m_l, X = sum t_l M_l - q P for q = floor(sum t_l / m_l) (estimated
//     in double, then made exact by one range correction in integers), made
//     balanced (X - P when X >= P/2), rounded once to double (nearest, ties
//     to even) and scaled by 2^-(2t - eA[i] - eB[j]).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lpgemm {

constexpr int kF64MaxModuli = 20;

// Constants of one emulation call, passed by value.
struct F64EmuConsts {
  int s;                                   // number of moduli
  int bits;                                // target bits t
  int m[kF64MaxModuli];                    // moduli
  double inv_m[kF64MaxModuli];             // RN(1 / m)
  float inv_mf[kF64MaxModuli];             // RN(1 / m) in binary32
  int crt_c[kF64MaxModuli];                // (P / m[l])^-1 mod m[l]
  uint64_t big_m[kF64MaxModuli][3];        // P / m[l], 192-bit little-endian
  uint64_t p[3];                           // product of all s moduli
  uint64_t p_half[3];                      // floor(P / 2)
};

// Binary exponent of the largest magnitude of each row (frexp convention);
// 0 for an all-zero row.  One workgroup of 256 per row.
__global__ __launch_bounds__(256) void f64_row_exponent(const double* __restrict__ X, int K,
                                                        int* __restrict__ e) {
  const double* row = X + (size_t)blockIdx.x * K;
  double amax = 0.0;
  for (int k = threadIdx.x; k < K; k += 256) amax = fmax(amax, fabs(row[k]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off));
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    amax = fmax(fmax(part[0], part[1]), fmax(part[2], part[3]));
    int ex = 0;
    if (amax > 0.0) frexp(amax, &ex);
    e[blockIdx.x] = ex;
  }
}

// Scaled integers of each element, reduced modulo every modulus:
// R[l][row][k] = balanced(rint(x 2^(t - e[row])) mod m[l]).  The integer v
// (|v| <= 2^53) is exact in double; q = rint(v * RN(1/m)) is within one of
// rint(v / m) (the relative error of the product is below 2^-51 and
// |v / m| < 2^46), so fma(-q, m, v) is an exact integer within m + m/2 of
// zero, and at most two corrections by m bring it into the balanced range.
// Each thread takes eight consecutive values of a row (K is a multiple of
// 16) and writes one 8-byte word per modulus.  S (the modulus count) is a
// template parameter so every loop unrolls with fixed register and
// kernel-argument offsets.
template <int S>
__global__ __launch_bounds__(256) void f64_residues(const double* __restrict__ X, const int* __restrict__ e,
                                                    int64_t total, int K, int8_t* __restrict__ R,
                                                    F64EmuConsts c) {
  const int64_t groups = total / 8;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += (int64_t)gridDim.x * 256) {
    const int64_t idx = g * 8;
    const int sh = c.bits - e[idx / K];
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = rint(ldexp(X[idx + q], sh));
#pragma unroll
    for (int l = 0; l < S; ++l) {
      const double m = (double)c.m[l];
      const double hi = (double)((c.m[l] - 1) / 2), lo = -(double)(c.m[l] / 2);
      uint64_t packed = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        double r = fma(-rint(v[q] * c.inv_m[l]), m, v[q]);
        if (r > hi) r -= m;
        if (r > hi) r -= m;
        if (r < lo) r += m;
        if (r < lo) r += m;
        packed |= (uint64_t)(uint8_t)(int8_t)(int)r << (8 * q);
      }
      *(uint64_t*)(R + (size_t)l * total + idx) = packed;
    }
  }
}

// x mod m for 0 <= x < 2^24, all in binary32 (every value here is an
// integer below 2^24, so exact): q = floor(x RN(1/m)) is within one of
// floor(x / m), fma(-q, m, x) is then exact, and one correction each way
// finishes.
__device__ __forceinline__ int mod_small(int x, int m, float inv) {
  const float xf = (float)x, mf = (float)m;
  float r = fmaf(-floorf(xf * inv), mf, xf);
  if (r < 0.f) r += mf;
  if (r >= mf) r -= mf;
  return (int)r;
}

// 192-bit unsigned helpers (three little-endian 64-bit limbs).
__device__ __forceinline__ void u192_add_mul_small(uint64_t (&a)[3], const uint64_t (&w)[3], uint32_t v) {
  unsigned __int128 carry = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const unsigned __int128 t = (unsigned __int128)w[i] * v + a[i] + carry;
    a[i] = (uint64_t)t;
    carry = t >> 64;
  }
}
__device__ __forceinline__ bool u192_ge(const uint64_t (&a)[3], const uint64_t (&b)[3]) {
  if (a[2] != b[2]) return a[2] > b[2];
  if (a[1] != b[1]) return a[1] > b[1];
  return a[0] >= b[0];
}
// a = b - a (requires b >= a)
__device__ __forceinline__ void u192_rsub(uint64_t (&a)[3], const uint64_t (&b)[3]) {
  uint64_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint64_t bi = b[i], ai = a[i];
    const uint64_t d = bi - ai - borrow;
    borrow = (bi < ai || (bi - ai) < borrow) ? 1 : 0;
    a[i] = d;
  }
}
// The nearest double to a (ties to even).
__device__ __forceinline__ double u192_to_double(const uint64_t (&a)[3]) {
  int top = -1;
  uint64_t hw = 0;
  if (a[2]) { top = 128 + 63 - __builtin_clzll(a[2]); }
  else if (a[1]) { top = 64 + 63 - __builtin_clzll(a[1]); }
  else if (a[0]) { top = 63 - __builtin_clzll(a[0]); }
  if (top < 0) return 0.0;
  if (top < 53) return (double)a[0];   // exact
  // the 64 bits below and including the top bit, and whether anything
  // below them is set
  const int lo_bit = top - 63;         // may be negative
  bool sticky = false;
  if (lo_bit <= 0) {
    hw = a[0] << (-lo_bit);            // top < 64 here
  } else {
    const int limb = lo_bit >> 6, sh = lo_bit & 63;
    hw = a[limb] >> sh;
    if (sh && limb + 1 < 3) hw |= a[limb + 1] << (64 - sh);
    sticky = (a[limb] & ((sh ? (1ull << sh) : 1ull) - 1)) != 0;
    for (int i = 0; i < limb; ++i) sticky |= a[i] != 0;
  }
  uint64_t mant = hw >> 11;            // 53 bits
  const uint64_t rest = hw & 0x7FF;
  const bool round = (rest >> 10) & 1;
  const bool below = (rest & 0x3FF) != 0 || sticky;
  int exp = top - 52;
  if (round && (below || (mant & 1))) {
    ++mant;
    if (mant == (1ull << 53)) { mant >>= 1; ++exp; }
  }
  return ldexp((double)mant, exp);
}

// The nearest double to a 128-bit unsigned integer (ties to even).
__device__ __forceinline__ double u128_to_double(unsigned __int128 a) {
  const uint64_t hi = (uint64_t)(a >> 64), lo = (uint64_t)a;
  const uint64_t a3[3] = {lo, hi, 0};
  return u192_to_double(a3);
}

// C[i][j] from the S reduced products (bytes r_l in [0, m_l)): the CRT sum,
// the exact range correction, the balanced integer, one rounding, the
// scaling undone.  With up to 16 moduli P < 2^128 (the first sixteen
// multiply to about 2^125.4): the sum is formed modulo 2^128, which is exact
// for the final X since |X| < 2P < 2^127; otherwise in 192 bits.  Small
// reductions use binary32 (mod_small).  CR holds the S byte matrices
// l * cr_stride bytes apart.
template <int S>
__global__ __launch_bounds__(256) void f64_crt(const uint8_t* __restrict__ CR, int64_t cr_stride,
                                               int64_t MN, int N, const int* __restrict__ eA,
                                               const int* __restrict__ eB, double* __restrict__ C,
                                               F64EmuConsts c) {
  constexpr bool WIDE = S > 16;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < MN;
       idx += (int64_t)gridDim.x * 256) {
    int rs[S];
#pragma unroll
    for (int l = 0; l < S; ++l) rs[l] = CR[(size_t)l * cr_stride + idx];
    double f = 0.0;                 // sum t_l / m_l, estimates q
    uint64_t x3[3] = {0, 0, 0};
    unsigned __int128 x2 = 0;
#pragma unroll
    for (int l = 0; l < S; ++l) {
      const int m = c.m[l];
      const float inv = c.inv_mf[l];
      const int t = mod_small((int)__umul24(rs[l], c.crt_c[l]), m, inv);
      f = fma((double)t, c.inv_m[l], f);
      if constexpr (WIDE) u192_add_mul_small(x3, c.big_m[l], (uint32_t)t);
      else x2 += ((unsigned __int128)c.big_m[l][1] << 64 | c.big_m[l][0]) * (uint64_t)t;
    }
    // q is floor(f) or one off (f carries at most a few ulps of error); the
    // sign of X - 0 and of X - P decide the correction exactly
    const uint32_t q = (uint32_t)floor(f);
    double out;
    if constexpr (WIDE) {
      // x3 -= q P; then bring into [0, P)
      uint64_t qp[3] = {0, 0, 0};
      u192_add_mul_small(qp, c.p, q);
      uint64_t d[3];
      if (u192_ge(x3, qp)) {
        d[0] = qp[0]; d[1] = qp[1]; d[2] = qp[2];
        u192_rsub(d, x3);                      // x3 - qP >= 0
        if (u192_ge(d, c.p)) {                 // q was one too small
          const uint64_t pp[3] = {c.p[0], c.p[1], c.p[2]};
          uint64_t e3[3] = {pp[0], pp[1], pp[2]};
          u192_rsub(e3, d);
          d[0] = e3[0]; d[1] = e3[1]; d[2] = e3[2];
        }
      } else {                                 // q was one too large: X = P - (qP - x3)
        d[0] = x3[0]; d[1] = x3[1]; d[2] = x3[2];
        u192_rsub(d, qp);                      // qP - x3 > 0
        u192_rsub(d, c.p);                     // P - (qP - x3)
      }
      bool neg = false;
      if (u192_ge(d, c.p_half)) {              // the balanced class: X - P
        u192_rsub(d, c.p);
        neg = true;
      }
      out = u192_to_double(d);
      if (neg) out = -out;
    } else {
      const unsigned __int128 p = (unsigned __int128)c.p[1] << 64 | c.p[0];
      const unsigned __int128 ph = (unsigned __int128)c.p_half[1] << 64 | c.p_half[0];
      __int128 x = (__int128)(x2 - p * q);     // exact: |x| < 2P < 2^127
      if (x < 0) x += (__int128)p;
      else if (x >= (__int128)p) x -= (__int128)p;
      const unsigned __int128 ux = (unsigned __int128)x;
      out = ux >= ph ? -u128_to_double(p - ux) : u128_to_double(ux);
    }
    const int64_t i = idx / N, j = idx - i * N;
    C[idx] = ldexp(out, -(2 * c.bits - eA[i] - eB[j]));
  }
}

}  // namespace lpgemm
