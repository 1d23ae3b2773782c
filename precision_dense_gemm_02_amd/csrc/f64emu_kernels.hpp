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
//     GEMM with int32 sums (|sum| <= K 2^14);
//   * reconstruction: Garner's mixed-radix digits, the 192-bit value
//     X = sum v_l W_l (W_l the product of the earlier moduli), made balanced
//     (X - P when X >= P/2), rounded once to double (nearest, ties to even)
//     and scaled by 2^-(2t - eA[i] - eB[j]).
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
  int w_mod[kF64MaxModuli][kF64MaxModuli]; // (product of m[0..k-1]) mod m[l], index [l][k]
  int w_inv[kF64MaxModuli];                // inverse of (product of m[0..l-1]) modulo m[l]
  uint64_t w[kF64MaxModuli][3];            // product of m[0..l-1], 192-bit little-endian
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
__global__ __launch_bounds__(256) void f64_residues(const double* __restrict__ X, const int* __restrict__ e,
                                                    int64_t total, int K, int8_t* __restrict__ R,
                                                    F64EmuConsts c) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t row = idx / K;
    const double v = rint(ldexp(X[idx], c.bits - e[row]));
    for (int l = 0; l < c.s; ++l) {
      const double m = (double)c.m[l];
      const double q = rint(v * c.inv_m[l]);
      double r = fma(-q, m, v);
      const double hi = (double)((c.m[l] - 1) / 2), lo = -(double)(c.m[l] / 2);
      if (r > hi) r -= m;
      if (r > hi) r -= m;
      if (r < lo) r += m;
      if (r < lo) r += m;
      R[(size_t)l * total + idx] = (int8_t)(int)r;
    }
  }
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

// C[i][j] from the s int32 products: residues of each modulus, Garner's
// digits, the balanced 192-bit integer, one rounding, the scaling undone.
// CL holds the s products l * cl_stride elements apart.
__global__ __launch_bounds__(256) void f64_crt(const int32_t* __restrict__ CL, int64_t cl_stride,
                                               int64_t MN, int N,
                                               const int* __restrict__ eA, const int* __restrict__ eB,
                                               double* __restrict__ C, F64EmuConsts c) {
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < MN;
       idx += (int64_t)gridDim.x * 256) {
    int v[kF64MaxModuli];
    uint64_t x[3] = {0, 0, 0};
    for (int l = 0; l < c.s; ++l) {
      const int m = c.m[l];
      int r = CL[(size_t)l * cl_stride + idx] % m;
      if (r < 0) r += m;
      // x mod m from the earlier digits, then this digit
      int acc = 0;
      for (int k = 0; k < l; ++k) acc += v[k] * c.w_mod[l][k];
      int d = (r - acc % m) % m;
      if (d < 0) d += m;
      d = (d * c.w_inv[l]) % m;
      v[l] = d;
      u192_add_mul_small(x, c.w[l], (uint32_t)d);
    }
    bool neg = false;
    if (u192_ge(x, c.p_half)) {   // the balanced class: X - P
      u192_rsub(x, c.p);
      neg = true;
    }
    double d = u192_to_double(x);
    if (neg) d = -d;
    const int64_t i = idx / N, j = idx - i * N;
    C[idx] = ldexp(d, -(2 * c.bits - eA[i] - eB[j]));
  }
}

}  // namespace lpgemm
