// MFMA-only ceiling of the GPU at its sustained clock.
//
// Runs back-to-back kernels that issue only 32x32 MFMAs (int8 32x32x32,
// fp16 32x32x16, and the 32x32x64 f8f6f4 MFMA with FP8 E4M3, FP6 E3M2 and
// FP4 E2M1 operands) on pseudo-random register operands, eight independent
// accumulators per wave, two waves per SIMD, for a given number of seconds
// each, and prints the achieved rates.  No memory traffic, so this is the upper
// bound a GEMM kernel can reach at the clock the board sustains under MFMA
// load (which is below the 2.4 GHz the datasheet peaks assume).
//
//   probes/mfma_ceiling [seconds]
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_i8(int iters, int* out, unsigned seed) {
  unsigned x = (threadIdx.x + 1) * 2654435761u ^ seed;
  i32x4 a[4], b[4];
  for (int i = 0; i < 4; ++i) {
    x = x * 1664525u + 1013904223u;
    a[i] = {(int)x, (int)(x * 3u), (int)(x * 7u), (int)(x * 11u)};
    x = x * 1664525u + 1013904223u;
    b[i] = {(int)x, (int)(x * 5u), (int)(x * 9u), (int)(x * 13u)};
  }
  i32x16 c[kChains] = {};
  // the operand rotation is unrolled so every register index is static
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int rot = 0; rot < 4; ++rot)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j & 3], b[(j + rot) & 3], c[j], 0, 0, 0);
  }
  int s = 0;
  for (int j = 0; j < kChains; ++j)
    for (int e = 0; e < 16; ++e) s += c[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_f16(int iters, int* out, unsigned seed) {
  // operands: small integers spread over [-8, 8] scaled to about [-1, 1],
  // different per lane, per element and per register set
  f16x8 a[4], b[4];
  const int t = (int)(threadIdx.x ^ seed);
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 8; ++e) {
      a[i][e] = (_Float16)(float)(((t * 7 + i * 13 + e * 5) % 17) - 8) * (_Float16)0.125f;
      b[i][e] = (_Float16)(float)(((t * 11 + i * 3 + e * 7) % 17) - 8) * (_Float16)0.125f;
    }
  f32x16 c[kChains] = {};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int rot = 0; rot < 4; ++rot)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j & 3], b[(j + rot) & 3], c[j], 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < kChains; ++j)
    for (int e = 0; e < 16; ++e) s += c[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = (int)s;
}

// The 16x16 forms of the same two contractions (int8 16x16x64, fp16
// 16x16x32): a quarter of the 32x32 forms' accumulator registers per MFMA for
// half the MACs, the same operand registers.
__global__ __launch_bounds__(256) void mfma_i8_16(int iters, int* out, unsigned seed) {
  unsigned x = (threadIdx.x + 1) * 2654435761u ^ seed;
  i32x4 a[4], b[4];
  for (int i = 0; i < 4; ++i) {
    x = x * 1664525u + 1013904223u;
    a[i] = {(int)x, (int)(x * 3u), (int)(x * 7u), (int)(x * 11u)};
    x = x * 1664525u + 1013904223u;
    b[i] = {(int)x, (int)(x * 5u), (int)(x * 9u), (int)(x * 13u)};
  }
  i32x4 c[kChains] = {};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int rot = 0; rot < 4; ++rot)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j & 3], b[(j + rot) & 3], c[j], 0, 0, 0);
  }
  int s = 0;
  for (int j = 0; j < kChains; ++j)
    for (int e = 0; e < 4; ++e) s += c[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_f16_16(int iters, int* out, unsigned seed) {
  f16x8 a[4], b[4];
  const int t = (int)(threadIdx.x ^ seed);
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 8; ++e) {
      a[i][e] = (_Float16)(float)(((t * 7 + i * 13 + e * 5) % 17) - 8) * (_Float16)0.125f;
      b[i][e] = (_Float16)(float)(((t * 11 + i * 3 + e * 7) % 17) - 8) * (_Float16)0.125f;
    }
  f32x4 c[kChains] = {};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int rot = 0; rot < 4; ++rot)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j & 3], b[(j + rot) & 3], c[j], 0, 0, 0);
  }
  float s = 0;
  for (int j = 0; j < kChains; ++j)
    for (int e = 0; e < 4; ++e) s += c[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = (int)s;
}

// FMT: 0 FP8 E4M3, 3 FP6 E3M2, 4 FP4 E2M1 (the f8f6f4 format codes); block
// scales 2^0.  Operand bytes are random six-bit values (for FP8 that keeps
// every code finite), so FP6 sees every E3M2 code.
template <int FMT>
__global__ __launch_bounds__(256) void mfma_f8f6f4(int iters, int* out, unsigned seed) {
  unsigned x = (threadIdx.x + 1) * 2654435761u ^ seed;
  i32x8 a[4], b[4];
  for (int i = 0; i < 4; ++i)
    for (int e = 0; e < 8; ++e) {
      x = x * 1664525u + 1013904223u;
      a[i][e] = (int)(x & 0x3f3f3f3fu);
      x = x * 1664525u + 1013904223u;
      b[i][e] = (int)(x & 0x3f3f3f3fu);
    }
  f32x16 c[kChains] = {};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int rot = 0; rot < 4; ++rot)
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j & 3], b[(j + rot) & 3], c[j], FMT, FMT,
                                                               0, 127, 0, 127);
  }
  float s = 0;
  for (int j = 0; j < kChains; ++j)
    for (int e = 0; e < 16; ++e) s += c[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = (int)s;
}

template <typename Kernel>
double sustained(Kernel k, double seconds, double macs_per_wave_iter, int cus, int* out) {
  const int blocks = cus * 2;   // 256 threads each: two waves per SIMD
  const int iters = 20000;   // a multiple of 4
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  long launches = 0;
  const auto t0 = std::chrono::steady_clock::now();
  (void)hipEventRecord(e0);
  while (std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() < seconds) {
    for (int r = 0; r < 10; ++r, ++launches)
      hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, iters, out, (unsigned)launches);
    if (hipDeviceSynchronize() != hipSuccess) return -1;
  }
  (void)hipEventRecord(e1);
  (void)hipEventSynchronize(e1);
  float ms = 0;
  (void)hipEventElapsedTime(&ms, e0, e1);
  const double ops = 2.0 * macs_per_wave_iter * kChains * iters * (double)blocks * 4 * launches;
  return ops / (ms * 1e-3) / 1e12;
}

int main(int argc, char** argv) {
  const double seconds = argc > 1 ? atof(argv[1]) : 3.0;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, 0) != hipSuccess) return 1;
  int* out = nullptr;
  if (hipMalloc(&out, (size_t)prop.multiProcessorCount * 2 * 256 * sizeof(int)) != hipSuccess) return 1;
  const double i8 = sustained(mfma_i8, seconds, 32.0 * 32 * 32, prop.multiProcessorCount, out);
  const double f16 = sustained(mfma_f16, seconds, 32.0 * 32 * 16, prop.multiProcessorCount, out);
  const double e3m2 = sustained(mfma_f8f6f4<3>, seconds, 32.0 * 32 * 64, prop.multiProcessorCount, out);
  const double fp8 = sustained(mfma_f8f6f4<0>, seconds, 32.0 * 32 * 64, prop.multiProcessorCount, out);
  const double fp4 = sustained(mfma_f8f6f4<4>, seconds, 32.0 * 32 * 64, prop.multiProcessorCount, out);
  // the 16x16 forms, each beside its 32x32 form measured again right before
  const double i8b = sustained(mfma_i8, seconds, 32.0 * 32 * 32, prop.multiProcessorCount, out);
  const double i8_16 = sustained(mfma_i8_16, seconds, 16.0 * 16 * 64, prop.multiProcessorCount, out);
  const double f16b = sustained(mfma_f16, seconds, 32.0 * 32 * 16, prop.multiProcessorCount, out);
  const double f16_16 = sustained(mfma_f16_16, seconds, 16.0 * 16 * 32, prop.multiProcessorCount, out);
  printf("{\"device\": \"%s\", \"cus\": %d, \"seconds_each\": %.1f, "
         "\"mfma_i8_tops\": %.1f, \"mfma_f16_tflops\": %.1f, \"mfma_fp6_e3m2_tflops\": %.1f, "
         "\"mfma_fp8_tflops\": %.1f, \"mfma_fp4_tflops\": %.1f, "
         "\"mfma_i8_32x32x32_again_tops\": %.1f, \"mfma_i8_16x16x64_tops\": %.1f, "
         "\"mfma_f16_32x32x16_again_tflops\": %.1f, \"mfma_f16_16x16x32_tflops\": %.1f}\n",
         prop.gcnArchName, prop.multiProcessorCount, seconds, i8, f16, e3m2, fp8, fp4, i8b, i8_16, f16b,
         f16_16);
  (void)hipFree(out);
  return (i8 > 0 && f16 > 0 && e3m2 > 0 && fp8 > 0 && fp4 > 0 && i8b > 0 && i8_16 > 0 && f16b > 0 &&
          f16_16 > 0)
             ? 0
             : 1;
}
