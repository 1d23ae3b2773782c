// Store-pattern probe: how fast can 256x256 int32 output tiles be written?
//
// 1024 workgroups of 4 waves each write one 256x256 tile of an 8192x8192
// int32 matrix (256 MiB), 16 bytes per lane per store, 300 launches per
// variant after 300 untimed ones:
//  PAT 0: wave (wm, wn) writes its 128x128 quadrant; a store covers 2 rows
//         x 512 B (the GEMM epilogue's pattern).
//  PAT 1: wave w writes rows 64w..64w+63, all 256 columns; a store covers
//         1 row x 1 KiB.
// each with ordinary and with non-temporal stores.
//
//   probes/store_pattern
#include <hip/hip_runtime.h>
#include <cstdio>
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int N = 8192;

template <int PAT, bool NT>
__global__ __launch_bounds__(256) void store_tile(int* C, int v) {
  const int id = blockIdx.x;               // 0..1023
  const int tm = id / 32, tn = id % 32;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const i32x4 val = {v + lane, v ^ lane, v - lane, v * 3 + lane};
  if (PAT == 0) {
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll 4
    for (int s = 0; s < 64; ++s) {          // 128 rows, 2 per store
      const int r = tm * 256 + wm * 128 + 2 * s + lane / 32;
      const int c = tn * 256 + wn * 128 + (lane % 32) * 4;
      i32x4* p = (i32x4*)(C + (size_t)r * N + c);
      if (NT) __builtin_nontemporal_store(val, p); else *p = val;
    }
  } else {
#pragma unroll 4
    for (int s = 0; s < 64; ++s) {          // 64 rows, 1 per store
      const int r = tm * 256 + wave * 64 + s;
      const int c = tn * 256 + lane * 4;
      i32x4* p = (i32x4*)(C + (size_t)r * N + c);
      if (NT) __builtin_nontemporal_store(val, p); else *p = val;
    }
  }
}

template <int PAT, bool NT>
float run(int* C) {
  for (int i = 0; i < 300; ++i) hipLaunchKernelGGL((store_tile<PAT, NT>), dim3(1024), dim3(256), 0, 0, C, i);
  (void)hipDeviceSynchronize();
  hipEvent_t e0, e1; (void)hipEventCreate(&e0); (void)hipEventCreate(&e1);
  (void)hipEventRecord(e0);
  for (int i = 0; i < 300; ++i) hipLaunchKernelGGL((store_tile<PAT, NT>), dim3(1024), dim3(256), 0, 0, C, i);
  (void)hipEventRecord(e1); (void)hipEventSynchronize(e1);
  float ms; (void)hipEventElapsedTime(&ms, e0, e1);
  return ms / 300 * 1000;
}

int main() {
  int* C;
  if (hipMalloc(&C, (size_t)N * N * 4) != hipSuccess) return 1;
  for (int rep = 0; rep < 2; ++rep) {
    float a = run<0, false>(C), b = run<0, true>(C), c = run<1, false>(C), d = run<1, true>(C);
    const double mb = (double)N * N * 4;
    printf("quadrant 2x512B: %.1f us (%.0f GB/s)  NT: %.1f us (%.0f GB/s)\n", a, mb / a / 1e3, b, mb / b / 1e3);
    printf("rows 1x1KiB:     %.1f us (%.0f GB/s)  NT: %.1f us (%.0f GB/s)\n", c, mb / c / 1e3, d, mb / d / 1e3);
  }
  (void)hipFree(C);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
