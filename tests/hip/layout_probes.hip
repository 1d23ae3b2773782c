// Layout probes: single-instruction kernels that pin, on the device, the
// lane layouts the GEMM kernels assume.  Test infrastructure only (built
// into tests/hip/liblayout_probes.so and called by
// tests/test_gpu_layout_probes.py); nothing in the library uses it.
//
// Each probe places operands in registers, or bytes in LDS, by the layout
// the kernels use, runs one instruction, and writes what every lane holds to
// memory by the same layout.  A test then compares that with the product
// (or the bytes) computed on the host from the plain definition; a wrong
// assumption about any lane's row, column or k-range shows up as a mismatch.
//
// The layouts (the MFMA descriptions of the CDNA4 instruction set; the pages
// describe none of this):
//   32 x 32 MFMA operands: lane l holds row (or column) l % 32 of its
//     operand, k-range 16 (l / 32) .. + 15 bytes of a 32-byte K-step
//     (int8: 16 values; fp16: 8 values; FP6: 32 six-bit codes in 24 bytes of
//     a 64-value step, k-range 32 (l / 32) .. + 31).
//   32 x 32 accumulators: element e of lane l is row 8 (e / 4) + 4 (l / 32)
//     + e % 4, column l % 32.
//   ds_read_b64_tr_b8: within each 16-lane group g, lane 16 g + 8 h + c
//     receives byte c of the eight 8-byte rows that lanes 16 g + 2 b + h
//     address (b = 0 .. 7), in order of b.
//   buffer_load_dwordx4 ... lds: lane l's 16 bytes land at M0 + 16 l.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../precision_dense_gemm_02_amd/csrc/gemm_kernels.hpp"

using namespace lpgemm;

namespace {

__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// A: 32 rows x 32 int8 (row-major), Bt: 32 rows (columns of B) x 32 int8;
// C = A . B, 32 x 32 int32 row-major
__global__ __launch_bounds__(64) void k_mfma_i8(const int8_t* A, const int8_t* Bt, int32_t* C) {
  const int l = threadIdx.x;
  const i32x4 a = *(const i32x4*)(A + (l & 31) * 32 + 16 * (l >> 5));
  const i32x4 b = *(const i32x4*)(Bt + (l & 31) * 32 + 16 * (l >> 5));
  i32x16 acc;
  for (int e = 0; e < 16; ++e) acc[e] = 0;
  acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc, 0, 0, 0);
  for (int e = 0; e < 16; ++e) C[acc_row(e, l) * 32 + (l & 31)] = acc[e];
}

// A: 32 x 16 binary16, Bt: 32 x 16 binary16; C = A . B in fp32
__global__ __launch_bounds__(64) void k_mfma_f16(const uint16_t* A, const uint16_t* Bt, float* C) {
  const int l = threadIdx.x;
  const i32x4 a = *(const i32x4*)(A + (l & 31) * 16 + 8 * (l >> 5));
  const i32x4 b = *(const i32x4*)(Bt + (l & 31) * 16 + 8 * (l >> 5));
  f32x16 acc;
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0,
                                               0, 0);
  for (int e = 0; e < 16; ++e) C[acc_row(e, l) * 32 + (l & 31)] = acc[e];
}

// FP6 E3M2 operands, 64 values of k per row: row r's codes for k = 32 h ..
// 32 h + 31 are 24 bytes at r * 48 + 24 h (code i in bits 6 i .. 6 i + 5,
// little-endian); both block scales 2^0
__global__ __launch_bounds__(64) void k_mfma_e3m2(const uint8_t* A, const uint8_t* Bt, float* C) {
  const int l = threadIdx.x;
  i32x8 a = {0, 0, 0, 0, 0, 0, 0, 0}, b = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint8_t* pa = A + (l & 31) * 48 + 24 * (l >> 5);
  const uint8_t* pb = Bt + (l & 31) * 48 + 24 * (l >> 5);
  for (int d = 0; d < 6; ++d) {
    uint32_t wa = 0, wb = 0;
    for (int x = 0; x < 4; ++x) {
      wa |= (uint32_t)pa[4 * d + x] << (8 * x);
      wb |= (uint32_t)pb[4 * d + x] << (8 * x);
    }
    a[d] = (int)wa;
    b[d] = (int)wb;
  }
  f32x16 acc;
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 3, 3, 0, 127, 0, 127);
  for (int e = 0; e < 16; ++e) C[acc_row(e, l) * 32 + (l & 31)] = acc[e];
}

// 1 KiB of bytes into LDS, then one ds_read_b64_tr_b8 per lane at the LDS
// byte offset addr[lane]; out: 8 bytes per lane
__global__ __launch_bounds__(64) void k_ds_read_tr8(const uint8_t* in, const int* addr, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[1024];
  const int l = threadIdx.x;
  *(i32x4*)(lds + 16 * l) = *(const i32x4*)(in + 16 * l);
  __syncthreads();
  typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
  const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(lds_address(lds + addr[l])));
  *(i32x2_t*)(out + 8 * l) = v;
}

// one direct-to-LDS load of 16 bytes per lane from in + voff[lane] (the
// library's lds_dma_16), then the whole 1 KiB of LDS copied out
__global__ __launch_bounds__(64) void k_lds_dma(const uint8_t* in, const uint32_t* voff, uint8_t* out) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[1024];
  const int l = threadIdx.x;
  *(i32x4*)(lds + 16 * l) = i32x4{-1, -1, -1, -1};
  __syncthreads();
  const i32x4 rsrc = make_rsrc(in, 4096);
  lds_dma_16(rsrc, lds_address(lds), voff[l]);
  wait_vmcnt<0>();
  __syncthreads();
  *(i32x4*)(out + 16 * l) = *(const i32x4*)(lds + 16 * l);
}

int launch1(const void* fn, void** args, hipStream_t s) {
  return hipLaunchKernel(fn, dim3(1), dim3(64), args, 0, s) == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

int probe_mfma_i8(const int8_t* A, const int8_t* Bt, int32_t* C, hipStream_t s) {
  void* a[] = {&A, &Bt, &C};
  return launch1((const void*)&k_mfma_i8, a, s);
}

int probe_mfma_f16(const uint16_t* A, const uint16_t* Bt, float* C, hipStream_t s) {
  void* a[] = {&A, &Bt, &C};
  return launch1((const void*)&k_mfma_f16, a, s);
}

int probe_mfma_e3m2(const uint8_t* A, const uint8_t* Bt, float* C, hipStream_t s) {
  void* a[] = {&A, &Bt, &C};
  return launch1((const void*)&k_mfma_e3m2, a, s);
}

int probe_ds_read_tr8(const uint8_t* in, const int* addr, uint8_t* out, hipStream_t s) {
  void* a[] = {&in, &addr, &out};
  return launch1((const void*)&k_ds_read_tr8, a, s);
}

int probe_lds_dma(const uint8_t* in, const uint32_t* voff, uint8_t* out, hipStream_t s) {
  void* a[] = {&in, &voff, &out};
  return launch1((const void*)&k_lds_dma, a, s);
}

}  // extern "C"
