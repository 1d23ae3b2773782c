// Host side of liblpgemm: the C-ABI entry points declared in include/lpgemm.h.
//
// Each call validates its arguments on the host (no HIP call before that),
// checks once per device that the device is gfx950, picks a tile
// configuration for the shape, and enqueues one kernel on the caller's
// stream.  Nothing is allocated and no state is kept between calls apart from
// the per-device property cache (and the configuration an ablation pins);
// the split-K entry points keep their per-tile counters in the caller's
// workspace.
// The GEMM launches themselves are in run_*.hip (one translation unit per
// operand kind, see dispatch.hpp).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/lpgemm.h"
#include "aux_kernels.hpp"
#include "dispatch.hpp"
#include "f64emu_kernels.hpp"

namespace lpgemm {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_device_mutex;
DeviceInfo g_devices[kMaxDevices];

// LPGEMM_FORCE_CONFIG=<n> in the environment pins a configuration from the
// library's load on (ablations from the command line); unset or out of
// range means automatic selection
int initial_forced_config() {
  const char* e = std::getenv("LPGEMM_FORCE_CONFIG");
  if (!e || !*e) return -1;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  return (end && *end == 0 && v >= 0 && v < CFG_COUNT) ? (int)v : -1;
}
}  // namespace

std::atomic<int> g_forced_config{initial_forced_config()};

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

}  // namespace lpgemm

using namespace lpgemm;

// Device memory of lpgemm_f64_emu_noalloc: the emulation's intermediates
// (row exponents, residues, reduced products) for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy until the
// process ends; host code uses only the address hipGetSymbolAddress returns
// for the current device, never this name.
static __device__ __align__(256) uint8_t scratch[LPGEMM_F64_EMU_NOALLOC_MAX_WORKSPACE];

namespace {

// The scratch's device address, looked up once per device with that device
// current (each device has its own copy at its own address).
std::mutex g_scratch_mutex;
void* g_scratch_ptr[64] = {};

lpgemm_status scratch_address(void*& out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LPGEMM_ERROR_ARCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LPGEMM_ERROR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  out = g_scratch_ptr[dev];
  return LPGEMM_SUCCESS;
}

}  // namespace

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

// Host checks of the fp64 emulation, in the header's order, short of the
// workspace; sets the modulus count and the workspace layout.  M = 0 or
// N = 0 returns success with nothing else checked.
lpgemm_status f64emu_check(int64_t M, int64_t N, int64_t K, const double* A, const double* B, const double* C,
                           int bits, int& s, F64EmuLayout& L) {
  if (M < 0 || N < 0 || K < 0 || M > INT32_MAX || N > INT32_MAX) return LPGEMM_ERROR_INVALID_VALUE;
  if (bits < 1 || bits > 53) return LPGEMM_ERROR_INVALID_VALUE;
  if (K % 16 != 0 || K > LPGEMM_MAX_K_INT) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return LPGEMM_SUCCESS;
  if (!C) return LPGEMM_ERROR_INVALID_VALUE;
  if (K > 0 && (!A || !B)) return LPGEMM_ERROR_INVALID_VALUE;
  s = f64emu_moduli(K, bits);
  if (s < 0) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  L = f64emu_layout(M, N, K, s);
  if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B)))) return LPGEMM_ERROR_MISALIGNED;
  return LPGEMM_SUCCESS;
}

// The emulation's launches on `stream`, with its intermediates in `ws`
// (laid out as L; every byte a launch reads was written by an earlier one).
lpgemm_status f64emu_enqueue(int64_t M, int64_t N, int64_t K, const double* A, const double* B, double* C,
                             int bits, int s, const F64EmuLayout& L, uint8_t* ws, hipStream_t stream) {
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
    const lpgemm_status st = run<KIND_I8_MOD>(M, N, K, RA + (size_t)l * M * K, RB + (size_t)l * N * K,
                                              CR + (size_t)l * cr_stride, nullptr, nullptr, stream, c.m[l]);
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
  int s = 0;
  F64EmuLayout L{};
  lpgemm_status st = f64emu_check(M, N, K, A, B, C, bits, s, L);
  if (st != LPGEMM_SUCCESS || M == 0 || N == 0) return st;
  if (!workspace) return LPGEMM_ERROR_INVALID_VALUE;
  if (workspace_bytes < L.total) return LPGEMM_ERROR_INVALID_VALUE;
  if (((uintptr_t)workspace & 255) != 0) return LPGEMM_ERROR_MISALIGNED;
  DeviceInfo dev;
  st = current_device(dev);
  if (st != LPGEMM_SUCCESS) return st;
  return f64emu_enqueue(M, N, K, A, B, C, bits, s, L, static_cast<uint8_t*>(workspace), stream);
}

lpgemm_status lpgemm_f64_emu_noalloc(int64_t M, int64_t N, int64_t K, const double* A, const double* B,
                                     double* C, int bits, hipStream_t stream) {
  int s = 0;
  F64EmuLayout L{};
  lpgemm_status st = f64emu_check(M, N, K, A, B, C, bits, s, L);
  if (st != LPGEMM_SUCCESS || M == 0 || N == 0) return st;
  if (L.total > LPGEMM_F64_EMU_NOALLOC_MAX_WORKSPACE) return LPGEMM_ERROR_UNSUPPORTED_SHAPE;
  DeviceInfo dev;
  st = current_device(dev);
  if (st != LPGEMM_SUCCESS) return st;
  void* ptr = nullptr;
  st = scratch_address(ptr);
  if (st != LPGEMM_SUCCESS) return st;
  return f64emu_enqueue(M, N, K, A, B, C, bits, s, L, static_cast<uint8_t*>(ptr), stream);
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

int64_t lpgemm_splitk_workspace(int64_t M, int64_t N) {
  if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX) return -1;
  DeviceInfo dev;
  if (current_device(dev) != LPGEMM_SUCCESS) return -1;
  const int64_t t = (int64_t)tiles(M, kSplitTile) * tiles(N, kSplitTile);
  return splitk_auto_shape(M, N, dev.cu_count) ? splitk_bytes(t, kMaxSplits) : 0;
}

lpgemm_status lpgemm_i8_splitk(int64_t M, int64_t N, int64_t K, const int8_t* A, const int8_t* B, int32_t* C,
                               void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return run<KIND_I8>(M, N, K, A, B, C, nullptr, nullptr, stream, 0, workspace, workspace_bytes);
}

lpgemm_status lpgemm_i4_splitk(int64_t M, int64_t N, int64_t K, const uint8_t* A_packed, const uint8_t* B_packed,
                               int32_t* C, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return run<KIND_I4>(M, N, K, A_packed, B_packed, C, nullptr, nullptr, stream, 0, workspace, workspace_bytes);
}

lpgemm_status lpgemm_f16_splitk(int64_t M, int64_t N, int64_t K, const void* A, const void* B, float* C,
                                void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return run<KIND_F16>(M, N, K, A, B, C, nullptr, nullptr, stream, 0, workspace, workspace_bytes);
}

lpgemm_status lpgemm_i8_dequant_splitk(int64_t M, int64_t N, int64_t K, const int8_t* A, const int8_t* B,
                                       const float* row_scale, const float* col_scale, float* C, void* workspace,
                                       int64_t workspace_bytes, hipStream_t stream) {
  return run<KIND_I8_DEQUANT>(M, N, K, A, B, C, row_scale, col_scale, stream, 0, workspace, workspace_bytes);
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
  return launch<32, 32>((const void*)&gemm_skinny_pipe<KIND_I8_DEQUANT, 4, 1, true, 1, 1>, args, 256, stream);
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

int lpgemm_version(void) { return 301; }

int lpgemm_config_count(void) { return CFG_COUNT; }

int lpgemm_auto_config(int kind, int64_t M, int64_t N, int64_t K, int cu_count) {
  if (kind < KIND_I8 || kind > KIND_I8_DEQUANT || cu_count < 1) return -1;
  if (M <= 0 || N <= 0 || K < 0 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return -1;
  return (int)auto_config(M, N, K, cu_count, kind);
}

int lpgemm_force_config(int config) {
  const int v = (config >= 0 && config < CFG_COUNT) ? config : -1;
  return g_forced_config.exchange(v);
}

}  // extern "C"
