// The GEMM kernels of the smaller paths: int4 re-encoded as FP6 E3M2, the
// int8 product reduced modulo a small integer (fp64 emulation), and int8
// with B stored K x N.
#include "run_kernels.hpp"

namespace lpgemm {
template lpgemm_status run<KIND_I4_E3M2, false>(int64_t, int64_t, int64_t, const void*, const void*, void*,
                                                const float*, const float*, hipStream_t, int, void*, int64_t);
template lpgemm_status run<KIND_I8_MOD, false>(int64_t, int64_t, int64_t, const void*, const void*, void*,
                                               const float*, const float*, hipStream_t, int, void*, int64_t);
template lpgemm_status run<KIND_I8, true>(int64_t, int64_t, int64_t, const void*, const void*, void*,
                                          const float*, const float*, hipStream_t, int, void*, int64_t);
}  // namespace lpgemm
