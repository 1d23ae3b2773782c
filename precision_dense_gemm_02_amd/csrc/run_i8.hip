// The int8 (K-contiguous B) GEMM kernels: every configuration of run<KIND_I8>.
#include "run_kernels.hpp"

namespace lpgemm {
template lpgemm_status run<KIND_I8, false>(int64_t, int64_t, int64_t, const void*, const void*, void*, const float*,
                                       const float*, hipStream_t, int, void*, int64_t);
}  // namespace lpgemm
