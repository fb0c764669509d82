// FP8 GEMM kernels for operands E4M3 X E5M2 (A x B); see gemm_kernels.hpp.
#include "gemm_kernels.hpp"

namespace fp8ln {
FP8LN_GEMM_PAIR_DEFINE(kE4M3, kE5M2, e4m3_e5m2)
}  // namespace fp8ln
