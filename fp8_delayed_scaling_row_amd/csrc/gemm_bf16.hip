// GEMM kernels on bf16 operands (the BF16 path); see gemm_kernels.hpp.
#include "gemm_kernels.hpp"

namespace fp8ln {

// The tiles count K in bytes: a bf16 product of K elements is 2 K bytes long.
hipError_t launch_gemm_bf16_ops(const GemmParams& p, hipStream_t stream) {
    GemmParams q = p;
    q.K = 2 * p.K;
    switch (p.epilogue) {
        case kEpiBf16Bias: return launch_typed<kOpBf16, kOpBf16, kEpiBf16Bias, kE4M3>(q, stream);
        case kEpiF32: return launch_typed<kOpBf16, kOpBf16, kEpiF32, kE4M3>(q, stream);
        case kEpiGeluBf16: return launch_act<kOpBf16, kOpBf16, kEpiGeluBf16, kE4M3>(q, stream);
        case kEpiDGeluF32: return launch_typed<kOpBf16, kOpBf16, kEpiDGeluF32, kE4M3>(q, stream);
        case kEpiDGeluBf16: return launch_typed<kOpBf16, kOpBf16, kEpiDGeluBf16, kE4M3>(q, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fp8ln
