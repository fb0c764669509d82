// The fused LayerNorm forward kernel: row statistics, affine, scale, FP8 cast
// and per-tensor amax in one pass (and the plain bf16-output LayerNorm); the
// per-row work lives in ln_fwd_body.hpp.
#include "device_common.hpp"
#include "launchers.hpp"
#include "ln_fwd_body.hpp"

namespace fp8ln {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

template <int CPL, int FMT, bool FULL>
__global__ __launch_bounds__(kThreads) void ln_cast_amax_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ gamma, const uint4* __restrict__ beta,
    int64_t rows, int hidden, float eps, const float* __restrict__ scale_ptr,
    float* __restrict__ amax_ptr, void* __restrict__ out, float* __restrict__ mean_out,
    float* __restrict__ rstd_out) {
    ln_cast_amax_rows<CPL, FMT, FULL, kThreads>(x, gamma, beta, rows, hidden, eps, scale_ptr,
                                                amax_ptr, out, mean_out, rstd_out, blockIdx.x,
                                                gridDim.x);
}

template <int CPL, bool FULL>
hipError_t launch_ln_fwd_full(int64_t rows, int hidden, const void* x, const void* gamma,
                              const void* beta, float eps, int fp8, const float* scale,
                              float* amax, void* out, float* mean, float* rstd,
                              hipStream_t stream) {
    // Resident grid: as many workgroups as the CUs hold at once, each looping
    // over rows, so the row prefetch runs across the whole sweep instead of
    // restarting per wave (a second round of workgroups would run alone at the
    // end of the sweep).
    static int resident[3] = {0, 0, 0};   // per output format, from the occupancy query
    int& per_cu = resident[fp8];
    if (per_cu == 0) {
        int nb = 0;
        hipError_t e = fp8 == kE4M3
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                  &nb, ln_cast_amax_kernel<CPL, kE4M3, FULL>, kThreads, 0)
            : fp8 == kE5M2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                 &nb, ln_cast_amax_kernel<CPL, kE5M2, FULL>, kThreads, 0)
                           : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                                 &nb, ln_cast_amax_kernel<CPL, kLnOutBf16, FULL>, kThreads, 0);
        if (e != hipSuccess) return e;
        int dev = 0, cus = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
            hipSuccess)
            return e;
        per_cu = (nb > 0 ? nb : 1) * cus;
    }
    if (rows == 0) return hipSuccess;
    int64_t want = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    const int blocks = (int)(want < per_cu ? want : per_cu);
    if (fp8 == kE4M3)
        hipLaunchKernelGGL((ln_cast_amax_kernel<CPL, kE4M3, FULL>), dim3(blocks), dim3(kThreads),
                           0, stream, (const uint4*)x, (const uint4*)gamma, (const uint4*)beta,
                           rows, hidden, eps, scale, amax, out, mean, rstd);
    else if (fp8 == kE5M2)
        hipLaunchKernelGGL((ln_cast_amax_kernel<CPL, kE5M2, FULL>), dim3(blocks), dim3(kThreads),
                           0, stream, (const uint4*)x, (const uint4*)gamma, (const uint4*)beta,
                           rows, hidden, eps, scale, amax, out, mean, rstd);
    else
        hipLaunchKernelGGL((ln_cast_amax_kernel<CPL, kLnOutBf16, FULL>), dim3(blocks),
                           dim3(kThreads), 0, stream, (const uint4*)x, (const uint4*)gamma,
                           (const uint4*)beta, rows, hidden, eps, scale, amax, out, mean, rstd);
    return hipGetLastError();
}

template <int CPL>
hipError_t launch_ln_fwd_cpl(int64_t rows, int hidden, const void* x, const void* gamma,
                             const void* beta, float eps, int fp8, const float* scale,
                             float* amax, void* out, float* mean, float* rstd,
                             hipStream_t stream) {
    if (hidden == CPL * kWave * 8)
        return launch_ln_fwd_full<CPL, true>(rows, hidden, x, gamma, beta, eps, fp8, scale, amax,
                                             out, mean, rstd, stream);
    return launch_ln_fwd_full<CPL, false>(rows, hidden, x, gamma, beta, eps, fp8, scale, amax,
                                          out, mean, rstd, stream);
}

}  // namespace

hipError_t launch_ln_cast_amax(int64_t rows, int hidden, const void* x, const void* gamma,
                               const void* beta, float eps, int fp8, const float* scale,
                               float* amax, void* out, float* mean, float* rstd,
                               hipStream_t stream) {
    const int chunks = hidden / 8;
    if (chunks <= 64)
        return launch_ln_fwd_cpl<1>(rows, hidden, x, gamma, beta, eps, fp8, scale, amax, out,
                                    mean, rstd, stream);
    if (chunks <= 128)
        return launch_ln_fwd_cpl<2>(rows, hidden, x, gamma, beta, eps, fp8, scale, amax, out,
                                    mean, rstd, stream);
    if (chunks <= 256)
        return launch_ln_fwd_cpl<4>(rows, hidden, x, gamma, beta, eps, fp8, scale, amax, out,
                                    mean, rstd, stream);
    if (chunks <= 512)
        return launch_ln_fwd_cpl<8>(rows, hidden, x, gamma, beta, eps, fp8, scale, amax, out,
                                    mean, rstd, stream);
    return launch_ln_fwd_cpl<16>(rows, hidden, x, gamma, beta, eps, fp8, scale, amax, out,
                                 mean, rstd, stream);
}

}  // namespace fp8ln
