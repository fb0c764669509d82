// The forward's memory-bound front in one launch: the LayerNorm + FP8 cast +
// amax of the input rows and the FP8 casts of the module's weights (one for
// LayerNormLinear, two for LayerNormMLP), each in its own workgroups.
//
// At the pages' GPT-sized shapes (a few hundred to a few thousand tokens through
// 768 -> 2304 or 768 -> 3072 -> 768 layers) these kernels are latency-bound: each
// touches a few MB, and separate launches would run one after the other with
// most CUs idle.  Side by side in one grid their latencies overlap.  The work of
// every workgroup is exactly that of the standalone kernels (the same device
// functions), so codes, statistics and amaxes are identical to theirs.
#include "cast_body.hpp"
#include "device_common.hpp"
#include "launchers.hpp"
#include "ln_fwd_body.hpp"
#include "step_update.hpp"

namespace fp8ln {

namespace {

constexpr int kThreads = 512;

struct ProloguePack {
    const uint4* x;
    const uint4* gamma;
    const uint4* beta;
    int64_t rows;
    int hidden;
    float eps;
    const float* scale;
    float* amax;
    void* out;
    float* mean;
    float* rstd;
    int ln_blocks;
    int n_casts;
    int cast_blocks[kMaxPrologueCasts];
    CastJob cast[kMaxPrologueCasts];
    int fused;          // the scaling update is folded in (upd below)
    FusedUpdate upd;
};

// Workgroups [0, ln_blocks) normalise rows; the following cast_blocks[0]
// workgroups cast the first weight, then the second.
template <int CPL, int FMT, bool FULL, bool FUSED>
__global__ __launch_bounds__(kThreads) void fwd_prologue_kernel(ProloguePack p) {
    // fused update: every slot's scale and 1 / scale, formed while the first
    // rows are in flight (the amaxes go to ws; the forward's last GEMM rolls
    // the history)
    __shared__ float sh[2 * kMaxMetaSlots];
    auto pre = [&]() { window_scales<kThreads>(p.upd, sh); };
    int b = blockIdx.x;
    if (b < p.ln_blocks) {
        if constexpr (FUSED) {
            const int q = p.upd.ln_slot;
            ln_cast_amax_rows<CPL, FMT, FULL, kThreads, true>(
                p.x, p.gamma, p.beta, p.rows, p.hidden, p.eps, sh + 2 * q,
                reinterpret_cast<float*>(p.upd.ws + q), p.out, p.mean, p.rstd, b, p.ln_blocks,
                pre);
        } else {
            ln_cast_amax_rows<CPL, FMT, FULL, kThreads>(p.x, p.gamma, p.beta, p.rows, p.hidden,
                                                        p.eps, p.scale, p.amax, p.out, p.mean,
                                                        p.rstd, b, p.ln_blocks);
        }
        return;
    }
    b -= p.ln_blocks;
    for (int j = 0; j < kMaxPrologueCasts; ++j) {   // block-uniform choice of the job
        if (j < p.n_casts && b < p.cast_blocks[j]) {
            const CastJob& c = p.cast[j];
            if constexpr (FUSED) {
                const int q = p.upd.cast_slot[j];
                cast_tiles<false, FMT, kThreads, true>(
                    c.in, c.rows, c.cols, sh + 2 * q, reinterpret_cast<float*>(p.upd.ws + q),
                    c.out, c.out_t, nullptr, sh + 2 * q + 1, c.copy_dst, b, p.cast_blocks[j], pre);
            } else {
                cast_tiles<false, FMT, kThreads>(c.in, c.rows, c.cols, c.scale, c.amax, c.out,
                                                 c.out_t, nullptr, c.copy_src, c.copy_dst, b,
                                                 p.cast_blocks[j]);
            }
            return;
        }
        b -= p.cast_blocks[j];
    }
}

template <class Kernel>
hipError_t capacity(Kernel k, int& cache) {
    if (cache > 0) return hipSuccess;
    int nb = 0, dev = 0, cus = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, kThreads, 0);
    if (e != hipSuccess) return e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
        hipSuccess)
        return e;
    cache = (nb > 0 ? nb : 1) * cus;
    return hipSuccess;
}

template <int CPL, int FMT, bool FULL, bool FUSED>
hipError_t launch_typed(ProloguePack& p, bool* launched, hipStream_t stream) {
    static int cap = 0;
    hipError_t e = capacity(fwd_prologue_kernel<CPL, FMT, FULL, FUSED>, cap);
    if (e != hipSuccess) return e;
    int64_t total = p.ln_blocks;
    for (int j = 0; j < p.n_casts; ++j) total += p.cast_blocks[j];
    // only when every workgroup is resident at once: the jobs then overlap fully
    if (total > cap) return hipSuccess;
    hipLaunchKernelGGL((fwd_prologue_kernel<CPL, FMT, FULL, FUSED>), dim3((unsigned)total),
                       dim3(kThreads), 0, stream, p);
    *launched = true;
    return hipGetLastError();
}

template <int CPL, bool FUSED>
hipError_t launch_cpl(ProloguePack& p, int fp8, bool* launched, hipStream_t stream) {
    const bool full = p.hidden == CPL * kWave * 8;
    if (fp8 == kE4M3)
        return full ? launch_typed<CPL, kE4M3, true, FUSED>(p, launched, stream)
                    : launch_typed<CPL, kE4M3, false, FUSED>(p, launched, stream);
    return full ? launch_typed<CPL, kE5M2, true, FUSED>(p, launched, stream)
                : launch_typed<CPL, kE5M2, false, FUSED>(p, launched, stream);
}

template <bool FUSED>
hipError_t launch_fused(ProloguePack& p, int fp8, bool* launched, hipStream_t stream) {
    const int chunks = p.hidden / 8;
    if (chunks <= 64) return launch_cpl<1, FUSED>(p, fp8, launched, stream);
    if (chunks <= 128) return launch_cpl<2, FUSED>(p, fp8, launched, stream);
    return launch_cpl<4, FUSED>(p, fp8, launched, stream);
}

}  // namespace

hipError_t launch_fwd_prologue(int64_t rows, int hidden, const void* x, const void* gamma,
                               const void* beta, float eps, int fp8, const float* scale,
                               float* amax, uint8_t* out, float* mean, float* rstd,
                               const CastJob* casts, int n_casts, bool* launched,
                               hipStream_t stream, const FusedUpdate* upd) {
    *launched = false;
    if (rows <= 0 || hidden > 2048 || n_casts < 0 || n_casts > kMaxPrologueCasts)
        return hipSuccess;
    ProloguePack p{};
    p.x = (const uint4*)x;
    p.gamma = (const uint4*)gamma;
    p.beta = (const uint4*)beta;
    p.rows = rows;
    p.hidden = hidden;
    p.eps = eps;
    p.scale = scale;
    p.amax = amax;
    p.out = out;
    p.mean = mean;
    p.rstd = rstd;
    p.ln_blocks = (int)((rows + kThreads / kWave - 1) / (kThreads / kWave));
    p.n_casts = n_casts;
    if (upd) {
        const int n = upd->n_slots;
        if (upd->len < 1 || upd->len > 1024 || n < 1 || n > kMaxMetaSlots || (n & (n - 1)))
            return hipSuccess;
        p.fused = 1;
        p.upd = *upd;
    }
    for (int j = 0; j < n_casts; ++j) {
        if (casts[j].rows <= 0 || casts[j].cols <= 0) return hipSuccess;
        p.cast[j] = casts[j];
        p.cast_blocks[j] = (int)(((casts[j].rows + kCT - 1) / kCT) * ((casts[j].cols + kCT - 1) / kCT));
    }
    return p.fused ? launch_fused<true>(p, fp8, launched, stream)
                   : launch_fused<false>(p, fp8, launched, stream);
}

}  // namespace fp8ln
