// LayerNorm backward: dx plus deterministic dgamma / dbeta.
//
// With xhat = (x - mean) * rstd and g = dy * gamma per row,
//     dx = rstd * (g - mean_j g - xhat * mean_j(g * xhat)),
//     dgamma = sum over rows of dy * xhat,  dbeta = sum over rows of dy,
// the gradient of the LayerNorm the fused modules apply before their first linear
// layer (tutorial "Accelerating Transformer Training with NVIDIA Transformer
// Engine ...", setup listing: LayerNormLinear, LayerNormMLP).  One wave per row,
// lane l owning 16-byte chunks l, l+64, ... of the row, as in the forward.
#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// ---- backward --------------------------------------------------------------

// Per block: rows handled by its waves in grid-stride order; per lane: dgamma and
// dbeta partial sums of its own columns.  Partials go to ws[block][2][hidden] and a
// second kernel adds the blocks in a fixed order, so results are deterministic.
// DY_BF16: dy arrives as bf16 (the plain LayerNorm module) instead of fp32 (the
// dgrad GEMM's output inside the fused modules).
template <int CPL, bool DY_BF16>
__global__ __launch_bounds__(kThreads) void ln_bwd_kernel(
    const void* __restrict__ dy_raw, const uint4* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const uint4* __restrict__ gamma, uint4* __restrict__ dx,
    float* __restrict__ partial, int64_t rows, int hidden) {
    extern __shared__ float4 sm_raw[];   // [2][hidden] floats: dgamma, dbeta of the block
    float* sm = reinterpret_cast<float*>(sm_raw);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nchunk = hidden / 8;
    const float inv_h = 1.0f / (float)hidden;

    float g[CPL * 8];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) unpack_bf16x8(gamma[c], g + 8 * i);
        else
#pragma unroll
            for (int k = 0; k < 8; ++k) g[8 * i + k] = 0.0f;
    }
    float dg[CPL * 8], db[CPL * 8];
#pragma unroll
    for (int j = 0; j < CPL * 8; ++j) { dg[j] = 0.0f; db[j] = 0.0f; }

    for (int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + wave; row < rows;
         row += (int64_t)gridDim.x * kWavesPerBlock) {
        // Every load of the row goes out before any is used: chunks past the row
        // read the row's last chunk (the index is clamped, so there is no branch
        // around the loads) and are masked below.  With a branch per chunk the
        // compiler waits for each chunk's loads before issuing the next chunk's,
        // and a row costs one memory round trip per chunk.
        const float mu = mean[row];
        const float rs = rstd[row];
        uint4 xr[CPL], dr[DY_BF16 ? CPL : 2 * CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + i * kWave;
            const int64_t cc = row * nchunk + (c < nchunk ? c : nchunk - 1);
            xr[i] = load_nt(x + cc);
            if constexpr (DY_BF16) {
                dr[i] = load_nt((const uint4*)dy_raw + cc);
            } else {
                dr[2 * i] = load_nt((const uint4*)dy_raw + 2 * cc);
                dr[2 * i + 1] = load_nt((const uint4*)dy_raw + 2 * cc + 1);
            }
        }
        float xh[CPL * 8], d[CPL * 8];
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const bool valid = lane + i * kWave < nchunk;
            unpack_bf16x8(xr[i], xh + 8 * i);
            if constexpr (DY_BF16) {
                unpack_bf16x8(dr[i], d + 8 * i);
            } else {
                const uint4 a = dr[2 * i], b2 = dr[2 * i + 1];
                const uint32_t w[8] = {a.x, a.y, a.z, a.w, b2.x, b2.y, b2.z, b2.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) d[8 * i + k] = __uint_as_float(w[k]);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {   // chunks past the row: xhat 0, no gradient
                xh[8 * i + k] = valid ? xh[8 * i + k] : mu;
                d[8 * i + k] = valid ? d[8 * i + k] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = 8 * i + k;
                xh[j] = (xh[j] - mu) * rs;
                const float gj = d[j] * g[j];
                s1 += gj;
                s2 += gj * xh[j];
                dg[j] += d[j] * xh[j];
                db[j] += d[j];
            }
        }
        const float c1 = wave_sum(s1) * inv_h;
        const float c2 = wave_sum(s2) * inv_h;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + i * kWave;
            if (c < nchunk) {
                float o[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int j = 8 * i + k;
                    o[k] = rs * (d[j] * g[j] - c1 - xh[j] * c2);
                }
                uint4 w;
                w.x = pack_bf16x2(o[0], o[1]);
                w.y = pack_bf16x2(o[2], o[3]);
                w.z = pack_bf16x2(o[4], o[5]);
                w.w = pack_bf16x2(o[6], o[7]);
                store_nt(dx + row * nchunk + c, w);
            }
        }
    }
    // combine the block's waves in a fixed order (wave 0 first), 16 bytes at a
    // time: a lane's eight columns are 32 contiguous bytes of LDS, and 4-byte
    // accesses at that lane stride would meet in a few banks
    float4* sg = reinterpret_cast<float4*>(sm);
    float4* sd = reinterpret_cast<float4*>(sm + hidden);
    for (int w = 0; w < kWavesPerBlock; ++w) {
        if (wave == w) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = lane + i * kWave;
                if (c < nchunk) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float* a = dg + 8 * i + 4 * h;
                        const float* b = db + 8 * i + 4 * h;
                        float4 ga = make_float4(a[0], a[1], a[2], a[3]);
                        float4 da = make_float4(b[0], b[1], b[2], b[3]);
                        if (w != 0) {
                            const float4 go = sg[2 * c + h], dold = sd[2 * c + h];
                            ga = make_float4(go.x + ga.x, go.y + ga.y, go.z + ga.z, go.w + ga.w);
                            da = make_float4(dold.x + da.x, dold.y + da.y, dold.z + da.z,
                                             dold.w + da.w);
                        }
                        sg[2 * c + h] = ga;
                        sd[2 * c + h] = da;
                    }
                }
            }
        }
        __syncthreads();
    }
    // 4-byte stores: the workspace carries no alignment promise
    float* pb = partial + (int64_t)blockIdx.x * 2 * hidden;
    for (int j = threadIdx.x; j < 2 * hidden; j += kThreads) pb[j] = sm[j];
}

int ln_bwd_blocks(int64_t rows) {
    const int64_t want = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = 512;
    return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

template <int CPL>
hipError_t launch_ln_bwd_cpl(int64_t rows, int hidden, const void* dy, bool dy_bf16,
                             const void* x, const float* mean, const float* rstd,
                             const void* gamma, void* dx, float* dgamma, float* dbeta,
                             void* workspace, hipStream_t stream, SumBatch* sums) {
    const int blocks = ln_bwd_blocks(rows);
    const size_t smem = (size_t)2 * hidden * sizeof(float);
    float* partial = (float*)workspace;
    if (dy_bf16)
        hipLaunchKernelGGL((ln_bwd_kernel<CPL, true>), dim3(blocks), dim3(kThreads), smem, stream,
                           dy, (const uint4*)x, mean, rstd, (const uint4*)gamma, (uint4*)dx,
                           partial, rows, hidden);
    else
        hipLaunchKernelGGL((ln_bwd_kernel<CPL, false>), dim3(blocks), dim3(kThreads), smem,
                           stream, dy, (const uint4*)x, mean, rstd, (const uint4*)gamma,
                           (uint4*)dx, partial, rows, hidden);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (sums && sums->add(partial, blocks, 2 * (int64_t)hidden, dgamma, dbeta, hidden))
        return hipSuccess;
    return launch_sum_partials(partial, blocks, 2 * (int64_t)hidden, dgamma, dbeta, hidden,
                               stream);
}

}  // namespace

size_t ln_bwd_workspace(int64_t rows, int hidden) {
    return (size_t)ln_bwd_blocks(rows) * 2 * (size_t)hidden * sizeof(float);
}

hipError_t launch_ln_bwd(int64_t rows, int hidden, const void* dy, bool dy_bf16, const void* x,
                         const float* mean, const float* rstd, const void* gamma, void* dx,
                         float* dgamma, float* dbeta, void* workspace, hipStream_t stream,
                         SumBatch* sums) {
    const int chunks = hidden / 8;
    if (chunks <= 64)
        return launch_ln_bwd_cpl<1>(rows, hidden, dy, dy_bf16, x, mean, rstd, gamma, dx, dgamma, dbeta,
                                    workspace, stream, sums);
    if (chunks <= 128)
        return launch_ln_bwd_cpl<2>(rows, hidden, dy, dy_bf16, x, mean, rstd, gamma, dx, dgamma, dbeta,
                                    workspace, stream, sums);
    if (chunks <= 256)
        return launch_ln_bwd_cpl<4>(rows, hidden, dy, dy_bf16, x, mean, rstd, gamma, dx, dgamma, dbeta,
                                    workspace, stream, sums);
    return launch_ln_bwd_cpl<8>(rows, hidden, dy, dy_bf16, x, mean, rstd, gamma, dx, dgamma, dbeta,
                                workspace, stream, sums);
}

}  // namespace fp8ln
