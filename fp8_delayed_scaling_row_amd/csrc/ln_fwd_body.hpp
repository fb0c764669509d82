// The fused LayerNorm forward's per-row work as a device function: row
// statistics, affine, scale, FP8 cast and per-tensor amax (or the plain bf16
// LayerNorm), for the LayerNorm kernel and for launches that run it beside
// other jobs.
//
// The fused modules normalise each row and feed the result to an FP8 linear
// layer in one operation (tutorial "Accelerating Transformer Training with
// NVIDIA Transformer Engine ...", setup listing: LayerNormLinear, LayerNormMLP;
// "Turbo-charging your transformer training", "The building blocks").  Epsilon
// and the variance estimator are not on the pages: biased variance and the
// recipe's epsilon (1e-5 by default, as in torch.nn.LayerNorm, which the
// tutorial's plain-PyTorch mirror block uses).
//
// Layout: one 64-lane wave owns one row at a time; lane l holds the row's 16-byte
// chunks l, l+64, l+128, ... (8 bf16 each), so every load and store of a wave is
// one contiguous, fully coalesced span.  The row stays in registers between the
// two statistics passes and the output pass, so x is read from HBM exactly once.
#pragma once

#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

// CPL: 16-byte chunks per lane (hidden <= CPL * 64 * 8).
//
// The kernel is bound by VALU issue (a wave64 fp32 operation occupies a SIMD for
// four cycles), so it is written to spend few operations per element: the row
// is widened once and kept centred (x - mean) in fp32 registers between the
// passes, gamma and beta are widened once per workgroup into LDS, rows that fill
// every lane skip the per-element validity test, and the amax uses a
// three-operand max.  Memory-level parallelism: a wave loads the next row it owns
// (packed bf16, non-temporal) before it works on the current one.  Row
// statistics use DPP reductions inside 16-lane rows.  FULL: hidden is exactly
// CPL * 512, so every lane owns CPL whole chunks and no lane needs masking.
// FMT kLnOutBf16 is the plain LayerNorm: y rounded to bf16, no scale, no amax.
// NTHR threads per workgroup; workgroup `vblock` of `vgrid` (the kernel's own
// grid, or a share of a larger launch that also runs other jobs).  `pre` runs
// once the first row is in flight and before *scale_ptr is read (a launch that
// forms the scale itself does so there, its loads overlapping the row's); all
// threads call it.  CHECK: as block_amax_atomic's.
template <int CPL, int FMT, bool FULL, int NTHR, bool CHECK = true, class Pre = NoPre>
__device__ __forceinline__ void ln_cast_amax_rows(
    const uint4* __restrict__ x, const uint4* __restrict__ gamma, const uint4* __restrict__ beta,
    int64_t rows, int hidden, float eps, const float* scale_ptr,
    float* __restrict__ amax_ptr, void* __restrict__ out, float* __restrict__ mean_out,
    float* __restrict__ rstd_out, int vblock, int vgrid, Pre pre = {}) {
    constexpr int kWavesPerBlock = NTHR / kWave;
    __shared__ float4 gb[2][CPL * kWave][2];   // gamma, beta widened to fp32, 8 per chunk
    __shared__ uint32_t red[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nchunk = FULL ? CPL * kWave : hidden / 8;
    const float inv_h = 1.0f / (float)hidden;
    constexpr bool kBf16 = FMT == kLnOutBf16;

    const int64_t stride = (int64_t)vgrid * kWavesPerBlock;
    int64_t row = (int64_t)vblock * kWavesPerBlock + wave;
    uint4 nxt[CPL];
    // Past the last row a wave reloads the last row instead (and never uses it),
    // so the loads need no branch and the loop-carried row needs no copies.
    auto load_row = [&](int64_t r) {
        const uint4* xr = x + (r < rows ? r : rows - 1) * nchunk;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + i * kWave;
            nxt[i] = (FULL || c < nchunk) ? load_nt(xr + c) : make_uint4(0, 0, 0, 0);
        }
    };
    // the first row is in flight while gamma and beta are staged (small grids
    // would otherwise wait for two memory round trips in a row)
    load_row(row);

    for (int c = threadIdx.x; c < CPL * kWave; c += NTHR) {
        float g[8], b[8];
        unpack_bf16x8(c < nchunk ? gamma[c] : make_uint4(0, 0, 0, 0), g);
        unpack_bf16x8(c < nchunk ? beta[c] : make_uint4(0, 0, 0, 0), b);
        gb[0][c][0] = make_float4(g[0], g[1], g[2], g[3]);
        gb[0][c][1] = make_float4(g[4], g[5], g[6], g[7]);
        gb[1][c][0] = make_float4(b[0], b[1], b[2], b[3]);
        gb[1][c][1] = make_float4(b[4], b[5], b[6], b[7]);
    }
    __syncthreads();
    pre();
    const float s = kBf16 ? 1.0f : *scale_ptr;

    uint32_t amax_bits = 0;
    for (; row < rows; row += stride) {
        float d[CPL * 8];
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            unpack_bf16x8(nxt[i], d + 8 * i);
#pragma unroll
            for (int k = 0; k < 8; ++k) sum += d[8 * i + k];
        }
        // the next row goes in flight now; the fence keeps the compiler from
        // hoisting these loads above the widening (which would copy the row)
        __builtin_amdgcn_sched_barrier(0);
        load_row(row + stride);
        const float mu = wave_sum_dpp(sum) * inv_h;
        float sq = 0.0f;
        if constexpr (FULL) {
#pragma unroll
            for (int j = 0; j < CPL * 8; ++j) {
                d[j] -= mu;
                sq += d[j] * d[j];
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const bool valid = lane + i * kWave < nchunk;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    d[8 * i + k] = valid ? d[8 * i + k] - mu : 0.0f;
                    sq += d[8 * i + k] * d[8 * i + k];
                }
            }
        }
        const float var = wave_sum_dpp(sq) * inv_h;
        const float rs = 1.0f / sqrtf(var + eps);

        uint2* orow = (uint2*)out + row * nchunk;
        uint4* orow16 = (uint4*)out + row * nchunk;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + i * kWave;
            if (FULL || c < nchunk) {
                const float4 g0 = gb[0][c][0], g1 = gb[0][c][1];
                const float4 b0 = gb[1][c][0], b1 = gb[1][c][1];
                const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                float y[8], ys[8];
                uint32_t cm = amax_bits;
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = fmaf(d[8 * i + k] * rs, gg[k], bb[k]);
                if constexpr (kBf16) {
                    uint4 w;
                    w.x = pack_bf16x2(y[0], y[1]);
                    w.y = pack_bf16x2(y[2], y[3]);
                    w.z = pack_bf16x2(y[4], y[5]);
                    w.w = pack_bf16x2(y[6], y[7]);
                    store_nt(orow16 + c, w);
                } else {
#pragma unroll
                    for (int k = 0; k < 8; k += 2)
                        cm = max(cm, max(abs_bits(y[k]), abs_bits(y[k + 1])));   // v_max3_u32
#pragma unroll
                    for (int k = 0; k < 8; ++k) ys[k] = y[k] * s;
                    uint2 q;
                    q.x = encode4<FMT>(ys[0], ys[1], ys[2], ys[3]);
                    q.y = encode4<FMT>(ys[4], ys[5], ys[6], ys[7]);
                    if (__builtin_expect(cm > kInfBits, 0)) {
                        q.x = patch_nan4(q.x, ys);
                        q.y = patch_nan4(q.y, ys + 4);
                    }
                    store_nt(orow + c, q);
                    amax_bits = cm;
                }
            }
        }
        if (lane == 0) {
            if (mean_out) mean_out[row] = mu;
            if (rstd_out) rstd_out[row] = rs;
        }
    }
    if constexpr (!kBf16) block_amax_atomic<CHECK>(amax_bits, amax_ptr, red);
}


}  // namespace fp8ln
