// FP8 GEMM on the CDNA4 matrix cores with fused dequantising epilogues.
//
// The linear layers of the fused modules run on FP8 operands ("Turbo-charging
// your transformer training", "Playing with lower-precision formats: BF16 vs
// FP8"; tutorial "Accelerating Transformer Training with NVIDIA Transformer
// Engine ...", intro: FP8 tensor cores).  Every product here is
//     C[m][n] = sum_k A[m][k] * B[n][k]
// with both operands stored with the contraction index last (u8 codes), fp32
// accumulation, and an epilogue that multiplies by the two operands' scale_inv
// and applies bias / GELU / GELU' and the output cast.  The forward, dgrad and
// wgrad products are all of this form once the cast kernels have written the
// transposed operand copies.
//
// Tiling (gfx950): a 256-thread workgroup computes a 128 x 128 tile; its four
// waves each own a 64 x 64 sub-tile made of 4 x 4 V_MFMA_F32_16X16X128_F8F6F4
// results (the operand formats E4M3/E5M2 are picked per operand by the
// instruction's cbsz/blgp fields).  The K loop steps 128 bytes at a time through
// a double-buffered LDS stage (2 x 32 KB) with an XOR swizzle on 16-byte chunks
// so that the fragment reads are bank-conflict free.  The epilogue goes through
// LDS so every global store is a full 16- or 32-byte vector per lane.  Tiles are
// ordered so that the blocks of one XCD (blocks are dealt to the 8 XCDs round
// robin) cover a compact band of the output and share its operands in their L2.
#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;                       // bytes of K per stage
constexpr int kStageBytes = BM * BK;          // one operand tile
constexpr int kCPitch = BN + 4;               // floats per row of the epilogue tile
constexpr int kCodePitch = BN + 16;           // bytes per row of the code tile
constexpr int kSmemBytes =
    (4 * kStageBytes > BM * kCPitch * 4) ? 4 * kStageBytes : BM * kCPitch * 4;
constexpr int kGroupM = 8;                    // tile rows per ordering group

// 16-byte chunk c of LDS row `row` lives at chunk position swz(row, c).
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }

// GELU, tanh form, with tanh(u) = 1 - 2 / (1 + e^(2u)).
__device__ __forceinline__ float gelu_f(float h, float* tanh_out) {
    const float k0 = 0.7978845608028654f;   // sqrt(2 / pi)
    const float k1 = 0.044715f;
    const float u = k0 * fmaf(k1 * h, h * h, h);
    const float e = __expf(2.0f * u);
    const float t = 1.0f - 2.0f / (1.0f + e);
    if (tanh_out) *tanh_out = t;
    return 0.5f * h * (1.0f + t);
}

__device__ __forceinline__ float gelu_grad_f(float h) {
    const float k0 = 0.7978845608028654f;
    const float k1 = 0.044715f;
    float t;
    gelu_f(h, &t);
    return 0.5f * (1.0f + t) + 0.5f * h * (1.0f - t * t) * k0 * fmaf(3.0f * k1, h * h, 1.0f);
}

template <int FA, int FB, int EPI, int QF>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const int64_t M = p.M, N = p.N, K = p.K;

    // ---- tile order ---------------------------------------------------------
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    int b = blockIdx.x;
    if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);   // one band per XCD
    const int per_group = kGroupM * tiles_n;
    const int first_m = (b / per_group) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int tile_m = first_m + (b % per_group) % gsize;
    const int tile_n = (b % per_group) / gsize;
    const int64_t m0 = (int64_t)tile_m * BM;
    const int64_t n0 = (int64_t)tile_n * BN;

    // ---- global -> LDS staging ---------------------------------------------
    const uint8_t* __restrict__ A = p.A;
    const uint8_t* __restrict__ B = p.B;
    uint4 ra[4], rb[4];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = t + kThreads * i;
            const int row = id >> 3;
            const int64_t k = k0 + (id & 7) * 16;
            const int64_t gm = m0 + row;
            const int64_t gn = n0 + row;
            ra[i] = (gm < M && k < K) ? *reinterpret_cast<const uint4*>(A + gm * K + k)
                                      : make_uint4(0, 0, 0, 0);
            rb[i] = (gn < N && k < K) ? *reinterpret_cast<const uint4*>(B + gn * K + k)
                                      : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
        uint8_t* sa = smem + buf * 2 * kStageBytes;
        uint8_t* sb = sa + kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = t + kThreads * i;
            const int row = id >> 3;
            const int off = row * BK + swz(row, id & 7) * 16;
            *reinterpret_cast<uint4*>(sa + off) = ra[i];
            *reinterpret_cast<uint4*>(sb + off) = rb[i];
        }
    };

    // ---- MFMA main loop ----------------------------------------------------
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int fr = lane & 15;   // row of the 16-row operand block this lane feeds
    const int fg = lane >> 4;   // which 32-byte slice of the 128-byte K step
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto load_frag = [&](const uint8_t* s, int row) -> v8i {
        const uint4 lo = *reinterpret_cast<const uint4*>(s + row * BK + swz(row, 2 * fg) * 16);
        const uint4 hi = *reinterpret_cast<const uint4*>(s + row * BK + swz(row, 2 * fg + 1) * 16);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    const int nk = (int)((K + BK - 1) / BK);
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
        const uint8_t* sa = smem + (kt & 1) * 2 * kStageBytes;
        const uint8_t* sb = sa + kStageBytes;
        v8i af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = load_frag(sa, wm * 64 + i * 16 + fr);
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[j] = load_frag(sb, wn * 64 + j * 16 + fr);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], bfr[j], acc[i][j], FA, FB, 0, 0, 0, 0);
        if (kt + 1 < nk) sstore((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: accumulators -> LDS tile (row-major fp32) ------------------
    float* cs = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                cs[(wm * 64 + i * 16 + 4 * fg + r) * kCPitch + wn * 64 + j * 16 + fr] = acc[i][j][r];
    __syncthreads();

    const float alpha = (*p.sinv_a) * (*p.sinv_b);
    // thread t handles 8 chunks of 8 consecutive columns: id = t + 256 i,
    // row = id / 16, columns 8 * (id % 16) .. +7
    uint2 codes[8];
    uint32_t amax_bits = 0;
    float qs = 0.0f;
    if constexpr (EPI == kEpiGeluFp8) qs = *p.q_scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int id = t + kThreads * i;
        const int row = id >> 4;
        const int c8 = (id & 15) * 8;
        const int64_t gm = m0 + row;
        const int64_t gn = n0 + c8;
        const float4 lo = *reinterpret_cast<const float4*>(cs + row * kCPitch + c8);
        const float4 hi = *reinterpret_cast<const float4*>(cs + row * kCPitch + c8 + 4);
        float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const bool ok = gm < M && gn < N;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] *= alpha;
        if constexpr (EPI == kEpiBf16Bias || EPI == kEpiGeluFp8) {
            if (p.bias && ok) {
                float bb[8];
                unpack_bf16x8(*reinterpret_cast<const uint4*>(p.bias + gn), bb);
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] += bb[k];
            }
        }
        if constexpr (EPI == kEpiBf16Bias) {
            if (ok) {
                uint4 w;
                w.x = pack_bf16x2(v[0], v[1]);
                w.y = pack_bf16x2(v[2], v[3]);
                w.z = pack_bf16x2(v[4], v[5]);
                w.w = pack_bf16x2(v[6], v[7]);
                *reinterpret_cast<uint4*>((uint16_t*)p.out + gm * N + gn) = w;
            }
        } else if constexpr (EPI == kEpiF32) {
            if (ok) {
                float4* o = reinterpret_cast<float4*>((float*)p.out + gm * N + gn);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        } else if constexpr (EPI == kEpiDGeluF32) {
            if (ok) {
                float hh[8];
                unpack_bf16x8(*reinterpret_cast<const uint4*>(p.h_in + gm * N + gn), hh);
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] *= gelu_grad_f(hh[k]);
                float4* o = reinterpret_cast<float4*>((float*)p.out + gm * N + gn);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        } else {   // kEpiGeluFp8
            if (ok && p.h_out) {
                uint4 w;
                w.x = pack_bf16x2(v[0], v[1]);
                w.y = pack_bf16x2(v[2], v[3]);
                w.z = pack_bf16x2(v[4], v[5]);
                w.w = pack_bf16x2(v[6], v[7]);
                *reinterpret_cast<uint4*>(p.h_out + gm * N + gn) = w;
            }
            float g[8], gs[8];
            uint32_t cm = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                g[k] = gelu_f(v[k], nullptr);
                const uint32_t ab = abs_bits(g[k]);
                cm = cm > ab ? cm : ab;
                gs[k] = g[k] * qs;
            }
            uint2 q;
            q.x = encode4<QF>(gs[0], gs[1], gs[2], gs[3]);
            q.y = encode4<QF>(gs[4], gs[5], gs[6], gs[7]);
            if (__builtin_expect(cm > kInfBits, 0)) {
                q.x = patch_nan4(q.x, gs);
                q.y = patch_nan4(q.y, gs + 4);
            }
            codes[i] = q;
            if (ok) {
                *reinterpret_cast<uint2*>(p.q_out + gm * N + gn) = q;
                amax_bits = amax_bits > cm ? amax_bits : cm;
            }
        }
    }

    if constexpr (EPI == kEpiGeluFp8) {
        if (p.q_out_t) {
            __syncthreads();   // every thread is done reading the fp32 tile
            uint8_t* ct = smem;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int id = t + kThreads * i;
                *reinterpret_cast<uint2*>(ct + (id >> 4) * kCodePitch + (id & 15) * 8) = codes[i];
            }
            __syncthreads();
            // thread t writes 8 chunks of 8 consecutive rows of one column:
            // id = t + 256 i, column = id / 16, rows 8 * (id % 16) .. +7
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int id = t + kThreads * i;
                const int col = id >> 4;
                const int r8 = (id & 15) * 8;
                const int64_t gn = n0 + col;
                const int64_t gm = m0 + r8;
                if (gn < N && gm < M) {
                    uint32_t w0 = 0, w1 = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        w0 |= (uint32_t)ct[(r8 + k) * kCodePitch + col] << (8 * k);
                        w1 |= (uint32_t)ct[(r8 + 4 + k) * kCodePitch + col] << (8 * k);
                    }
                    uint8_t* dst = p.q_out_t + gn * M + gm;
                    if (gm + 8 <= M) {
                        *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
                    } else {
                        for (int k = 0; gm + k < M; ++k)
                            dst[k] = (uint8_t)((k < 4 ? w0 : w1) >> (8 * (k & 3)));
                    }
                }
            }
        }
        __shared__ uint32_t red[kThreads / kWave];
        block_amax_atomic(amax_bits, p.q_amax, red);
    }
}

template <int FA, int FB, int EPI, int QF>
hipError_t launch_typed(const GemmParams& p, hipStream_t stream) {
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_kernel<FA, FB, EPI, QF>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_epi(const GemmParams& p, hipStream_t stream) {
    switch (p.epilogue) {
        case kEpiBf16Bias: return launch_typed<FA, FB, kEpiBf16Bias, kE4M3>(p, stream);
        case kEpiF32: return launch_typed<FA, FB, kEpiF32, kE4M3>(p, stream);
        case kEpiDGeluF32: return launch_typed<FA, FB, kEpiDGeluF32, kE4M3>(p, stream);
        case kEpiGeluFp8:
            return p.q_fp8 == kE4M3 ? launch_typed<FA, FB, kEpiGeluFp8, kE4M3>(p, stream)
                                    : launch_typed<FA, FB, kEpiGeluFp8, kE5M2>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (p.a_fp8 == kE4M3 && p.b_fp8 == kE4M3) return launch_epi<kE4M3, kE4M3>(p, stream);
    if (p.a_fp8 == kE5M2 && p.b_fp8 == kE4M3) return launch_epi<kE5M2, kE4M3>(p, stream);
    if (p.a_fp8 == kE4M3 && p.b_fp8 == kE5M2) return launch_epi<kE4M3, kE5M2>(p, stream);
    return launch_epi<kE5M2, kE5M2>(p, stream);
}

}  // namespace fp8ln
