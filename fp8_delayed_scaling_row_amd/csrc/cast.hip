// FP8 cast kernels: tensor cast with amax, optional transposed copy and column
// sums (weights, output gradients, fc1 gradients), a byte transpose, and the
// encoder over a range of binary32 bit patterns.  The cast scales with a
// round-to-odd product, so its codes are those of the exact value * scale.
//
// Autocast casts the operands of the linear layers to FP8 with the delayed
// scale and hands gradients back in higher precision ("Turbo-charging your
// transformer training", "Playing with lower-precision formats: BF16 vs FP8";
// HYBRID: E4M3 forward, E5M2 gradients).  The transposed copy exists because the
// backward's GEMMs contract over the other index (dgrad over output features,
// wgrad over tokens) and the GEMM reads operands with the contraction index last.
#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;           // rows and columns of one tile
constexpr int kTPad = kTile + 16;   // byte pitch of the transposition tile

// One block casts a 64 x 64 tile; thread t owns row t/4, columns 16*(t%4) .. +15.
template <bool IN_F32, int FMT>
__global__ __launch_bounds__(kThreads) void cast_tile_kernel(
    const void* __restrict__ in, int64_t rows, int64_t cols, const float* __restrict__ scale_ptr,
    float* __restrict__ amax_ptr, uint8_t* __restrict__ out, uint8_t* __restrict__ out_t,
    float* __restrict__ partial) {
    __shared__ uint8_t tq[kTile][kTPad];
    __shared__ float tv[kTile][kTile + 1];
    __shared__ uint32_t red[kThreads / kWave];
    const int t = threadIdx.x;
    const int lr = t / 4;
    const int lc = (t % 4) * 16;
    const int64_t r = (int64_t)blockIdx.y * kTile + lr;
    const int64_t c0 = (int64_t)blockIdx.x * kTile + lc;
    const float s = *scale_ptr;
    const bool active = r < rows && c0 < cols;

    float v[16];
    if (active) {
        if constexpr (IN_F32) {
            const float4* p = reinterpret_cast<const float4*>((const float*)in + r * cols + c0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 w = p[i];
                v[4 * i + 0] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
            }
        } else {
            const uint4* p = reinterpret_cast<const uint4*>((const uint16_t*)in + r * cols + c0);
            unpack_bf16x8(p[0], v);
            unpack_bf16x8(p[1], v + 8);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }

    uint32_t cm = 0;
    float vs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t ab = abs_bits(v[i]);
        cm = cm > ab ? cm : ab;
        vs[i] = mul_round_odd(v[i], s);
    }
    uint4 q;
    q.x = encode4<FMT>(vs[0], vs[1], vs[2], vs[3]);
    q.y = encode4<FMT>(vs[4], vs[5], vs[6], vs[7]);
    q.z = encode4<FMT>(vs[8], vs[9], vs[10], vs[11]);
    q.w = encode4<FMT>(vs[12], vs[13], vs[14], vs[15]);
    if (__builtin_expect(cm > kInfBits, 0)) {
        q.x = patch_nan4(q.x, vs);
        q.y = patch_nan4(q.y, vs + 4);
        q.z = patch_nan4(q.z, vs + 8);
        q.w = patch_nan4(q.w, vs + 12);
    }
    if (active) *reinterpret_cast<uint4*>(out + r * cols + c0) = q;

    if (out_t) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) tq[lc + i][lr] = (uint8_t)(w[i / 4] >> (8 * (i % 4)));
    }
    if (partial) {
#pragma unroll
        for (int i = 0; i < 16; ++i) tv[lr][lc + i] = v[i];
    }
    __syncthreads();
    if (out_t) {
        // thread t writes column t/4 of the tile, rows 16*(t%4) .. +15 (rows % 16 == 0)
        const int64_t oc = (int64_t)blockIdx.x * kTile + lr;
        const int64_t orow0 = (int64_t)blockIdx.y * kTile + lc;
        if (oc < cols && orow0 < rows)
            *reinterpret_cast<uint4*>(out_t + oc * rows + orow0) =
                *reinterpret_cast<const uint4*>(&tq[lr][lc]);
    }
    if (partial && t < kTile) {
        const int64_t pc = (int64_t)blockIdx.x * kTile + t;
        if (pc < cols) {
            float acc = 0.0f;
            for (int i = 0; i < kTile; ++i) acc += tv[i][t];   // rows past the end are 0
            partial[(int64_t)blockIdx.y * cols + pc] = acc;
        }
    }
    block_amax_atomic(cm, amax_ptr, red);
}

// out[c] = sum over p of partial[p][c], in order of p.
__global__ __launch_bounds__(kThreads) void colsum_kernel(const float* __restrict__ partial,
                                                          int64_t np, int64_t cols,
                                                          float* __restrict__ out) {
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= cols) return;
    float acc = 0.0f;
    for (int64_t p = 0; p < np; ++p) acc += partial[p * cols + c];
    out[c] = acc;
}

// in [rows][cols] -> out [cols][rows], 64 x 64 byte tiles (cols % 16 == 0,
// rows % 16 == 0).
__global__ __launch_bounds__(kThreads) void transpose_u8_kernel(const uint8_t* __restrict__ in,
                                                                int64_t rows, int64_t cols,
                                                                uint8_t* __restrict__ out) {
    __shared__ uint8_t tile[kTile][kTPad];
    const int t = threadIdx.x;
    const int lr = t / 4;
    const int lc = (t % 4) * 16;
    const int64_t r = (int64_t)blockIdx.y * kTile + lr;
    const int64_t c0 = (int64_t)blockIdx.x * kTile + lc;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (r < rows && c0 < cols) w = *reinterpret_cast<const uint4*>(in + r * cols + c0);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[lc + i][lr] = (uint8_t)(ws[i / 4] >> (8 * (i % 4)));
    __syncthreads();
    const int64_t oc = (int64_t)blockIdx.x * kTile + lr;
    const int64_t orow0 = (int64_t)blockIdx.y * kTile + lc;
    if (oc < cols && orow0 < rows)
        *reinterpret_cast<uint4*>(out + oc * rows + orow0) =
            *reinterpret_cast<const uint4*>(&tile[lr][lc]);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void encode_range_kernel(uint32_t start, int64_t count,
                                                                uint8_t* __restrict__ out) {
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (i0 >= count) return;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(start + (uint32_t)(i0 + k));
    uint32_t q = encode4<FMT>(v[0], v[1], v[2], v[3]);
    q = patch_nan4(q, v);
    if (i0 + 4 <= count) {
        *reinterpret_cast<uint32_t*>(out + i0) = q;
    } else {
        for (int k = 0; i0 + k < count; ++k) out[i0 + k] = (uint8_t)(q >> (8 * k));
    }
}

template <bool IN_F32>
hipError_t launch_cast_fmt(int64_t rows, int64_t cols, const void* in, int fp8,
                           const float* scale, float* amax, uint8_t* out, uint8_t* out_t,
                           float* partial, hipStream_t stream) {
    const dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
    if (fp8 == kE4M3)
        hipLaunchKernelGGL((cast_tile_kernel<IN_F32, kE4M3>), grid, dim3(kThreads), 0, stream, in,
                           rows, cols, scale, amax, out, out_t, partial);
    else
        hipLaunchKernelGGL((cast_tile_kernel<IN_F32, kE5M2>), grid, dim3(kThreads), 0, stream, in,
                           rows, cols, scale, amax, out, out_t, partial);
    return hipGetLastError();
}

}  // namespace

size_t cast_workspace(int64_t rows, int64_t cols) {
    return (size_t)((rows + kTile - 1) / kTile) * (size_t)cols * sizeof(float);
}

hipError_t launch_cast_amax(int64_t rows, int64_t cols, bool in_f32, const void* in, int fp8,
                            const float* scale, float* amax, uint8_t* out, uint8_t* out_t,
                            float* colsum, void* workspace, hipStream_t stream) {
    if (cols == 0) return hipSuccess;
    float* partial = colsum ? (float*)workspace : nullptr;
    if (rows > 0) {
        hipError_t e = in_f32 ? launch_cast_fmt<true>(rows, cols, in, fp8, scale, amax, out,
                                                      out_t, partial, stream)
                              : launch_cast_fmt<false>(rows, cols, in, fp8, scale, amax, out,
                                                       out_t, partial, stream);
        if (e != hipSuccess) return e;
    }
    if (!colsum) return hipSuccess;
    const int64_t np = (rows + kTile - 1) / kTile;
    hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((cols + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, partial, np, cols, colsum);
    return hipGetLastError();
}

hipError_t launch_transpose_u8(int64_t rows, int64_t cols, const uint8_t* in, uint8_t* out,
                               hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
    hipLaunchKernelGGL(transpose_u8_kernel, grid, dim3(kThreads), 0, stream, in, rows, cols, out);
    return hipGetLastError();
}

hipError_t launch_encode_range(uint32_t start, int64_t count, int fp8, uint8_t* out,
                               hipStream_t stream) {
    if (count == 0) return hipSuccess;
    const int64_t threads = (count + 3) / 4;
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    if (fp8 == kE4M3)
        hipLaunchKernelGGL(encode_range_kernel<kE4M3>, dim3(blocks), dim3(kThreads), 0, stream,
                           start, count, out);
    else
        hipLaunchKernelGGL(encode_range_kernel<kE5M2>, dim3(blocks), dim3(kThreads), 0, stream,
                           start, count, out);
    return hipGetLastError();
}

}  // namespace fp8ln
