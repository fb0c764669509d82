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
#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;           // rows and columns of one transposition tile
constexpr int kTPad = kTile + 16;   // byte pitch of the transposition tile
constexpr int kCT = 128;            // rows and columns of one cast tile
constexpr int kCPitch = kCT + 4;    // byte pitch of the cast kernel's transposed codes

// A workgroup casts 128 x 128 tiles, looping over them with the grid sized to
// what the CUs hold at once; the next tile's loads go out before the current
// tile is processed, so every workgroup keeps a tile's reads in flight.  Thread
// t owns columns 8 (t % 16) .. +7 of rows 4 (t / 16) .. +3 and 64 + 4 (t / 16)
// .. +3 of a tile, so each row is read and written by 16 consecutive lanes as
// one contiguous segment.  For the transposed copy a thread packs the codes of
// its four consecutive rows of one column into a word in LDS; the tile then
// leaves as full 128-byte rows of the transposed output.  Column sums of a tile
// (for the bias gradient) are formed in a fixed order: a thread's eight rows,
// then the sixteen threads of a column in order of t / 16.
template <bool IN_F32, int FMT>
__global__ __launch_bounds__(kThreads) void cast_tile_kernel(
    const void* __restrict__ in, int64_t rows, int64_t cols, const float* __restrict__ scale_ptr,
    float* __restrict__ amax_ptr, uint8_t* __restrict__ out, uint8_t* __restrict__ out_t,
    float* __restrict__ partial, const float* __restrict__ copy_src, float* __restrict__ copy_dst) {
    __shared__ uint32_t tq[kCT * kCPitch / 4];
    if (copy_dst && blockIdx.x == 0 && threadIdx.x == 0) *copy_dst = *copy_src;
    __shared__ float psum[kThreads / 16][kCT];
    __shared__ uint32_t red[kThreads / kWave];
    const int t = threadIdx.x;
    const int j = t % 16;
    const int p = t / 16;
    const int tiles_x = (int)((cols + kCT - 1) / kCT);
    const int tiles = tiles_x * (int)((rows + kCT - 1) / kCT);
    const float s = *scale_ptr;

    typedef typename std::conditional<IN_F32, float4, uint4>::type Raw;
    constexpr int RPR = IN_F32 ? 2 : 1;   // 16-byte loads per row segment of 8 values
    Raw raw[8][RPR];
    // the thread's eight row segments of tile `tile` (zeros outside the tensor)
    auto load_tile = [&](int tile) {
        const int64_t r0 = (int64_t)(tile / tiles_x) * kCT;
        const int64_t c0 = (int64_t)(tile % tiles_x) * kCT + 8 * j;
        const bool col_ok = tile < tiles && c0 < cols;   // cols % 16 == 0: all in or all out
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int64_t r = r0 + 64 * (h / 4) + 4 * p + (h % 4);
            const bool ok = col_ok && r < rows;
#pragma unroll
            for (int k = 0; k < RPR; ++k) {
                if constexpr (IN_F32) {
                    const float4* q =
                        reinterpret_cast<const float4*>((const float*)in + r * cols + c0);
                    raw[h][k] = ok ? load_nt(q + k) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                } else {
                    const uint4* q =
                        reinterpret_cast<const uint4*>((const uint16_t*)in + r * cols + c0);
                    raw[h][k] = ok ? load_nt(q) : make_uint4(0, 0, 0, 0);
                }
            }
        }
    };

    uint32_t cm = 0;
    load_tile(blockIdx.x);
    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int64_t r0 = (int64_t)(tile / tiles_x) * kCT;
        const int64_t c0 = (int64_t)(tile % tiles_x) * kCT + 8 * j;
        const bool col_ok = c0 < cols;
        Raw cur[8][RPR];
#pragma unroll
        for (int h = 0; h < 8; ++h)
#pragma unroll
            for (int k = 0; k < RPR; ++k) cur[h][k] = raw[h][k];
        load_tile(tile + gridDim.x);   // in flight while this tile is processed

        float cs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint32_t packed[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) packed[e] = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = r0 + 64 * half + 4 * p + i;
                const bool ok = col_ok && r < rows;
                const Raw* w = cur[4 * half + i];
                float v[8];
                if constexpr (IN_F32) {
                    v[0] = w[0].x; v[1] = w[0].y; v[2] = w[0].z; v[3] = w[0].w;
                    v[4] = w[1].x; v[5] = w[1].y; v[6] = w[1].z; v[7] = w[1].w;
                } else {
                    unpack_bf16x8(w[0], v);
                }
                float vs[8];
                uint32_t rm = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t ab = abs_bits(v[e]);
                    rm = rm > ab ? rm : ab;
                    vs[e] = mul_round_odd(v[e], s);
                    cs[e] += v[e];
                }
                uint32_t lo = encode4<FMT>(vs[0], vs[1], vs[2], vs[3]);
                uint32_t hi = encode4<FMT>(vs[4], vs[5], vs[6], vs[7]);
                if (__builtin_expect(rm > kInfBits, 0)) {
                    lo = patch_nan4(lo, vs);
                    hi = patch_nan4(hi, vs + 4);
                }
                cm = cm > rm ? cm : rm;
                if (ok) store_nt(reinterpret_cast<uint2*>(out + r * cols + c0), make_uint2(lo, hi));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    packed[e] |= ((lo >> (8 * e)) & 0xFFu) << (8 * i);
                    packed[4 + e] |= ((hi >> (8 * e)) & 0xFFu) << (8 * i);
                }
            }
            if (out_t) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    tq[(8 * j + e) * (kCPitch / 4) + 16 * half + p] = packed[e];
            }
        }
        if (partial) {
#pragma unroll
            for (int e = 0; e < 8; ++e) psum[p][8 * j + e] = cs[e];
        }
        __syncthreads();
        if (out_t) {
            // eight lanes per column write one 128-byte row of the transposed tile
            const int seg = t % 8;
            const int64_t orow = r0 + 16 * seg;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int cc = t / 8 + 32 * k;
                const int64_t oc = (int64_t)(tile % tiles_x) * kCT + cc;
                const uint32_t* src = tq + cc * (kCPitch / 4) + 4 * seg;
                if (oc < cols && orow < rows)
                    store_nt(reinterpret_cast<uint4*>(out_t + oc * rows + orow),
                             make_uint4(src[0], src[1], src[2], src[3]));
            }
        }
        if (partial && t < kCT) {
            const int64_t pc = (int64_t)(tile % tiles_x) * kCT + t;
            if (pc < cols) {
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < kThreads / 16; ++k) acc += psum[k][t];
                partial[(int64_t)(tile / tiles_x) * cols + pc] = acc;
            }
        }
        __syncthreads();   // tq and psum are rewritten by the next tile
    }
    block_amax_atomic(cm, amax_ptr, red);
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
    if (r < rows && c0 < cols) w = load_nt(reinterpret_cast<const uint4*>(in + r * cols + c0));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[lc + i][lr] = (uint8_t)(ws[i / 4] >> (8 * (i % 4)));
    __syncthreads();
    const int64_t oc = (int64_t)blockIdx.x * kTile + lr;
    const int64_t orow0 = (int64_t)blockIdx.y * kTile + lc;
    if (oc < cols && orow0 < rows)
        store_nt(reinterpret_cast<uint4*>(out + oc * rows + orow0),
                 *reinterpret_cast<const uint4*>(&tile[lr][lc]));
}

// in [rows][cols] -> out [cols][rows] for 16-bit elements (bf16), 64 x 64 tiles
// (rows % 8 == 0, cols % 8 == 0).  With partial set, row tile y also writes the
// fp32 column sums of its 64 rows to partial[y][cols], summed in row order.
__global__ __launch_bounds__(kThreads) void transpose_b16_kernel(const uint16_t* __restrict__ in,
                                                                 int64_t rows, int64_t cols,
                                                                 uint16_t* __restrict__ out,
                                                                 float* __restrict__ partial) {
    __shared__ uint16_t tile[kTile][kTile + 2];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * kTile;
    const int64_t c0 = (int64_t)blockIdx.x * kTile;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int u = t + h * kThreads;        // 64 rows x 8 chunks of 8 elements
        const int lr = u / 8, lc = (u % 8) * 8;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (r0 + lr < rows && c0 + lc < cols)
            w = load_nt(reinterpret_cast<const uint4*>(in + (r0 + lr) * cols + c0 + lc));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) tile[lr][lc + i] = (uint16_t)(ws[i / 2] >> (16 * (i % 2)));
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int u = t + h * kThreads;        // 64 output rows x 8 chunks
        const int oc = u / 8, orr = (u % 8) * 8;
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = (uint32_t)tile[orr + 2 * i][oc] | ((uint32_t)tile[orr + 2 * i + 1][oc] << 16);
        if (c0 + oc < cols && r0 + orr < rows)
            store_nt(reinterpret_cast<uint4*>(out + (c0 + oc) * rows + r0 + orr),
                     make_uint4(v[0], v[1], v[2], v[3]));
    }
    if (partial && t < kTile && c0 + t < cols) {
        float a = 0.0f;
        for (int r = 0; r < kTile; ++r) a += __uint_as_float((uint32_t)tile[r][t] << 16);
        partial[(int64_t)blockIdx.y * cols + c0 + t] = a;
    }
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

// Workgroups the CUs hold at once for kernel k (queried once per kernel).
template <class Kernel>
hipError_t resident_blocks(Kernel k, int& cache) {
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

template <bool IN_F32, int FMT>
hipError_t launch_cast_typed(int64_t rows, int64_t cols, const void* in, const float* scale,
                             float* amax, uint8_t* out, uint8_t* out_t, float* partial,
                             const float* copy_src, float* copy_dst, hipStream_t stream) {
    static int resident = 0;
    hipError_t e = resident_blocks(cast_tile_kernel<IN_F32, FMT>, resident);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((cols + kCT - 1) / kCT) * ((rows + kCT - 1) / kCT);
    const unsigned blocks = (unsigned)(tiles < resident ? tiles : resident);
    hipLaunchKernelGGL((cast_tile_kernel<IN_F32, FMT>), dim3(blocks), dim3(kThreads), 0, stream,
                       in, rows, cols, scale, amax, out, out_t, partial, copy_src, copy_dst);
    return hipGetLastError();
}

template <bool IN_F32>
hipError_t launch_cast_fmt(int64_t rows, int64_t cols, const void* in, int fp8,
                           const float* scale, float* amax, uint8_t* out, uint8_t* out_t,
                           float* partial, const float* copy_src, float* copy_dst,
                           hipStream_t stream) {
    if (fp8 == kE4M3)
        return launch_cast_typed<IN_F32, kE4M3>(rows, cols, in, scale, amax, out, out_t, partial,
                                                copy_src, copy_dst, stream);
    return launch_cast_typed<IN_F32, kE5M2>(rows, cols, in, scale, amax, out, out_t, partial,
                                            copy_src, copy_dst, stream);
}

}  // namespace

size_t cast_workspace(int64_t rows, int64_t cols) {
    return (size_t)((rows + kCT - 1) / kCT) * (size_t)cols * sizeof(float);
}

hipError_t launch_cast_amax(int64_t rows, int64_t cols, bool in_f32, const void* in, int fp8,
                            const float* scale, float* amax, uint8_t* out, uint8_t* out_t,
                            float* colsum, void* workspace, hipStream_t stream,
                            const float* copy_src, float* copy_dst) {
    if (cols == 0) return hipSuccess;
    float* partial = colsum ? (float*)workspace : nullptr;
    if (rows > 0) {
        hipError_t e = in_f32 ? launch_cast_fmt<true>(rows, cols, in, fp8, scale, amax, out,
                                                      out_t, partial, copy_src, copy_dst, stream)
                              : launch_cast_fmt<false>(rows, cols, in, fp8, scale, amax, out,
                                                       out_t, partial, copy_src, copy_dst, stream);
        if (e != hipSuccess) return e;
    }
    if (!colsum) return hipSuccess;
    return launch_sum_partials(partial, (rows + kCT - 1) / kCT, cols, colsum, nullptr, cols,
                               stream);
}

hipError_t launch_transpose_u8(int64_t rows, int64_t cols, const uint8_t* in, uint8_t* out,
                               hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)((rows + kTile - 1) / kTile));
    hipLaunchKernelGGL(transpose_u8_kernel, grid, dim3(kThreads), 0, stream, in, rows, cols, out);
    return hipGetLastError();
}

size_t transpose_b16_workspace(int64_t rows, int64_t cols) {
    return (size_t)((rows + kTile - 1) / kTile) * (size_t)cols * sizeof(float);
}

hipError_t launch_transpose_b16(int64_t rows, int64_t cols, const void* in, void* out,
                                float* colsum, void* workspace, hipStream_t stream) {
    if (cols == 0) return hipSuccess;
    float* partial = colsum ? (float*)workspace : nullptr;
    if (rows > 0) {
        const dim3 grid((unsigned)((cols + kTile - 1) / kTile),
                        (unsigned)((rows + kTile - 1) / kTile));
        hipLaunchKernelGGL(transpose_b16_kernel, grid, dim3(kThreads), 0, stream,
                           (const uint16_t*)in, rows, cols, (uint16_t*)out, partial);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!colsum) return hipSuccess;
    return launch_sum_partials(partial, (rows + kTile - 1) / kTile, cols, colsum, nullptr, cols,
                               stream);
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
