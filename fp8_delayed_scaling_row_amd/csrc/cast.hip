// FP8 cast kernels: tensor cast with amax, optional transposed copy and column
// sums (weights, output gradients, fc1 gradients; the per-tile work lives in
// cast_body.hpp), a byte transpose, and the encoder over a range of binary32 bit
// patterns.
//
// Autocast casts the operands of the linear layers to FP8 with the delayed
// scale and hands gradients back in higher precision ("Turbo-charging your
// transformer training", "Playing with lower-precision formats: BF16 vs FP8";
// HYBRID: E4M3 forward, E5M2 gradients).  The transposed copy exists because the
// backward's GEMMs contract over the other index (dgrad over output features,
// wgrad over tokens) and the GEMM reads operands with the contraction index last.
#include <type_traits>

#include "cast_body.hpp"
#include "device_common.hpp"
#include "launchers.hpp"
#include "step_update.hpp"

namespace fp8ln {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;           // rows and columns of one bf16 transposition tile

template <bool IN_F32, int FMT, int NT>
__global__ __launch_bounds__(NT) void cast_tile_kernel(
    const void* __restrict__ in, int64_t rows, int64_t cols, const float* __restrict__ scale_ptr,
    float* __restrict__ amax_ptr, uint8_t* __restrict__ out, uint8_t* __restrict__ out_t,
    float* __restrict__ partial, const float* __restrict__ copy_src, float* __restrict__ copy_dst) {
    cast_tiles<IN_F32, FMT, NT>(in, rows, cols, scale_ptr, amax_ptr, out, out_t, partial, copy_src,
                                copy_dst, blockIdx.x, gridDim.x);
}

// The cast with the step's scaling update folded in (bf16 input): every
// workgroup forms the scales from the history window while its first tile is in
// flight, casts with slot u.cast_slot[0]'s and records its amax into u.ws; the
// history is rolled by a later launch of the step.
template <int FMT, int NT>
__global__ __launch_bounds__(NT) void cast_tile_step_kernel(
    const void* __restrict__ in, int64_t rows, int64_t cols, FusedUpdate u,
    uint8_t* __restrict__ out, uint8_t* __restrict__ out_t, float* __restrict__ partial) {
    __shared__ float sh[2 * kMaxMetaSlots];
    const int q = u.cast_slot[0];
    cast_tiles<false, FMT, NT, true>(in, rows, cols, sh + 2 * q,
                                     reinterpret_cast<float*>(u.ws + q), out, out_t, partial,
                                     nullptr, nullptr, blockIdx.x, gridDim.x,
                                     [&]() { window_scales<NT>(u, sh); });
}

// in [rows][cols] -> out [cols][rows] (rows % 16 == 0, cols % 16 == 0), over
// kTR x kTC byte tiles on a resident grid, the next tile's loads in flight while
// the current one is transposed; reads are kTC-byte row segments and writes
// kTR-byte row segments of the output.  Thread t owns the 4 x 4 byte blocks at
// columns 4 (t % (kTC / 4)) .. +3 and rows 4 (t / (kTC / 4)) + kRP p .. +3 of a
// tile: it loads one word of each of those rows (kTC / 4 lanes read kTC
// contiguous bytes of a row), transposes each block in registers with byte
// selects and writes one word per column (four rows) into LDS; then each thread
// reads 16-byte pieces of output rows (columns of the tile) and stores them.
constexpr int kTR = 128;                    // tile rows (bytes of an output row segment)
constexpr int kTC = 128;                    // tile columns (bytes of an input row segment)
constexpr int kTB = kTC / 4;                // threads across a tile row
constexpr int kRP = 4 * (256 / kTB);        // rows covered by one pass of the workgroup
constexpr int kTPass = kTR / kRP;           // passes per tile
constexpr int kTW = kTR / 4 + 1;            // words per LDS row of the transposed tile
constexpr int kTChunks = kTC * (kTR / 16) / 256;   // 16-byte output pieces per thread

__device__ __forceinline__ void transpose4x4_u8(const uint32_t w[4], uint32_t col[4]) {
    // perm(hi, lo, s): byte i of the result is byte s_i of {hi:lo} (lo = bytes 0-3)
    const uint32_t t01l = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
    const uint32_t t01h = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
    const uint32_t t23l = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t t23h = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    col[0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
    col[1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
    col[2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
    col[3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
}

__global__ __launch_bounds__(kThreads) void transpose_u8_kernel(const uint8_t* __restrict__ in,
                                                                int64_t rows, int64_t cols,
                                                                uint8_t* __restrict__ out) {
    static_assert(kThreads == 256, "thread layout");
    __shared__ uint32_t tw[kTC][kTW];
    const int t = threadIdx.x;
    const int a = t / kTB, b = t % kTB;
    const int64_t tiles_x = (cols + kTC - 1) / kTC;
    const int64_t tiles = tiles_x * ((rows + kTR - 1) / kTR);
    uint32_t w[kTPass][4];
    auto load = [&](int64_t tile) {
        const int64_t r0 = (tile / tiles_x) * kTR + 4 * a;
        const int64_t c = (tile % tiles_x) * kTC + 4 * b;
#pragma unroll
        for (int p = 0; p < kTPass; ++p) {
            const int64_t r = r0 + kRP * p;
            const bool ok = tile < tiles && r < rows && c < cols;   // 4-row, 4-column groups are whole
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[p][k] = ok ? __builtin_nontemporal_load(
                                   reinterpret_cast<const uint32_t*>(in + (r + k) * cols + c))
                             : 0u;
        }
    };
    load(blockIdx.x);
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        uint32_t col[kTPass][4];
#pragma unroll
        for (int p = 0; p < kTPass; ++p) transpose4x4_u8(w[p], col[p]);
        load(tile + gridDim.x);   // in flight while this tile goes through LDS
#pragma unroll
        for (int p = 0; p < kTPass; ++p)
#pragma unroll
            for (int k = 0; k < 4; ++k) tw[4 * b + k][kRP / 4 * p + a] = col[p][k];
        __syncthreads();
        const int64_t c0 = (tile % tiles_x) * kTC, r0 = (tile / tiles_x) * kTR;
#pragma unroll
        for (int q = 0; q < kTChunks; ++q) {
            const int u = t + q * kThreads;      // piece u: column u / (kTR / 16), rows 16 (u % ..)
            const int oc = u / (kTR / 16), om = u % (kTR / 16);
            uint4 v;
            v.x = tw[oc][4 * om];
            v.y = tw[oc][4 * om + 1];
            v.z = tw[oc][4 * om + 2];
            v.w = tw[oc][4 * om + 3];
            const int64_t gc = c0 + oc, gr = r0 + 16 * om;
            if (gc < cols && gr < rows) store_nt(reinterpret_cast<uint4*>(out + gc * rows + gr), v);
        }
        __syncthreads();   // the tile's LDS is free for the next
    }
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

// Workgroups of nt threads the CUs hold at once for kernel k (queried once per
// kernel), and the CU count.
template <class Kernel>
hipError_t resident_blocks(Kernel k, int nt, int& cache, int* cu_count = nullptr) {
    static int cus = 0;
    if (cache > 0 && cus > 0) {
        if (cu_count) *cu_count = cus;
        return hipSuccess;
    }
    int nb = 0, dev = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, nt, 0);
    if (e != hipSuccess) return e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
        hipSuccess)
        return e;
    cache = (nb > 0 ? nb : 1) * cus;
    if (cu_count) *cu_count = cus;
    return hipSuccess;
}

template <bool IN_F32, int FMT>
hipError_t launch_cast_typed(int64_t rows, int64_t cols, const void* in, const float* scale,
                             float* amax, uint8_t* out, uint8_t* out_t, float* partial,
                             const float* copy_src, float* copy_dst, hipStream_t stream) {
    static int resident = 0, resident_wide = 0;
    int cus = 0;
    hipError_t e = resident_blocks(cast_tile_kernel<IN_F32, FMT, 256>, 256, resident, &cus);
    if (e != hipSuccess) return e;
    e = resident_blocks(cast_tile_kernel<IN_F32, FMT, 512>, 512, resident_wide);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((cols + kCT - 1) / kCT) * ((rows + kCT - 1) / kCT);
    if (tiles <= 2 * (int64_t)cus) {
        // few tiles: each one's latency is the kernel's, so twice the threads per tile
        const unsigned blocks = (unsigned)(tiles < resident_wide ? tiles : resident_wide);
        hipLaunchKernelGGL((cast_tile_kernel<IN_F32, FMT, 512>), dim3(blocks), dim3(512), 0,
                           stream, in, rows, cols, scale, amax, out, out_t, partial, copy_src,
                           copy_dst);
    } else {
        const unsigned blocks = (unsigned)(tiles < resident ? tiles : resident);
        hipLaunchKernelGGL((cast_tile_kernel<IN_F32, FMT, 256>), dim3(blocks), dim3(256), 0,
                           stream, in, rows, cols, scale, amax, out, out_t, partial, copy_src,
                           copy_dst);
    }
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_cast_step_typed(int64_t rows, int64_t cols, const void* in,
                                  const FusedUpdate& u, uint8_t* out, uint8_t* out_t,
                                  float* partial, hipStream_t stream) {
    static int resident = 0, resident_wide = 0;
    int cus = 0;
    hipError_t e = resident_blocks(cast_tile_step_kernel<FMT, 256>, 256, resident, &cus);
    if (e != hipSuccess) return e;
    e = resident_blocks(cast_tile_step_kernel<FMT, 512>, 512, resident_wide);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((cols + kCT - 1) / kCT) * ((rows + kCT - 1) / kCT);
    if (tiles <= 2 * (int64_t)cus) {   // as launch_cast_typed
        const unsigned blocks = (unsigned)(tiles < resident_wide ? tiles : resident_wide);
        hipLaunchKernelGGL((cast_tile_step_kernel<FMT, 512>), dim3(blocks), dim3(512), 0, stream,
                           in, rows, cols, u, out, out_t, partial);
    } else {
        const unsigned blocks = (unsigned)(tiles < resident ? tiles : resident);
        hipLaunchKernelGGL((cast_tile_step_kernel<FMT, 256>), dim3(blocks), dim3(256), 0, stream,
                           in, rows, cols, u, out, out_t, partial);
    }
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

namespace {

// The second stage of the column sums: added to `sums` when given, else launched.
hipError_t cast_colsums(const float* partial, int64_t rows, int64_t cols, float* colsum,
                        SumBatch* sums, hipStream_t stream) {
    const int64_t nrows = (rows + kCT - 1) / kCT;
    if (sums && sums->add(partial, nrows, cols, colsum, nullptr, cols)) return hipSuccess;
    return launch_sum_partials(partial, nrows, cols, colsum, nullptr, cols, stream);
}

}  // namespace

hipError_t launch_cast_amax(int64_t rows, int64_t cols, bool in_f32, const void* in, int fp8,
                            const float* scale, float* amax, uint8_t* out, uint8_t* out_t,
                            float* colsum, void* workspace, hipStream_t stream,
                            const float* copy_src, float* copy_dst, SumBatch* sums) {
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
    return cast_colsums(partial, rows, cols, colsum, sums, stream);
}

hipError_t launch_cast_amax_step(int64_t rows, int64_t cols, const void* in, int fp8,
                                 const FusedUpdate& u, uint8_t* out, uint8_t* out_t,
                                 float* colsum, void* workspace, SumBatch* sums,
                                 hipStream_t stream) {
    const int n = u.n_slots, q = u.cast_slot[0];
    if (rows <= 0 || cols <= 0 || u.len < 1 || u.len > 1024 || n < 1 || n > kMaxMetaSlots ||
        (n & (n - 1)) || q < 0 || q >= n)
        return hipErrorInvalidValue;
    float* partial = colsum ? (float*)workspace : nullptr;
    hipError_t e = fp8 == kE4M3
        ? launch_cast_step_typed<kE4M3>(rows, cols, in, u, out, out_t, partial, stream)
        : launch_cast_step_typed<kE5M2>(rows, cols, in, u, out, out_t, partial, stream);
    if (e != hipSuccess || !colsum) return e;
    return cast_colsums(partial, rows, cols, colsum, sums, stream);
}

hipError_t launch_transpose_u8(int64_t rows, int64_t cols, const uint8_t* in, uint8_t* out,
                               hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    static int resident = 0;
    hipError_t e = resident_blocks(transpose_u8_kernel, kThreads, resident);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((cols + kTC - 1) / kTC) * ((rows + kTR - 1) / kTR);
    const unsigned blocks = (unsigned)(tiles < resident ? tiles : resident);
    hipLaunchKernelGGL(transpose_u8_kernel, dim3(blocks), dim3(kThreads), 0, stream, in, rows,
                       cols, out);
    return hipGetLastError();
}

size_t transpose_b16_workspace(int64_t rows, int64_t cols) {
    return (size_t)((rows + kTile - 1) / kTile) * (size_t)cols * sizeof(float);
}

hipError_t launch_transpose_b16(int64_t rows, int64_t cols, const void* in, void* out,
                                float* colsum, void* workspace, hipStream_t stream) {
    if (cols == 0) return hipSuccess;
    float* partial = colsum ? (float*)workspace : nullptr;
    if ((rows + kTile - 1) / kTile > 65535) return hipErrorInvalidValue;   // grid y limit
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
