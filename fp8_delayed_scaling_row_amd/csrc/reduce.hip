// Deterministic column sums of per-block partial results: the second stage of
// every two-stage reduction here (bias gradients from the cast kernels and the
// GEMM epilogue, dgamma / dbeta from the LayerNorm backward).  Each output is
// summed in one fixed order, so repeated runs give identical bits.
#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

namespace {

constexpr int kCols = 16;     // columns per workgroup
constexpr int kSlices = 16;   // row slices per column, summed in slice order

// out[j] = sum over r of partial[r][j]; thread (slice s, column c) sums rows
// s, s + 16, s + 32, ... with four interleaved accumulators, then the slices are
// added in order 0..15.  Columns below split go to out0, the rest to out1.
__global__ __launch_bounds__(kCols * kSlices) void sum_partials_kernel(
    const float* __restrict__ partial, int64_t nrows, int64_t width, float* __restrict__ out0,
    float* __restrict__ out1, int64_t split) {
    __shared__ float red[kSlices][kCols + 1];
    const int c = threadIdx.x % kCols;
    const int s = threadIdx.x / kCols;
    const int64_t j = (int64_t)blockIdx.x * kCols + c;
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (j < width) {
        int64_t r = s;
        for (; r + 3 * kSlices < nrows; r += 4 * kSlices) {
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] += partial[(r + u * kSlices) * width + j];
        }
        if (r < nrows) a[0] += partial[r * width + j];
        if (r + kSlices < nrows) a[1] += partial[(r + kSlices) * width + j];
        if (r + 2 * kSlices < nrows) a[2] += partial[(r + 2 * kSlices) * width + j];
    }
    red[s][c] = (a[0] + a[1]) + (a[2] + a[3]);
    __syncthreads();
    if (s == 0 && j < width) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < kSlices; ++k) acc += red[k][c];
        if (j < split) out0[j] = acc;
        else out1[j - split] = acc;
    }
}

}  // namespace

hipError_t launch_sum_partials(const float* partial, int64_t nrows, int64_t width, float* out0,
                               float* out1, int64_t split, hipStream_t stream) {
    if (width == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((width + kCols - 1) / kCols);
    hipLaunchKernelGGL(sum_partials_kernel, dim3(blocks), dim3(kCols * kSlices), 0, stream,
                       partial, nrows, width, out0, out1, split);
    return hipGetLastError();
}

}  // namespace fp8ln
