// Deterministic column sums of per-block partial results: the second stage of
// every two-stage reduction here (bias gradients from the cast kernels and the
// GEMM epilogue, dgamma / dbeta from the LayerNorm backward).  Each output is
// summed in one fixed order, so repeated runs give identical bits, and a
// backward gathers its sums into one launch (SumBatch) with the same per-column
// order as separate launches.
#include "device_common.hpp"
#include "launchers.hpp"
#include "step_update.hpp"

namespace fp8ln {

namespace {

constexpr int kCols = 16;     // columns per workgroup
constexpr int kSlices = 16;   // row slices per column, summed in slice order

// out[j] = sum over r of partial[r][j] for the kCols columns of workgroup
// `block`; thread (slice s, column c) sums rows s, s + 16, s + 32, ... with four
// interleaved accumulators, then the slices are added in order 0..15.  Columns
// below split go to out0, the rest to out1.  All threads call it.
__device__ __forceinline__ void sum_columns(const SumJob& q, int64_t block) {
    __shared__ float red[kSlices][kCols + 1];
    const int c = threadIdx.x % kCols;
    const int s = threadIdx.x / kCols;
    const int64_t j = block * kCols + c;
    const float* __restrict__ partial = q.partial;
    const int64_t nrows = q.nrows, width = q.width;
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
        if (j < q.split) q.out0[j] = acc;
        else q.out1[j - q.split] = acc;
    }
}

__global__ __launch_bounds__(kCols * kSlices) void sum_partials_kernel(SumJob q) {
    sum_columns(q, blockIdx.x);
}

struct SumLaunch {
    SumJob job[kMaxSumJobs];
    int64_t start[kMaxSumJobs + 1];   // first workgroup of each job
    int n;
    float* roll_hist;
    uint32_t* roll_ws;
    int roll_len, roll_slots;
};

// Workgroups [start[k], start[k + 1]) sum job k; workgroup 0 also rolls the
// history of a folded scaling update when one is given (after its own sums).
__global__ __launch_bounds__(kCols * kSlices) void sum_batch_kernel(SumLaunch b) {
    const int64_t w = blockIdx.x;
    for (int k = 0; k < b.n; ++k)   // workgroup-uniform choice of the job
        if (w >= b.start[k] && w < b.start[k + 1]) sum_columns(b.job[k], w - b.start[k]);
    if (b.roll_hist && w == 0) {
        __syncthreads();
        roll_history(b.roll_hist, b.roll_ws, b.roll_len, b.roll_slots);
    }
}

int64_t col_blocks(int64_t width) { return (width + kCols - 1) / kCols; }

}  // namespace

hipError_t launch_sum_partials(const float* partial, int64_t nrows, int64_t width, float* out0,
                               float* out1, int64_t split, hipStream_t stream) {
    if (width == 0) return hipSuccess;
    hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)col_blocks(width)),
                       dim3(kCols * kSlices), 0, stream,
                       SumJob{partial, nrows, width, out0, out1, split});
    return hipGetLastError();
}

bool SumBatch::add(const float* partial, int64_t nrows, int64_t width, float* out0, float* out1,
                   int64_t split) {
    if (width == 0) return true;
    if (n >= kMaxSumJobs) return false;
    job[n++] = SumJob{partial, nrows, width, out0, out1, split};
    return true;
}

hipError_t launch_sum_batch(const SumBatch& b, hipStream_t stream) {
    SumLaunch l{};
    l.n = b.n;
    l.start[0] = 0;
    for (int k = 0; k < b.n; ++k) {
        l.job[k] = b.job[k];
        l.start[k + 1] = l.start[k] + col_blocks(b.job[k].width);
    }
    l.roll_hist = b.roll_hist;
    l.roll_ws = b.roll_ws;
    l.roll_len = b.roll_len;
    l.roll_slots = b.roll_slots;
    int64_t blocks = l.start[b.n];
    if (blocks == 0 && b.roll_hist) blocks = 1;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(sum_batch_kernel, dim3((unsigned)blocks), dim3(kCols * kSlices), 0, stream,
                       l);
    return hipGetLastError();
}

}  // namespace fp8ln
