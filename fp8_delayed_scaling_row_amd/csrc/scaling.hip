// Delayed-scaling bookkeeping on the device: state initialisation and the
// step-start scale update with history roll.
//
// The recipe keeps a per-tensor scale and a 2-D amax history with the newest
// amaxes in row 0, reduced with "max" over 16 or 1024 steps (tutorial
// "Accelerating Transformer Training with NVIDIA Transformer Engine ...", setup
// and benchmark listings); "Turbo-charging your transformer training", "Playing
// with lower-precision formats", says the scale follows each tensor's amax.
// The update computes scale = fp8_max / max(history) / 2^margin as one binary32
// division plus an exact power-of-two step, keeps the old scale when the
// window's max is zero or not finite or the result is not a finite positive
// number, sets scale_inv = 1 / scale, then moves every row down by one and clears
// row 0.  All of it stays on the device: no value returns to the host.
#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxHist = 1024;
constexpr int kMaxSlots = 8;
constexpr int kPerThread = kMaxHist * kMaxSlots / kThreads;   // history values per thread

__global__ __launch_bounds__(kThreads) void meta_init_kernel(float* hist, float* scale,
                                                            float* scale_inv, int total,
                                                            int n_slots) {
    for (int i = threadIdx.x + blockIdx.x * blockDim.x; i < total; i += blockDim.x * gridDim.x)
        hist[i] = 0.0f;
    if (blockIdx.x == 0 && threadIdx.x < n_slots) {
        scale[threadIdx.x] = 1.0f;
        scale_inv[threadIdx.x] = 1.0f;
    }
}

// One workgroup updates every slot of one state block in a single pass over the
// history: every thread loads its share once into registers, the per-slot max
// comes from those registers, and the shifted rows are written back from them.
// Element j = tid + 256 t of the flattened [len][n_slots] history belongs to
// slot j % n_slots; when n_slots divides 256 (1, 2, 4, 8 slots) that slot is the
// same for all of a thread's elements and one running max suffices.
__device__ __forceinline__ void scaling_update_block(float* hist, float* scale, float* scale_inv,
                                                     int len, int n_slots, int margin,
                                                     float fp8_max) {
    __shared__ float red_max[kThreads / kWave][kMaxSlots];
    __shared__ int red_nan[kThreads / kWave][kMaxSlots];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int total = len * n_slots;

    float keep[kPerThread];
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) {
        const int j = tid + t * kThreads;
        keep[t] = j < total ? hist[j] : 0.0f;
    }
    float m[kMaxSlots];
    int nan[kMaxSlots];
#pragma unroll
    for (int q = 0; q < kMaxSlots; ++q) { m[q] = 0.0f; nan[q] = 0; }
    if (kThreads % n_slots == 0) {
        float mm = 0.0f;
        int nn = 0;
#pragma unroll
        for (int t = 0; t < kPerThread; ++t) {   // elements past the end hold 0
            mm = fmaxf(mm, keep[t]);
            nn |= keep[t] != keep[t];
        }
        const int sl = tid % n_slots;
#pragma unroll
        for (int q = 0; q < kMaxSlots; ++q)
            if (q == sl) { m[q] = mm; nan[q] = nn; }
    } else {
        const int ds = kThreads % n_slots;
        int sl = tid % n_slots;
#pragma unroll
        for (int t = 0; t < kPerThread; ++t) {
#pragma unroll
            for (int q = 0; q < kMaxSlots; ++q)
                if (q == sl) {
                    m[q] = fmaxf(m[q], keep[t]);
                    nan[q] |= keep[t] != keep[t];
                }
            sl += ds;
            sl -= sl >= n_slots ? n_slots : 0;
        }
    }
    for (int q = 0; q < n_slots; ++q) {   // uniform bound
        const float wm = wave_max_f32(m[q]);
        const int wn = __any(nan[q]);
        if (lane == 0) {
            red_max[wave][q] = wm;
            red_nan[wave][q] = wn;
        }
    }
    __syncthreads();
    if (tid < n_slots) {
        float a = 0.0f;
        int any_nan = 0;
        for (int w = 0; w < kThreads / kWave; ++w) {
            a = fmaxf(a, red_max[w][tid]);
            any_nan |= red_nan[w][tid];
        }
        const float sc = delayed_scale(a, any_nan != 0, scale[tid], fp8_max, margin);
        scale[tid] = sc;
        scale_inv[tid] = 1.0f / sc;
    }
    // Roll: row i <- row i-1 for i >= 1, row 0 <- 0, from the registers.  Every
    // value was read before the barrier above, so no thread overwrites a value
    // another thread still has to read.
#pragma unroll
    for (int t = 0; t < kPerThread; ++t) {
        const int j = tid + t * kThreads;
        if (j + n_slots < total) hist[j + n_slots] = keep[t];
    }
    if (tid < n_slots) hist[tid] = 0.0f;
}

__global__ __launch_bounds__(kThreads) void scaling_update_kernel(float* hist, float* scale,
                                                                 float* scale_inv, int len,
                                                                 int n_slots, int margin,
                                                                 float fp8_max) {
    scaling_update_block(hist, scale, scale_inv, len, n_slots, margin, fp8_max);
}

// Many state blocks in one launch, one workgroup each (the same work as one
// scaling_update_kernel per block).
__global__ __launch_bounds__(kThreads) void scaling_update_batch_kernel(UpdateBatch b) {
    const UpdateJob& j = b.job[blockIdx.x];
    scaling_update_block(j.hist, j.scale, j.scale_inv, b.len, j.n_slots, b.margin, j.fp8_max);
}

}  // namespace

hipError_t launch_scaling_update_batch(const UpdateBatch& b, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    if (n > kMaxUpdateBatch) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scaling_update_batch_kernel, dim3(n), dim3(kThreads), 0, stream, b);
    return hipGetLastError();
}

hipError_t launch_meta_init(float* hist, float* scale, float* scale_inv, int len, int n_slots,
                            hipStream_t stream) {
    const int total = len * n_slots;
    const int blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(meta_init_kernel, dim3(blocks), dim3(kThreads), 0, stream, hist, scale,
                       scale_inv, total, n_slots);
    return hipGetLastError();
}

hipError_t launch_scaling_update(float* hist, float* scale, float* scale_inv, int len,
                                 int n_slots, int margin, float fp8_max, hipStream_t stream) {
    hipLaunchKernelGGL(scaling_update_kernel, dim3(1), dim3(kThreads), 0, stream, hist, scale,
                       scale_inv, len, n_slots, margin, fp8_max);
    return hipGetLastError();
}

}  // namespace fp8ln
