// The step-start scaling update folded into a step's kernels (FusedUpdate): the
// scales formed from the history window by every workgroup that needs them, and
// the history roll done once, after every reader of the window has finished.
//
// The delayed recipe takes each step's scale from the amax history of earlier
// steps only (tutorial "Accelerating Transformer Training with NVIDIA Transformer
// Engine ...", setup and benchmark listings: the recipe's history length and
// "max" reduction), so the scale is known before the step's data is read: the
// update can ride inside the launches that read the data.
#pragma once

#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

// The update's scales of every slot from the history window (fmaxf max, a NaN
// flagged apart), as fp8ln's scaling update forms them: sh[2 q] = scale of slot
// q, sh[2 q + 1] = 1 / scale.  Thread t reads entries t, t + NT, ... of the
// flattened [len][n_slots] history; n_slots divides NT, so all of a thread's
// entries belong to slot t % n_slots, and lanes of one slot meet in a butterfly
// over the lane bits at and above n_slots.  Workgroup 0 also writes the scales
// into the state block: every workgroup computes the same values, and a
// workgroup that reads a slot's old scale after the write gets the same result
// (the old scale enters only where it is kept), so the write needs no ordering.
// All NT threads call it.
template <int NT>
__device__ __forceinline__ void window_scales(const FusedUpdate& u, float* sh) {
    __shared__ float wmax[NT / kWave][kMaxMetaSlots];
    __shared__ int wnan[NT / kWave][kMaxMetaSlots];
    const int n = u.n_slots, total = u.len * n;
    float m = 0.0f;
    int nan = 0;
#pragma unroll 8
    for (int j = threadIdx.x; j < total; j += NT) {   // independent loads in flight together
        const float v = u.hist[j];
        m = fmaxf(m, v);
        nan |= v != v;
    }
    for (int off = n; off < kWave; off <<= 1) {   // n is a power of two
        m = fmaxf(m, __shfl_xor(m, off, kWave));
        nan |= __shfl_xor(nan, off, kWave);
    }
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane < n) {
        wmax[wave][lane] = m;
        wnan[wave][lane] = nan;
    }
    __syncthreads();
    if (threadIdx.x < n) {
        const int q = threadIdx.x;
        float a = 0.0f;
        int any = 0;
        for (int w = 0; w < NT / kWave; ++w) {
            a = fmaxf(a, wmax[w][q]);
            any |= wnan[w][q];
        }
        const float sc = delayed_scale(a, any != 0, u.scale[q], u.fp8_max, u.margin);
        sh[2 * q] = sc;
        sh[2 * q + 1] = 1.0f / sc;
        if (blockIdx.x == 0) {
            u.scale[q] = sc;
            u.scale_inv[q] = 1.0f / sc;
        }
    }
    __syncthreads();
}

// The history roll of a folded update, by one workgroup (at least 256 threads,
// all calling it): rows 0 .. len - 2 move down one row, row 0 takes the amaxes
// recorded in ws (every slot), and ws is cleared.  Every value is read into
// registers before any is written.  The caller is a launch that follows the one
// that recorded the amaxes on the same stream.
__device__ __forceinline__ void roll_history(float* hist, uint32_t* ws, int len, int n) {
    constexpr int kPer = 32;   // len * n <= 1024 * 8 values over at least 256 threads
    const int t = threadIdx.x, nt = blockDim.x, moved = (len - 1) * n;
    float keep[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int j = t + k * nt;
        keep[k] = j < moved ? hist[j] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int j = t + k * nt;
        if (j < moved) hist[j + n] = keep[k];
    }
    if (t < n) {
        hist[t] = __uint_as_float(ws[t]);
        ws[t] = 0u;
    }
}

}  // namespace fp8ln
