// Device helpers shared by the gfx950 kernels: bf16 unpacking, the FP8 encoder,
// wave reductions and the amax atomic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launchers.hpp"

namespace fp8ln {

constexpr int kWave = 64;

template <int FMT>
struct Fp8Traits;
template <>
struct Fp8Traits<kE4M3> {
    static constexpr float kMax = 448.0f;
};
template <>
struct Fp8Traits<kE5M2> {
    static constexpr float kMax = 57344.0f;
};

// ---- streaming memory access ------------------------------------------------
// Non-temporal loads and stores for data touched once per kernel (the whole-
// tensor streams of the LayerNorm, cast and transpose kernels): on MI355X they
// raise a 2:1 read:write stream from about 5.6 to about 6.5 TB/s.

typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_nt(const float4* p) {
    const nt_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
    __builtin_nontemporal_store(nt_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4*>(p));
}
__device__ __forceinline__ void store_nt(uint2* p, uint2 v) {
    __builtin_nontemporal_store(nt_u32x2{v.x, v.y}, reinterpret_cast<nt_u32x2*>(p));
}

// ---- bf16 ------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two binary32 values -> two bf16 (lo in the low half), rounded to nearest even
// by gfx950's packed conversion (one v_cvt_pk_bf16_f32 for the pair); a NaN
// stays a quiet NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 values held in a 16-byte word.
__device__ __forceinline__ void unpack_bf16x8(const uint4& w, float* v) {
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

// ---- FP8 encoder -------------------------------------------------------------
//
// The hardware conversion rounds to nearest even in the OCP formats; the value is
// first clamped to +-max with a median-of-three so that overflow (infinities
// included) saturates.  The median does not keep NaN, so a NaN input is patched
// to the canonical code 0x7F afterwards; callers find NaNs cheaply from the amax
// bits they already track (|x| bits above 0x7f800000) and call the patch only then.

template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
    constexpr float M = Fp8Traits<FMT>::kMax;
    a = __builtin_amdgcn_fmed3f(a, -M, M);
    b = __builtin_amdgcn_fmed3f(b, -M, M);
    if constexpr (FMT == kE4M3)
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
    else
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

// Four values -> four codes in one 32-bit word (byte i = code of v[i]).
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float v0, float v1, float v2, float v3) {
    uint32_t r = cvt_pk<FMT, false>(v0, v1, 0u);
    return cvt_pk<FMT, true>(v2, v3, r);
}

// v * s rounded to odd: the binary32 product with its last bit forced to 1
// when it is inexact (moving one ulp toward the exact product when needed).  A
// round-to-odd result at 24 bits followed by one round-to-nearest-even at <= 22
// bits equals the correct rounding of the exact product, so the FP8 code of
// v * s comes out as if the product had never been rounded to binary32.
// Without it, inputs with few significant bits (bf16 weights and gradients)
// times a binary32 scale land on FP8 rounding midpoints after the binary32
// rounding for whole mantissa patterns at once.
__device__ __forceinline__ float mul_round_odd(float v, float s) {
    const float p = v * s;
    const float e = fmaf(v, s, -p);            // exact remainder of the product
    const uint32_t b = __float_as_uint(p);
    // Inexact (a non-zero finite remainder; an infinite product has a NaN or
    // infinite remainder and stays infinite, so that the encoder saturates it):
    // the product truncated toward zero is p itself when the remainder has p's
    // sign and one step below p in magnitude otherwise, and forcing its last bit
    // to 1 gives the round-to-odd result.
    const uint32_t down = (uint32_t)((int32_t)(__float_as_uint(e) ^ b) >> 31);   // 0 or -1
    const bool inexact = __builtin_amdgcn_classf(e, 0x198);   // +-normal, +-subnormal
    return __uint_as_float(inexact ? ((b + down) | 1u) : b);
}

// The delayed scale from a history window: fp8_max / max / 2^margin as one
// binary32 division and an exact power-of-two step; the old scale stays when the
// window holds a NaN, its max is zero or not finite, or the result is not a
// finite positive number.
__device__ __forceinline__ float delayed_scale(float window_max, bool any_nan, float old_scale,
                                               float fp8_max, int margin) {
    float sc = old_scale;
    if (!any_nan && window_max > 0.0f && window_max <= 3.402823466e38f) {
        float ns = fp8_max / window_max;   // IEEE binary32 division
        ns = ldexpf(ns, -margin);          // exact unless the result is subnormal
        if (ns > 0.0f && ns <= 3.402823466e38f) sc = ns;
    }
    return sc;
}

// Replace the code of every NaN among v[0..3] by 0x7F.
__device__ __forceinline__ uint32_t patch_nan4(uint32_t codes, const float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (v[i] != v[i]) codes = (codes & ~(0xffu << (8 * i))) | (0x7fu << (8 * i));
    return codes;
}

// |x| as bits; integer max over these ranks NaN above +inf above every finite value.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

constexpr uint32_t kInfBits = 0x7f800000u;

// A body's hook that does nothing (see ln_cast_amax_rows, cast_tiles).
struct NoPre {
    __device__ void operator()() const {}
};

// ---- reductions ----------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// DPP lane permutations (VOP DPP control values of the gfx9 family).
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes, every lane receiving the result: four DPP steps inside
// each 16-lane row, then two cross-row exchanges.  Each step adds a value to its
// mirror image, so every lane of a group computes the same bits.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f32<kDppQuadSwap1>(v);
    v += dpp_f32<kDppQuadSwap2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    return v;
}

// Wave-wide max with fmaxf semantics (a NaN operand is dropped): DPP steps
// inside each 16-lane row, then two shuffles across rows.
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, dpp_f32<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
    v = fmaxf(v, __shfl_xor(v, 16, kWave));
    v = fmaxf(v, __shfl_xor(v, 32, kWave));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
        v = v > o ? v : o;
    }
    return v;
}

// Block-wide max of amax bits followed by at most one atomic into *amax (a float
// whose bits order like unsigned integers because it is never negative).  All
// threads of the block must call it.  `smem` holds at least one uint32 per wave.
//
// Atomics on one address serialise in the L2 (some ten nanoseconds each), so the
// thousands of workgroups of a streaming kernel, which all finish together,
// would queue thousands of them.  The stored value only ever grows during a
// step, so any value read from it is at most its final value: with CHECK, a
// block whose max does not exceed what it reads cannot change the result and
// skips the atomic; typically only a handful of blocks, those that raise the
// running max, issue one.  GEMM epilogues finish spread over the whole kernel,
// where the atomics do not queue and the read would only add a round trip to
// each tile's end: they call it without CHECK.
template <bool CHECK = true>
__device__ __forceinline__ void block_amax_atomic(uint32_t bits, float* amax, uint32_t* smem) {
    bits = wave_max_u32(bits);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (lane == 0) smem[wave] = bits;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = 0;
        const int nw = (blockDim.x + kWave - 1) / kWave;
        for (int w = 0; w < nw; ++w) m = smem[w] > m ? smem[w] : m;
        unsigned int* a = reinterpret_cast<unsigned int*>(amax);
        if (m != 0 &&
            (!CHECK || m > __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)))
            atomicMax(a, m);
    }
}

}  // namespace fp8ln
