// FP8 GEMM on the CDNA4 matrix cores with fused dequantising epilogues: the tile
// template, its kernels and their per-format launchers (instantiated per operand
// format pair in gemm_<a>_<b>.hip, so the pairs compile in parallel).
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
// Tiling (gfx950): every wave owns a sub-tile of V_MFMA_F32_32X32X64_F8F6F4
// results accumulated in fp32 registers (64 x 128 in the large tiles), two or
// more waves per SIMD.  Four workgroup shapes: 256 x 256 over eight waves (one
// workgroup per CU, least LDS and L2 traffic per MFMA, for long K); 128 x 256
// over four waves with a three-stage ring, two workgroups per CU so that one's
// epilogue overlaps the other's main loop (K up to 2048); 128 x 128 over four
// waves of 64 x 64 and 64 x 64 over four waves of 32 x 32 for problems too
// small to fill the CUs otherwise; independent small products can share one
// grouped launch.  The
// operand formats (E4M3 / E5M2) are chosen per operand by the instruction's
// cbsz / blgp fields.  K advances 64 bytes per stage through an LDS ring filled
// by direct-to-LDS buffer loads issued NS - 1 stages ahead, so memory latency
// hides behind MFMA work without holding any registers; an XOR layout of
// 16-byte chunks keeps fragment reads free of bank conflicts.
//
// The MFMA computes the transposed product (B rows in, A rows out), so each
// lane ends up holding four consecutive output columns of one row; the
// epilogue stages results through the (then idle) LDS ring and writes whole
// output rows.  Tiles are ordered so that the blocks of one XCD (blocks are
// dealt to the 8 XCDs round robin) cover a compact band of the output and
// share operands in their L2.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"
#include "step_update.hpp"

namespace fp8ln {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BKS = 64;        // bytes of K per pipeline stage
constexpr int kGroupM = 8;     // tile rows per ordering group
constexpr int kBufferWord3 = 0x00020000;      // raw buffer descriptor flags (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u; // offset past any tile: loads read 0

// 16-byte chunk c of LDS row r lives at chunk position swz(r, c).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

// GELU, tanh form: gelu(h) = h/2 (1 + t), t = tanh(k0 (h + k1 h^3)), with
// k0 = sqrt(2 / pi), k1 = 0.044715, and its derivative
//     gelu'(h) = (1 + t)/2 + h/2 (1 - t^2) k0 (1 + 3 k1 h^2).
// With v = 2 log2(e) k0 h (1 + k1 h^2): s = (1 + t)/2 = 1 / (1 + 2^-v) and
// (1 - t^2) / 4 = s (1 - s), so
//     gelu(h) = h s,   gelu'(h) = s (1 + 2 k0 (1 + 3 k1 h^2) h (1 - s)),
// neither of which cancels for negative h (the forms h/2 + h/2 t and
// (1 + t)/2 + ... lose the relative accuracy of small values there).  2^-v and
// the reciprocal are the hardware's (about one ulp each).
constexpr float kGeluK0 = 0.7978845608028654f;                 // sqrt(2 / pi)
constexpr float kGeluK1 = 0.044715f;
constexpr float kGeluV0 = 2.0f * 1.4426950408889634f * 0.7978845608028654f;   // 2 log2(e) k0
constexpr float kGeluV1 = kGeluV0 * 0.044715f;

__device__ __forceinline__ float gelu_f(float h) {
    const float nv = h * fmaf(-kGeluV1, h * h, -kGeluV0);   // -v
    return h * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(nv));
}

__device__ __forceinline__ float gelu_grad_f(float h) {
    const float h2 = h * h;
    const float nv = h * fmaf(-kGeluV1, h2, -kGeluV0);                      // -v
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(nv));
    const float c = fmaf(6.0f * kGeluK0 * kGeluK1, h2, 2.0f * kGeluK0);    // 2 k0 (1 + 3 k1 h^2)
    return sg * fmaf(h * (1.0f - sg), c, 1.0f);
}

// GELU, erf form: gelu(h) = h/2 (1 + erf(h / sqrt 2)) = h/2 erfc(-h / sqrt 2)
// and gelu'(h) = erfc(-h / sqrt 2) / 2 + h exp(-h^2 / 2) / sqrt(2 pi) (erfc keeps
// the small values for negative h accurate).
__device__ __forceinline__ float gelu_erf_f(float h) {
    return 0.5f * h * erfcf(h * -0.70710678118654752f);
}

__device__ __forceinline__ float gelu_erf_grad_f(float h) {
    const float e = erfcf(h * -0.70710678118654752f);
    const float d = __expf(-0.5f * h * h) * 0.39894228040143268f;   // 1 / sqrt(2 pi)
    return fmaf(h, d, 0.5f * e);
}

// The activation form as a compile-time choice.  Epilogues branch on the
// (uniform) runtime flag once, around whole loops, so a value never pays for
// both forms.
template <bool ERF>
__device__ __forceinline__ float act_f(float h) {
    if constexpr (ERF) return gelu_erf_f(h);
    else return gelu_f(h);
}
template <bool ERF>
__device__ __forceinline__ float act_grad_f(float h) {
    if constexpr (ERF) return gelu_erf_grad_f(h);
    else return gelu_grad_f(h);
}

// LDS layout of one operand stage: 64-byte rows stored in pairs as 128-byte
// lines (line L holds rows 2L and 2L+1); the eight 16-byte slots of a line are
// XOR-permuted with f(L) so that fragment reads of 16 consecutive rows (or 8,
// in a 32-bank view) touch distinct banks.
__device__ __forceinline__ int line_perm(int L) { return (L & 3) ^ ((L >> 2) & 1); }

// Byte offset inside a stage of 16-byte chunk c (0..3) of row r.
__device__ __forceinline__ int lds_off(int r, int c) {
    const int L = r >> 1;
    return L * 128 + ((((r & 1) << 2) | c) ^ line_perm(L)) * 16;
}

// s_waitcnt immediate that waits for at most n outstanding vector-memory ops
// and leaves the other counters unconstrained (gfx9 encoding).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

typedef __attribute__((address_space(3))) uint8_t lds8;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS accesses through address-space-3 pointers (ds_read / ds_write).
template <class T>
__device__ __forceinline__ void lds_st(lds8* a, T v) {
    *reinterpret_cast<__attribute__((address_space(3))) T*>(a) = v;
}
template <class T>
__device__ __forceinline__ T lds_ld(const lds8* a) {
    return *reinterpret_cast<const __attribute__((address_space(3))) T*>(a);
}

// Smallest power of two P such that a stage of STAGE bytes holds a multiple of 32
// rows of LB / P bytes.
constexpr int staging_parts(int LB, int STAGE) {
    int p = 1;
    while ((STAGE / (LB / p)) % 32 != 0) p *= 2;
    return p;
}

// A tile of ROWS rows of LB bytes staged in a ring of LDS stages of STAGE bytes.
// Each row is cut into P parts of RB = LB / P bytes, P chosen so that a stage holds
// RPS part rows with RPS a multiple of 32: the 32 rows that the lanes of a wave
// touch at once (rows 32 k .. 32 k + 31 of one part) then always share a stage,
// and the stage is picked from wave-uniform values, by scalar instructions, with
// no per-lane select.  Part row s = part * ROWS + r lives in stage s / RPS, and
// its 16-byte chunk c at chunk position c ^ (s & SWM).
template <int LB, int ROWS, int STAGE>
struct Staging {
    static constexpr int P = staging_parts(LB, STAGE);
    static constexpr int RB = LB / P;
    static constexpr int NC = RB / 16;
    static constexpr int RPS = STAGE / RB;
    static constexpr int SWM = (NC < 32 ? NC : 32) - 1;
    static constexpr int UNITS = ROWS * P * NC;   // 16-byte chunks of the tile
    static_assert(RB % 16 == 0 && RPS % 32 == 0 && ROWS % 32 == 0, "staging geometry");

    // Start of part row part * ROWS + r_u, for a wave-uniform part and a
    // wave-uniform multiple of 32 r_u (a scalar value, computed once per block of
    // 32 rows and kept).
    template <class Ring>
    __device__ __forceinline__ static lds8* row(Ring ring, int part, int r_u) {
        const int s_u = part * ROWS + r_u;
        return ring(s_u / RPS) + (s_u % RPS) * RB;
    }
    // Chunk c (of the part) of row r_l in [0, 32) below a row() start.
    __device__ __forceinline__ static lds8* in_row(lds8* base, int r_l, int c) {
        return base + r_l * RB + ((c ^ (r_l & SWM)) << 4);
    }
    // LDS address of chunk position u (positions in stage order)
    template <class Ring>
    __device__ __forceinline__ static lds8* pos(Ring ring, int u) {
        return ring(u / (RPS * NC)) + (u % (RPS * NC)) * 16;
    }
    // tile row and byte column of the chunk that chunk position u holds
    __device__ __forceinline__ static void source(int u, int& row, int& byte) {
        const int s = u / NC, c = u % NC;
        row = s % ROWS;
        byte = (s / ROWS) * RB + ((c ^ (s & SWM)) << 4);
    }
    // Copies the staged tile to dst, whose rows are ld bytes apart, as 16-byte
    // chunks; rows at or past rows_valid and bytes at or past bytes_valid are
    // skipped.  Each wave writes whole part rows, with non-temporal stores (the
    // output is not read again by this kernel).  Thread t always takes chunk
    // t % NC of part row t / NC of each group of NT / NC part rows, so its global
    // address is one per-thread base plus a uniform offset per iteration.
    template <int NT, bool CHECK, class Ring>
    __device__ __forceinline__ static void copy_out(Ring ring, int t, uint8_t* dst, int64_t ld,
                                                    int64_t rows_valid, int64_t bytes_valid) {
        constexpr int PER_STAGE = RPS * NC / NT;   // loop iterations per stage
        constexpr int RPI = NT / NC;               // part rows per iteration
        static_assert(UNITS % NT == 0 && (RPS * NC) % NT == 0, "copy split");
        static_assert(NT % NC == 0 && ROWS % RPI == 0 && RPS % RPI == 0, "copy rows");
        const int r_t = t / NC, c = t % NC;
        const int rv = (int)(rows_valid < ROWS ? rows_valid : ROWS) - r_t;
        const int bv = (int)(bytes_valid < LB ? bytes_valid : LB) - c * 16;
        uint8_t* base = dst + r_t * ld + c * 16;
#pragma unroll
        for (int it = 0; it < UNITS / NT; ++it) {
            const int s_u = it * RPI;                      // first part row of the iteration
            const int r_u = s_u % ROWS, part = s_u / ROWS;
            const int s = s_u + r_t;
            const u32x4 w = lds_ld<u32x4>(ring(it / PER_STAGE) + (s_u % RPS + r_t) * RB +
                                          ((c ^ (s & SWM)) << 4));
            if (!CHECK || (r_u < rv && part * RB < bv))
                __builtin_nontemporal_store(
                    w, reinterpret_cast<u32x4*>(base + r_u * ld + part * RB));
        }
    }
};

// One butterfly step over lanes l and l ^ MASK: each keeps one half of its N
// values and adds the partner's copy of that half.
template <int N, int MASK>
__device__ __forceinline__ void butterfly_step(float* v, int fr) {
    const bool upper = (fr & MASK) != 0;
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
        const float send = upper ? v[k] : v[k + N / 2];
        const float keep = upper ? v[k + N / 2] : v[k];
        v[k] = keep + __shfl_xor(send, MASK, kWave);
    }
}

// Sums NV values over the 32 lanes that share lane / 32.  Afterwards lane l
// holds in v[0 .. NV/32) the sums of the values at index (l % 32) * NV/32 + k.
template <int NV>
__device__ __forceinline__ void butterfly_sum(float* v, int fr) {
    static_assert(NV % 32 == 0, "butterfly width");
    butterfly_step<NV, 16>(v, fr);
    butterfly_step<NV / 2, 8>(v, fr);
    butterfly_step<NV / 4, 4>(v, fr);
    butterfly_step<NV / 8, 2>(v, fr);
    butterfly_step<NV / 16, 1>(v, fr);
}

// EPIX = epilogue + 16 ACT + 64 FULL: ACT 1 and 2 fix the GELU form at compile
// time (tanh, erf) for the GELU / GELU' epilogues whose loops would otherwise be
// compiled once per form behind a runtime branch, which makes the register
// allocator spill the accumulators; ACT 0 reads the form from the parameters.
// FULL 1: no tile crosses the product's edge (the epilogue drops its bounds
// tests; one copy of the epilogue per kernel, as two copies behind a branch
// spill).
// vb: the tile's block index (the kernel's own, or its index inside one problem
// of a grouped launch).  GROUP only tags the grouped kernel's instantiation (the
// same specialization called from two kernels does not resolve in hipcc's host
// pass).
template <int BM, int BN, int WGM, int WGN, int NS, int FA, int FB, int EPIX, int QF,
          bool GROUP = false>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int vb) {
    constexpr int EPI = EPIX % 16;
    constexpr int ACT = EPIX / 16 % 4;
    constexpr bool FULLX = EPIX >= 64;
    static_assert(NS == 3 || NS == 4, "three or four pipeline stages");
    constexpr int NW = WGM * WGN;              // waves per workgroup
    constexpr int WM = BM / WGM, WN = BN / WGN;  // wave sub-tile
    constexpr int TM = WM / 32, TN = WN / 32;  // 32 x 32 MFMA tiles per wave
    constexpr int A_BYTES = BM * BKS, B_BYTES = BN * BKS;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_DMA = A_BYTES / 1024 / NW;  // 1 KB direct-to-LDS loads per wave and stage
    constexpr int B_DMA = B_BYTES / 1024 / NW;
    constexpr int P = A_DMA + B_DMA;           // vector-memory ops per wave and stage
    // one LDS array per pipeline stage, so the compiler tracks each stage's loads
    __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st3[NS == 4 ? STAGE : 16];

    const int t = threadIdx.x;
    if constexpr (!GROUP) {
        if (p.roll_hist && vb == 0) roll_history(p.roll_hist, p.roll_ws, p.roll_len, p.roll_slots);
    }
    const int lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    static_assert(A_DMA * NW * 1024 == A_BYTES && B_DMA * NW * 1024 == B_BYTES, "stage split");
    const int64_t M = p.M, N = p.N, K = p.K;

    // ---- tile order ---------------------------------------------------------
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    int b = vb;
    if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);   // one band per XCD
    const int per_group = kGroupM * tiles_n;
    const int first_m = (b / per_group) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int tile_m = first_m + (b % per_group) % gsize;
    const int tile_n = (b % per_group) / gsize;
    const int64_t m0 = (int64_t)tile_m * BM;
    const int64_t n0 = (int64_t)tile_n * BN;

    // ---- global -> LDS, direct ------------------------------------------------
    // Buffer descriptors cover only this tile's rows, so rows past M (or N) read
    // as zero in hardware.  Their record count and the offsets below are 32-bit,
    // and kOutOfRange (2^31) must lie past every record: a tile spans at most
    // 256 rows of K bytes, so K (in bytes) must stay below 2^31 / 256 = 2^23
    // (launch_gemm refuses larger K, and the C-ABI checks it before any launch).  A direct-to-LDS load writes lane l's 16 bytes at
    // base + 16 l, so each lane fetches the global chunk that belongs at its LDS
    // position: DMA j of this wave fills positions u = (wave * DMA + j) * 64 + lane.
    const int64_t rows_a = min<int64_t>(BM, M - m0);
    const int64_t rows_b = min<int64_t>(BN, N - n0);
    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.A + m0 * K), (short)0, (int)(rows_a * K), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.B + n0 * K), (short)0, (int)(rows_b * K), kBufferWord3);
    uint32_t voff_a[A_DMA], voff_b[B_DMA];
    int cofs_a[A_DMA], cofs_b[B_DMA];
    auto place = [&](int u, uint32_t& voff, int& cofs) {
        const int L = u >> 3;
        const int x = (u & 7) ^ line_perm(L);
        const int r = 2 * L + (x >> 2);
        cofs = (x & 3) * 16;
        voff = (uint32_t)(r * K + cofs);
    };
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) place((wave * A_DMA + j) * 64 + lane, voff_a[j], cofs_a[j]);
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) place((wave * B_DMA + j) * 64 + lane, voff_b[j], cofs_b[j]);

    using lds_ptr = __attribute__((address_space(3))) void*;
    // One code path for every step: the K offset goes into the (range-checked)
    // vector offset and chunks at or past K get an out-of-range offset, so the
    // last partial step and the zero steps past the end read zeros.
    auto issue = [&](uint8_t* stage, int64_t k0) {
        uint8_t* sa = stage + wave * A_DMA * 1024;
        uint8_t* sb = stage + A_BYTES + wave * B_DMA * 1024;
#pragma unroll
        for (int j = 0; j < A_DMA; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (lds_ptr)(sa + j * 1024), 16,
                k0 + cofs_a[j] < K ? voff_a[j] + (uint32_t)k0 : kOutOfRange, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < B_DMA; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (lds_ptr)(sb + j * 1024), 16,
                k0 + cofs_b[j] < K ? voff_b[j] + (uint32_t)k0 : kOutOfRange, 0, 0, 0);
    };

    // ---- MFMA main loop ----------------------------------------------------
    // A 32x32x64 operand fragment: lane l feeds row l % 32 with the K bytes
    // [32 (l / 32), +32) of the stage, i.e. chunks 2 (l / 32) and 2 (l / 32) + 1.
    const int wm = wave / WGN;
    const int wn = wave % WGN;
    const int fr = lane & 31;
    const int fh = lane >> 5;
    v16f acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[j][i] = v16f{};

    auto frag = [&](const uint8_t* s, int r) -> v8i {
        const uint4 lo = *reinterpret_cast<const uint4*>(s + lds_off(r, 2 * fh));
        const uint4 hi = *reinterpret_cast<const uint4*>(s + lds_off(r, 2 * fh + 1));
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // The 256 x 256 tile reads each stage's fragments one step early (its waves
    // have registers for a second fragment set); the other tiles read them at the
    // start of the step that uses them.
    constexpr bool kEarlyFrags = BM == 256 && BN == 256;
    if constexpr (kEarlyFrags) {
        // One stage's operand fragments: TM of A, TN of B.
        struct Frags {
            v8i a[TM];
            v8i b[TN];
        };
        auto read_frags = [&](const uint8_t* stage, Frags& f) {
    #pragma unroll
            for (int i = 0; i < TM; ++i) f.a[i] = frag(stage, wm * WM + 32 * i + fr);
    #pragma unroll
            for (int j = 0; j < TN; ++j) f.b[j] = frag(stage + A_BYTES, wn * WN + 32 * j + fr);
        };
        auto mfmas = [&](const Frags& f) {
            if constexpr (FA == kOpBf16) {
                // bf16: a stage holds 32 elements of K per row, two 32x32x16 MFMAs.
                // Each lane splits its 32-byte fragment into halves h = 0, 1; MFMA h
                // sums over the elements of half h of every lane.  A and B split
                // alike, so every k meets its partner exactly once.
                static_assert(FB == kOpBf16, "bf16 takes bf16");
    #pragma unroll
                for (int h = 0; h < 2; ++h)
    #pragma unroll
                    for (int j = 0; j < TN; ++j)
    #pragma unroll
                        for (int i = 0; i < TM; ++i) {
                            const v8i& bv = f.b[j];
                            const v8i& av = f.a[i];
                            const v4i b4 = h ? v4i{bv[4], bv[5], bv[6], bv[7]}
                                             : v4i{bv[0], bv[1], bv[2], bv[3]};
                            const v4i a4 = h ? v4i{av[4], av[5], av[6], av[7]}
                                             : v4i{av[0], av[1], av[2], av[3]};
                            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(v8bf, b4), __builtin_bit_cast(v8bf, a4),
                                acc[j][i], 0, 0, 0);
                        }
            } else {
                // D[n][m] = sum_k B[n][k] A[m][k]: the B rows are the MFMA's first operand
    #pragma unroll
                for (int j = 0; j < TN; ++j)
    #pragma unroll
                    for (int i = 0; i < TM; ++i)
                        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            f.b[j], f.a[i], acc[j][i], FB, FA, 0, 0, 0, 0);
            }
        };
        // Stage kt lives in st[kt % NS] and its fragments are read into registers one
        // step early: step kt multiplies the fragments of stage kt (read during step
        // kt - 1) while it reads those of stage kt + 1, so the MFMAs never wait on LDS
        // at the start of a step.  Before reading stage kt + 1 a wave waits for its
        // own loads of that stage (the NS - 2 later stages may stay in flight); the
        // barrier then makes every wave's loads visible and shows that every wave has
        // its stage-kt fragments in registers, so st[kt % NS] is refilled right away,
        // with stage kt + NS.  The barrier is a bare s_barrier: __syncthreads() adds a
        // workgroup fence, which waits for every outstanding load, the prefetched
        // stages included.  Every step looks the same: the look-ahead stages past the
        // end of K are filled with zeros (all chunks out of range), so the wait count
        // is a constant.  Two fragment sets alternate, so the step sequence is
        // unrolled by 2 NS and the stage buffers and fragment sets are fixed per step.
        uint8_t* const ring_st[4] = {st0, st1, st2, st3};
        Frags fa, fb;
        auto step = [&](int i, int kt) {   // i: position in the unrolled sequence
            Frags& use = (i & 1) ? fb : fa;
            Frags& load = (i & 1) ? fa : fb;
            // Scheduling fences keep the wait, the barrier and the refill at the top
            // of the step: left to itself the scheduler sinks the refill below the
            // MFMAs (and lifts MFMAs of the previous step past the barrier), which
            // costs a step of latency cover.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * P));
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            issue(ring_st[i % NS], (int64_t)(kt + NS) * BKS);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(ring_st[(i + 1) % NS], load);
            mfmas(use);
        };

        const int nk = (int)((K + BKS - 1) / BKS);
        issue(st0, 0);
        issue(st1, BKS);
        issue(st2, 2 * BKS);
        if constexpr (NS == 4) issue(st3, 3 * BKS);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * P));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        read_frags(st0, fa);
        int kt = 0;
        for (; kt + 2 * NS <= nk; kt += 2 * NS) {
    #pragma unroll
            for (int i = 0; i < 2 * NS; ++i) step(i, kt + i);
        }
    #pragma unroll
        for (int i = 0; i < 2 * NS - 1; ++i)
            if (kt + i < nk) step(i, kt + i);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the zero-filled look-ahead stages
    } else {
        auto compute = [&](const uint8_t* stage) {
            const uint8_t* sa = stage;
            const uint8_t* sb = stage + A_BYTES;
            v8i af[TM];
    #pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = frag(sa, wm * WM + 32 * i + fr);
            if constexpr (FA == kOpBf16) {
                // bf16: a stage holds 32 elements of K per row, two 32x32x16 MFMAs.
                // Each lane splits its 32-byte fragment into halves h = 0, 1; MFMA h
                // sums over the elements of half h of every lane.  A and B split
                // alike, so every k meets its partner exactly once.
                static_assert(FB == kOpBf16, "bf16 takes bf16");
                v8i bfr[TN];
    #pragma unroll
                for (int j = 0; j < TN; ++j) bfr[j] = frag(sb, wn * WN + 32 * j + fr);
    #pragma unroll
                for (int h = 0; h < 2; ++h)
    #pragma unroll
                    for (int j = 0; j < TN; ++j)
    #pragma unroll
                        for (int i = 0; i < TM; ++i) {
                            const v8i& bv = bfr[j];
                            const v8i& av = af[i];
                            const v4i b4 = h ? v4i{bv[4], bv[5], bv[6], bv[7]}
                                             : v4i{bv[0], bv[1], bv[2], bv[3]};
                            const v4i a4 = h ? v4i{av[4], av[5], av[6], av[7]}
                                             : v4i{av[0], av[1], av[2], av[3]};
                            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(v8bf, b4), __builtin_bit_cast(v8bf, a4),
                                acc[j][i], 0, 0, 0);
                        }
                return;
            }
            // D[n][m] = sum_k B[n][k] A[m][k]: the B rows are the MFMA's first operand
    #pragma unroll
            for (int j = 0; j < TN; ++j) {
                const v8i bf = frag(sb, wn * WN + 32 * j + fr);
    #pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bf, af[i], acc[j][i], FB, FA, 0, 0, 0, 0);
            }
        };
        // Stage kt lives in st[kt % NS]; loads run NS - 1 stages ahead.  Before
        // reading stage kt a wave waits for its own loads of that stage (the NS - 2
        // later stages may stay in flight), then the barrier makes every wave's loads
        // visible and frees the stage read in the previous step, which is refilled
        // right away.  The barrier is a bare s_barrier: __syncthreads() adds a
        // workgroup fence, which waits for every outstanding load, the prefetched
        // stages included.  The barrier also waits for the wave's own LDS reads, so
        // no wave refills a stage another wave is still reading.  Every step looks
        // the same: the look-ahead stages past the end of K are filled with zeros
        // (all chunks out of range), so the wait count is a constant.
        auto step = [&](uint8_t* cur, uint8_t* refill, int kt) {
            // Scheduling fences keep the wait, the barrier and the refill at the top
            // of the step: left to itself the scheduler sinks the refill below the
            // MFMAs (and lifts MFMAs of the previous step past the barrier), which
            // costs a step of latency cover.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * P));
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            issue(refill, (int64_t)(kt + NS - 1) * BKS);
            __builtin_amdgcn_sched_barrier(0);
            compute(cur);
        };

        // Whole rounds of NS steps, then the last nk % NS steps one by one (the same
        // step code, so the waits stay constant; only stages past K are zero-filled,
        // and no step multiplies one).
        const int nk = (int)((K + BKS - 1) / BKS);
        int kt = 0;
        issue(st0, 0);
        issue(st1, BKS);
        if constexpr (NS == 4) {
            issue(st2, 2 * BKS);
            for (; kt + 4 <= nk; kt += 4) {
                step(st0, st3, kt);
                step(st1, st0, kt + 1);
                step(st2, st1, kt + 2);
                step(st3, st2, kt + 3);
            }
            if (kt < nk) step(st0, st3, kt);
            if (kt + 1 < nk) step(st1, st0, kt + 1);
            if (kt + 2 < nk) step(st2, st1, kt + 2);
        } else {
            for (; kt + 3 <= nk; kt += 3) {
                step(st0, st2, kt);
                step(st1, st0, kt + 1);
                step(st2, st1, kt + 2);
            }
            if (kt < nk) step(st0, st2, kt);
            if (kt + 1 < nk) step(st1, st0, kt + 1);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the zero-filled look-ahead stages
    }
    __syncthreads();                            // the ring is free for the epilogue

    // ---- epilogue ----------------------------------------------------------------
    // acc[j][i] register r holds C[m][n] with m = m0 + wm WM + 32 i + (lane % 32)
    // and n = n0 + wn WN + 32 j + 8 (r / 4) + 4 (lane / 32) + (r % 4).  Results go
    // through the LDS ring so that global stores are whole rows: a wave writes its
    // values into a staged copy of (part of) the output tile, then every thread
    // copies 16-byte chunks of complete rows out.  Staged rows of RB bytes fill
    // the ring stages in order; chunk c of staged row r sits at chunk position
    // c ^ (r % 32) (or r % chunks-per-row when a row holds fewer than 32 chunks),
    // so the 32 rows a wave writes at once fall on different banks.
    constexpr int NT = 64 * NW;
    auto ring = [&](int sidx) -> lds8* {
        return sidx == 0 ? (lds8*)st0 : sidx == 1 ? (lds8*)st1 : sidx == 2 ? (lds8*)st2 : (lds8*)st3;
    };
    const float alpha = FA == kOpBf16 ? 1.0f : (*p.sinv_a) * (*p.sinv_b);   // bf16: no scales
    const int row_w = wm * WM + fr;      // tile row of this lane's i = 0 values
    const int col_w = wn * WN + 4 * fh;  // tile column of this lane's j = q = 0 values
    // tile rows and columns inside the product (32-bit bounds tests below)
    const int rows_in = (int)min<int64_t>(BM, M - m0);
    const int cols_in = (int)min<int64_t>(BN, N - n0);
    // FULLX: every tile lies wholly inside the product (M and N are multiples of
    // the tile, checked by the launcher), so the epilogue has no bounds tests.
    __shared__ float colp[EPI == kEpiDGeluFp8 ? WGM : 1][EPI == kEpiDGeluFp8 ? BN : 1];
    __shared__ uint32_t red[NW];
    auto epilogue = [&](auto full_tile) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tile)::value;
        auto in_rows = [&](int r) { return FULL || r < rows_in; };
        auto in_cols = [&](int c) { return FULL || c < cols_in; };

        if constexpr (EPI == kEpiDGeluFp8) {
            // Bring the tile of h into the ring in the bf16 staging layout (direct
            // loads, rows past M read as zero), then scale by gelu'(h) in place.
            using G = Staging<BN * 2, BM, STAGE>;
            static_assert(BM * G::P <= NS * G::RPS && G::UNITS % (64 * NW) == 0, "h staging");
            constexpr int IPW = G::UNITS / 64 / NW;    // 64-chunk loads per wave
            const int64_t rows_h = min<int64_t>(BM, M - m0);
            const __amdgpu_buffer_rsrc_t rsrc_h = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(p.h_in + m0 * N), (short)0, (int)(rows_h * N * 2), kBufferWord3);
#pragma unroll
            for (int jj = 0; jj < IPW; ++jj) {
                const int u0 = (wave * IPW + jj) * 64;
                int lr, byte;
                G::source(u0 + lane, lr, byte);
                const uint32_t voff = (uint32_t)(lr * N * 2 + n0 * 2 + byte);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_h, (lds_ptr)G::pos(ring, u0), 16, voff,
                                                         0, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
            // staged row starts of the wave's 32 x 32 blocks, once per block
            lds8* hrow[TM][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    hrow[i][j] = G::row(ring, (wn * WN + 32 * j) / 8 / G::NC, wm * WM + 32 * i);
            auto scale_by_dgelu = [&](auto erf) __attribute__((always_inline)) {
                constexpr bool ERF = decltype(erf)::value;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        // one 32 x 32 block at a time: without bounds branches the
                        // scheduler would otherwise load every h value up front and
                        // spill
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int lr = row_w + 32 * i;
                            const int lc = col_w + 32 * j + 8 * q;
                            const u32x2 hw = lds_ld<u32x2>(
                                G::in_row(hrow[i][j], fr, (wn * WN + 32 * j + 8 * q) / 8 % G::NC) +
                                8 * fh);
                            const bool ok = in_rows(lr) && in_cols(lc);
                            const float hv[4] = {bf16_lo(hw.x), bf16_hi(hw.x), bf16_lo(hw.y),
                                                 bf16_hi(hw.y)};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float gp = act_grad_f<ERF>(hv[e]);
                                float v = ok ? acc[j][i][4 * q + e] * alpha * gp : 0.0f;
                                // the product is formed here: the compiler would
                                // otherwise sink it to its uses past the barrier and
                                // keep (spill) both factors
                                asm volatile("" : "+v"(v));
                                acc[j][i][4 * q + e] = v;
                            }
                        }
                    }
            };
            if constexpr (ACT != 0) {
                scale_by_dgelu(std::integral_constant<bool, ACT == 2>{});
            } else {
                if (p.gelu_erf) scale_by_dgelu(std::true_type{});
                else scale_by_dgelu(std::false_type{});
            }
            __syncthreads();   // h is consumed: the ring takes the codes next
        } else {
            // alpha (and the bias) in place; values outside the product become 0
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cn = col_w + 32 * j + 8 * q;
                    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (EPI == kEpiBf16Bias || EPI == kEpiGeluFp8 || EPI == kEpiGeluBf16) {
                        if (p.bias && in_cols(cn)) {
                            const uint2 bw = *reinterpret_cast<const uint2*>(p.bias + n0 + cn);
                            bv[0] = bf16_lo(bw.x); bv[1] = bf16_hi(bw.x);
                            bv[2] = bf16_lo(bw.y); bv[3] = bf16_hi(bw.y);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const bool ok = in_rows(row_w + 32 * i) && in_cols(cn);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = acc[j][i][4 * q + e];
                            if constexpr (EPI == kEpiBf16Bias || EPI == kEpiGeluFp8 ||
                                          EPI == kEpiGeluBf16)
                                acc[j][i][4 * q + e] = ok ? fmaf(x, alpha, bv[e]) : 0.0f;
                            else
                                acc[j][i][4 * q + e] = ok ? x * alpha : 0.0f;
                        }
                    }
                }
        }

        if constexpr (EPI == kEpiDGeluF32 || EPI == kEpiDGeluBf16) {
            // gelu'(h) from global memory, one 8-byte read per four values (here the
            // per-value choice of the form measured faster than two loop copies)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t gm = m0 + row_w + 32 * i;
                        const int64_t gn = n0 + col_w + 32 * j + 8 * q;
                        if (in_rows(row_w + 32 * i) && in_cols(col_w + 32 * j + 8 * q)) {
                            const uint2 hw = *reinterpret_cast<const uint2*>(p.h_in + gm * N + gn);
                            const float hv[4] = {bf16_lo(hw.x), bf16_hi(hw.x), bf16_lo(hw.y),
                                                 bf16_hi(hw.y)};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[j][i][4 * q + e] *= p.gelu_erf ? gelu_erf_grad_f(hv[e])
                                                                   : gelu_grad_f(hv[e]);
                        }
                    }
        }

        if constexpr (EPI == kEpiF32 || EPI == kEpiDGeluF32) {
            // fp32 rows; a 256 x 256 tile goes out in two passes of 128 rows
            constexpr int P4 = staging_parts(BN * 4, STAGE);
            constexpr int CAP = NS * (STAGE / (BN * 4 / P4)) / P4;   // tile rows one pass holds
            constexpr int PASSES = (BM + CAP - 1) / CAP;
            constexpr int RPP = BM / PASSES;
            using G = Staging<BN * 4, RPP, STAGE>;
            static_assert(RPP * PASSES == BM && RPP % WM == 0 && RPP * G::P <= NS * G::RPS,
                          "f32 staging");
#pragma unroll
            for (int ps = 0; ps < PASSES; ++ps) {
                if (wm * WM >= ps * RPP && wm * WM < (ps + 1) * RPP) {
                    lds8* frow[TM][TN];
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            frow[i][j] = G::row(ring, (wn * WN + 32 * j) / 4 / G::NC,
                                                wm * WM + 32 * i - ps * RPP);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                lds_st(G::in_row(frow[i][j], fr,
                                                 (wn * WN + 32 * j + 8 * q) / 4 % G::NC + fh),
                                       f32x4{acc[j][i][4 * q], acc[j][i][4 * q + 1],
                                             acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]});
                            }
                }
                __syncthreads();
                G::template copy_out<NT, !FULL>(ring, t, (uint8_t*)p.out + ((m0 + ps * RPP) * N + n0) * 4,
                                             N * 4, M - m0 - ps * RPP, (N - n0) * 4);
                __syncthreads();
            }
        }

        // bf16 rows of the tile through the ring
        auto bf16_out = [&](uint16_t* dst) {
            using G = Staging<BN * 2, BM, STAGE>;
            static_assert(BM * G::P <= NS * G::RPS, "bf16 staging");
            lds8* brow[TM][TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    brow[i][j] = G::row(ring, (wn * WN + 32 * j) / 8 / G::NC, wm * WM + 32 * i);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        lds_st(G::in_row(brow[i][j], fr, (wn * WN + 32 * j + 8 * q) / 8 % G::NC) +
                                   8 * fh,
                               u32x2{pack_bf16x2(acc[j][i][4 * q], acc[j][i][4 * q + 1]),
                                     pack_bf16x2(acc[j][i][4 * q + 2], acc[j][i][4 * q + 3])});
                    }
            __syncthreads();
            G::template copy_out<NT, !FULL>(ring, t, (uint8_t*)(dst + m0 * N + n0), N * 2, M - m0,
                                        (N - n0) * 2);
            __syncthreads();
        };
        if constexpr (EPI == kEpiBf16Bias || EPI == kEpiGeluFp8 || EPI == kEpiGeluBf16) {
            uint16_t* hdst = EPI == kEpiBf16Bias ? (uint16_t*)p.out : p.h_out;
            if (hdst) bf16_out(hdst);
        }
        if constexpr (EPI == kEpiDGeluBf16) bf16_out((uint16_t*)p.out);
        // gelu in place on every accumulator (values outside the product are 0, and
        // gelu(0) = 0)
        auto apply_gelu = [&](auto erf) __attribute__((always_inline)) {
            constexpr bool ERF = decltype(erf)::value;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[j][i][r] = act_f<ERF>(acc[j][i][r]);
        };
        if constexpr (EPI == kEpiGeluBf16 || EPI == kEpiGeluFp8) {
            if constexpr (ACT != 0) {
                apply_gelu(std::integral_constant<bool, ACT == 2>{});
            } else {
                if (p.gelu_erf) apply_gelu(std::true_type{});
                else apply_gelu(std::false_type{});
            }
        }
        if constexpr (EPI == kEpiGeluBf16) bf16_out((uint16_t*)p.out);

        if constexpr (EPI == kEpiGeluFp8 || EPI == kEpiDGeluFp8) {
            // FP8 codes: first the row-major tile goes through the ring, then the
            // transposed one (rows = output columns).  For the transposed copy the
            // four lanes of a quad swap bytes so that each holds one column of four
            // consecutive rows, written as one word.
            using Q = Staging<BN, BM, STAGE>;
            using QT = Staging<BM, BN, STAGE>;
            static_assert(BM * Q::P <= NS * Q::RPS && BN * QT::P <= NS * QT::RPS, "code staging");
            static_assert(QT::P == 1, "transposed code rows are never cut");
            lds8* qrow[TM][TN];
            lds8* qtrow[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    qrow[i][j] = Q::row(ring, (wn * WN + 32 * j) / 16 / Q::NC, wm * WM + 32 * i);
                qtrow[j] = QT::row(ring, 0, wn * WN + 32 * j);
            }
            const float qs = *p.q_scale;
            uint32_t amax_bits = 0;
            uint32_t codes[TM][TN][4];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int lr = row_w + 32 * i;
                        const int lc = col_w + 32 * j + 8 * q;
                        float gs[4];
                        uint32_t cm = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float g;
                            if constexpr (EPI == kEpiGeluFp8) {
                                g = acc[j][i][4 * q + e];   // gelu(h), applied above
                                gs[e] = g * qs;
                            } else {
                                g = acc[j][i][4 * q + e];
                                gs[e] = mul_round_odd(g, qs);
                            }
                            const uint32_t ab = abs_bits(g);
                            cm = cm > ab ? cm : ab;
                        }
                        uint32_t code = encode4<QF>(gs[0], gs[1], gs[2], gs[3]);
                        if (__builtin_expect(cm > kInfBits, 0)) code = patch_nan4(code, gs);
                        if constexpr (EPI == kEpiGeluFp8) {
                            // rows and columns outside the product carry gelu(0) = 0
                            if (!(in_rows(lr) && in_cols(lc))) cm = 0;
                        }
                        amax_bits = amax_bits > cm ? amax_bits : cm;
                        codes[i][j][q] = code;
                        lds_st(Q::in_row(qrow[i][j], fr, (wn * WN + 32 * j + 8 * q) / 16 % Q::NC) +
                                   4 * ((lc / 4) % 4),
                               code);
                    }
            __syncthreads();
            Q::template copy_out<NT, !FULL>(ring, t, p.q_out + m0 * N + n0, N, M - m0, N - n0);
            if (p.q_out_t) {
                __syncthreads();
                const bool odd = fr & 1, hi2 = fr & 2;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t code = codes[i][j][q];
                            const uint32_t o2 = (uint32_t)__builtin_amdgcn_mov_dpp(
                                (int)code, kDppQuadSwap2, 0xF, 0xF, false);
                            const uint32_t c2 = hi2 ? __builtin_amdgcn_perm(o2, code, 0x03020706u)
                                                    : __builtin_amdgcn_perm(o2, code, 0x05040100u);
                            const uint32_t o1 = (uint32_t)__builtin_amdgcn_mov_dpp(
                                (int)c2, kDppQuadSwap1, 0xF, 0xF, false);
                            const uint32_t ct = odd ? __builtin_amdgcn_perm(o1, c2, 0x03070105u)
                                                    : __builtin_amdgcn_perm(o1, c2, 0x06020400u);
                            const int tm = (row_w + 32 * i) & ~3;              // first of four rows
                            lds_st(QT::in_row(qtrow[j], 8 * q + 4 * fh + (fr & 3),
                                              (wm * WM + 32 * i) / 16 + (fr >> 4)) +
                                       4 * ((tm / 4) % 4),
                                   ct);
                        }
                __syncthreads();
                QT::template copy_out<NT, !FULL>(ring, t, p.q_out_t + n0 * M + m0, M, N - n0, M - m0);
            }
            if constexpr (EPI == kEpiDGeluFp8) {
                if (p.col_partial) {
                    // column sums of the tile in a fixed order: over i in a lane, a
                    // butterfly over the 32 lanes of equal lane / 32, then over wm
                    constexpr int NV = 16 * TN;   // columns per lane
                    float v[NV];
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            float a = 0.0f;
#pragma unroll
                            for (int i = 0; i < TM; ++i) a += acc[j][i][r];
                            v[16 * j + r] = a;
                        }
                    butterfly_sum<NV>(v, fr);
#pragma unroll
                    for (int k = 0; k < NV / 32; ++k) {
                        const int c = fr * (NV / 32) + k;   // = 16 j + 4 q + e
                        const int j = c / 16, q = (c / 4) % 4, e = c % 4;
                        colp[wm][col_w + 32 * j + 8 * q + e] = v[k];
                    }
                    __syncthreads();
                    if (t < BN && in_cols(t)) {
                        float a = 0.0f;
#pragma unroll
                        for (int w = 0; w < WGM; ++w) a += colp[w][t];
                        p.col_partial[(int64_t)tile_m * N + n0 + t] = a;
                    }
                }
            }
            block_amax_atomic<false>(amax_bits, p.q_amax, red);
        }
    };
    epilogue(std::integral_constant<bool, FULLX>{});
}

// 256 x 256 tiles, eight waves of 64 x 128 (two waves per SIMD), one workgroup
// per CU.
template <int FA, int FB, int EPI, int QF>
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(512)
void gemm_kernel_256(GemmParams p) {
    gemm_tile<256, 256, 4, 2, 4, FA, FB, EPI, QF>(p, blockIdx.x);
}

// 128 x 256 tiles, four waves of 64 x 128 and a three-stage ring (72 KB), so two
// workgroups share a CU and one's epilogue overlaps the other's main loop.
template <int FA, int FB, int EPI, int QF>
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(256)
void gemm_kernel_128x256(GemmParams p) {
    gemm_tile<128, 256, 2, 2, 3, FA, FB, EPI, QF>(p, blockIdx.x);
}

// 128 x 128 tiles, four waves of 64 x 64, two workgroups per CU.
template <int FA, int FB, int EPI, int QF>
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(256)
void gemm_kernel_128(GemmParams p) {
    gemm_tile<128, 128, 2, 2, 4, FA, FB, EPI, QF>(p, blockIdx.x);
}

// 64 x 64 tiles, four waves of 32 x 32, up to four workgroups per CU: for
// problems that leave most CUs idle even with 128 x 128 tiles.
template <int FA, int FB, int EPI, int QF>
__global__ __attribute__((amdgpu_waves_per_eu(4, 4))) __launch_bounds__(256)
void gemm_kernel_64(GemmParams p) {
    gemm_tile<64, 64, 2, 2, 4, FA, FB, EPI, QF>(p, blockIdx.x);
}

// Up to kMaxGemmGroup independent small fp32-output products in one launch:
// blocks [start[k], start[k + 1]) are the tiles of product k, each computed
// exactly as the kernel of that tile shape computes it alone.  Small problems leave
// most CUs idle one by one; side by side their tiles share the GPU and their
// launch latencies overlap.
struct GemmGroup {
    GemmParams p[kMaxGemmGroup];
    int start[kMaxGemmGroup + 1];
};

template <int FA, int FB>
__global__ __attribute__((amdgpu_waves_per_eu(4, 4))) __launch_bounds__(256)
void gemm_kernel_64_group(GemmGroup g) {
    const int b = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int j = 1; j < kMaxGemmGroup; ++j) k += b >= g.start[j];
    gemm_tile<64, 64, 2, 2, 4, FA, FB, kEpiF32, kE4M3, true>(g.p[k], b - g.start[k]);
}

// The same on 128 x 128 tiles (half the LDS traffic per MFMA of 64 x 64 tiles),
// when the grouped products together have enough of them to occupy the CUs.
template <int FA, int FB>
__global__ __attribute__((amdgpu_waves_per_eu(2, 2))) __launch_bounds__(256)
void gemm_kernel_128_group(GemmGroup g) {
    const int b = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int j = 1; j < kMaxGemmGroup; ++j) k += b >= g.start[j];
    gemm_tile<128, 128, 2, 2, 4, FA, FB, kEpiF32, kE4M3, true>(g.p[k], b - g.start[k]);
}

enum TileShape { kTile256, kTile128x256, kTile128, kTile64 };

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Large problems: with K up to 2048 the epilogue is a large share of a tile's
// time, and two 128 x 256 workgroups per CU hide one's epilogue behind the
// other's main loop; with longer K the 256 x 256 tile's lower LDS and L2
// traffic per MFMA wins.  The plain epilogues (fp32 or bf16 + bias out) are
// short enough that the 256 x 256 tile already wins at K = 2048 (16384 x 8192
// x 2048, fp32 out: 314 against 330 us); the GELU and GELU' epilogues measured
// faster on 128 x 256 there.  Smaller problems take 128 x 128 tiles, and 64 x 64
// tiles when even those would leave most CUs idle (the fused dH epilogue needs
// at least 64 columns per wave, so it stays on 128 x 128).
TileShape pick_tile(int64_t M, int64_t N, int64_t K, int epi) {
    const bool light = epi == kEpiF32 || epi == kEpiBf16Bias;
    const bool long_k = light ? K >= 2048 : K > 2048;
    if (long_k && cdiv(M, 256) * cdiv(N, 256) >= 256) return kTile256;
    if (cdiv(M, 128) * cdiv(N, 256) >= 512) return kTile128x256;
    if (epi == kEpiDGeluFp8 || cdiv(M, 128) * cdiv(N, 128) >= 128) return kTile128;
    return kTile64;
}

template <int FA, int FB, int EPI, int QF>
hipError_t launch_typed(const GemmParams& p, hipStream_t stream) {
    switch (pick_tile(p.M, p.N, p.K, EPI % 16)) {
        case kTile256:
            hipLaunchKernelGGL((gemm_kernel_256<FA, FB, EPI, QF>),
                               dim3((unsigned)(cdiv(p.M, 256) * cdiv(p.N, 256))), dim3(512), 0,
                               stream, p);
            break;
        case kTile128x256:
            // the FP8-output epilogues (the longest) without bounds tests where
            // every tile is whole
            if constexpr (EPI % 16 == kEpiGeluFp8 || EPI % 16 == kEpiDGeluFp8) {
                if (p.M % 128 == 0 && p.N % 256 == 0) {
                    hipLaunchKernelGGL((gemm_kernel_128x256<FA, FB, EPI + 64, QF>),
                                       dim3((unsigned)(p.M / 128 * (p.N / 256))), dim3(256), 0,
                                       stream, p);
                    break;
                }
            }
            hipLaunchKernelGGL((gemm_kernel_128x256<FA, FB, EPI, QF>),
                               dim3((unsigned)(cdiv(p.M, 128) * cdiv(p.N, 256))), dim3(256), 0,
                               stream, p);
            break;
        case kTile64:
            if constexpr (EPI % 16 != kEpiDGeluFp8) {
                hipLaunchKernelGGL((gemm_kernel_64<FA, FB, EPI, QF>),
                                   dim3((unsigned)(cdiv(p.M, 64) * cdiv(p.N, 64))), dim3(256), 0,
                                   stream, p);
                break;
            }
            [[fallthrough]];
        default:
            hipLaunchKernelGGL((gemm_kernel_128<FA, FB, EPI, QF>),
                               dim3((unsigned)(cdiv(p.M, 128) * cdiv(p.N, 128))), dim3(256), 0,
                               stream, p);
    }
    return hipGetLastError();
}

// The GELU form as a compile-time part of the epilogue (epilogue + 16 for tanh,
// + 32 for erf) where a runtime choice would spill.
template <int FA, int FB, int EPI, int QF>
hipError_t launch_act(const GemmParams& p, hipStream_t stream) {
    return p.gelu_erf ? launch_typed<FA, FB, EPI + 32, QF>(p, stream)
                      : launch_typed<FA, FB, EPI + 16, QF>(p, stream);
}

template <int FA, int FB>
hipError_t launch_epi(const GemmParams& p, hipStream_t stream) {
    switch (p.epilogue) {
        case kEpiBf16Bias: return launch_typed<FA, FB, kEpiBf16Bias, kE4M3>(p, stream);
        case kEpiF32: return launch_typed<FA, FB, kEpiF32, kE4M3>(p, stream);
        case kEpiDGeluF32: return launch_typed<FA, FB, kEpiDGeluF32, kE4M3>(p, stream);
        case kEpiGeluFp8:
            return p.q_fp8 == kE4M3 ? launch_act<FA, FB, kEpiGeluFp8, kE4M3>(p, stream)
                                    : launch_act<FA, FB, kEpiGeluFp8, kE5M2>(p, stream);
        case kEpiDGeluFp8:
            return p.q_fp8 == kE4M3 ? launch_act<FA, FB, kEpiDGeluFp8, kE4M3>(p, stream)
                                    : launch_act<FA, FB, kEpiDGeluFp8, kE5M2>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

// Groups of small fp32-output products (see gemm_kernel_64_group): tile128
// picks the 128 x 128 kernel, total is the number of tiles of all products.
template <int FA, int FB>
hipError_t launch_group_typed(const GemmGroup& g, bool tile128, int total, hipStream_t stream) {
    if (tile128)
        hipLaunchKernelGGL((gemm_kernel_128_group<FA, FB>), dim3(total), dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_kernel_64_group<FA, FB>), dim3(total), dim3(256), 0, stream, g);
    return hipGetLastError();
}

}  // namespace

// One operand format pair's launchers (defined in gemm_<a>_<b>.hip).
#define FP8LN_GEMM_PAIR_DECL(NAME)                                                     \
    hipError_t launch_gemm_##NAME(const GemmParams& p, hipStream_t stream);            \
    hipError_t launch_group_##NAME(const GemmParams* ps, const int* start, bool tile128, \
                                   int total, hipStream_t stream);
FP8LN_GEMM_PAIR_DECL(e4m3_e4m3)
FP8LN_GEMM_PAIR_DECL(e5m2_e4m3)
FP8LN_GEMM_PAIR_DECL(e4m3_e5m2)
FP8LN_GEMM_PAIR_DECL(e5m2_e5m2)
#undef FP8LN_GEMM_PAIR_DECL
hipError_t launch_gemm_bf16_ops(const GemmParams& p, hipStream_t stream);

#define FP8LN_GEMM_PAIR_DEFINE(A, B, NAME)                                                \
    hipError_t launch_gemm_##NAME(const GemmParams& p, hipStream_t stream) {              \
        return launch_epi<A, B>(p, stream);                                               \
    }                                                                                     \
    hipError_t launch_group_##NAME(const GemmParams* ps, const int* start, bool tile128,  \
                                   int total, hipStream_t stream) {                       \
        GemmGroup g{};                                                                    \
        for (int k = 0; k < kMaxGemmGroup; ++k) g.p[k] = ps[k];                           \
        for (int k = 0; k <= kMaxGemmGroup; ++k) g.start[k] = start[k];                   \
        return launch_group_typed<A, B>(g, tile128, total, stream);                       \
    }

}  // namespace fp8ln
