// The FP8 tensor cast's per-tile work as a device function (cast with amax,
// optional transposed copy and column sums), for the cast kernel and for
// launches that run it beside other jobs.  The cast scales with a round-to-odd
// product, so its codes are those of the exact value * scale.
//
// Autocast casts the operands of the linear layers to FP8 with the delayed
// scale and hands gradients back in higher precision ("Turbo-charging your
// transformer training", "Playing with lower-precision formats: BF16 vs FP8";
// HYBRID: E4M3 forward, E5M2 gradients).  The transposed copy exists because the
// backward's GEMMs contract over the other index (dgrad over output features,
// wgrad over tokens) and the GEMM reads operands with the contraction index last.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

constexpr int kCT = 128;            // rows and columns of one cast tile
constexpr int kCPitch = kCT + 4;    // byte pitch of the cast kernel's transposed codes

// A workgroup of NT threads casts 128 x 128 tiles, looping over them with the
// grid sized to what the CUs hold at once; the next tile's loads go out before
// the current tile is processed, so every workgroup keeps a tile's reads in
// flight.  Thread t owns columns 8 (t % 16) .. +7 of rows 4 (t / 16) .. +3 of
// each NT / 4-row band of a tile (two bands for 256 threads, one for 512), so
// each row is read and written by 16 consecutive lanes as one contiguous
// segment.  For the transposed copy a thread packs the codes of its four
// consecutive rows of one column into a word in LDS; the tile then leaves as
// full 128-byte rows of the transposed output.  Column sums of a tile (for the
// bias gradient) are formed in a fixed order: a thread's rows, then the
// threads of a column in order of t / 16.  512-thread workgroups halve the
// per-tile latency of tensors with few tiles (a weight of a few MB leaves most
// CUs idle, and each tile's arithmetic is then on the critical path).
// Workgroup `vblock` of `vgrid` (the kernel's own grid, or a share of a larger
// launch that also runs other jobs).  `pre` runs once the first tile is in
// flight and before *scale_ptr and *copy_src are read (all threads call it).
// CHECK: as block_amax_atomic's.
template <bool IN_F32, int FMT, int NT, bool CHECK = true, class Pre = NoPre>
__device__ __forceinline__ void cast_tiles(
    const void* __restrict__ in, int64_t rows, int64_t cols, const float* scale_ptr,
    float* __restrict__ amax_ptr, uint8_t* __restrict__ out, uint8_t* __restrict__ out_t,
    float* __restrict__ partial, const float* copy_src, float* __restrict__ copy_dst,
    int vblock, int vgrid, Pre pre = {}) {
    __shared__ uint32_t tq[kCT * kCPitch / 4];
    constexpr int BANDS = 512 / NT;     // 128-row tile = BANDS bands of NT / 4 rows
    constexpr int RPT = 4 * BANDS;      // rows per thread
    __shared__ float psum[NT / 16][kCT];
    __shared__ uint32_t red[NT / kWave];
    const int t = threadIdx.x;
    const int j = t % 16;
    const int p = t / 16;
    const int tiles_x = (int)((cols + kCT - 1) / kCT);
    const int tiles = tiles_x * (int)((rows + kCT - 1) / kCT);

    typedef typename std::conditional<IN_F32, float4, uint4>::type Raw;
    constexpr int RPR = IN_F32 ? 2 : 1;   // 16-byte loads per row segment of 8 values
    Raw raw[RPT][RPR];
    // the thread's row segments of tile `tile` (zeros outside the tensor)
    auto load_tile = [&](int tile) {
        const int64_t r0 = (int64_t)(tile / tiles_x) * kCT;
        const int64_t c0 = (int64_t)(tile % tiles_x) * kCT + 8 * j;
        const bool col_ok = tile < tiles && c0 < cols;   // cols % 16 == 0: all in or all out
#pragma unroll
        for (int h = 0; h < RPT; ++h) {
            const int64_t r = r0 + (NT / 4) * (h / 4) + 4 * p + (h % 4);
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
    load_tile(vblock);
    pre();
    const float s = *scale_ptr;
    if (copy_dst && vblock == 0 && threadIdx.x == 0) *copy_dst = *copy_src;
    for (int tile = vblock; tile < tiles; tile += vgrid) {
        const int64_t r0 = (int64_t)(tile / tiles_x) * kCT;
        const int64_t c0 = (int64_t)(tile % tiles_x) * kCT + 8 * j;
        const bool col_ok = c0 < cols;
        Raw cur[RPT][RPR];
#pragma unroll
        for (int h = 0; h < RPT; ++h)
#pragma unroll
            for (int k = 0; k < RPR; ++k) cur[h][k] = raw[h][k];
        load_tile(tile + vgrid);   // in flight while this tile is processed

        float cs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = 0.0f;
#pragma unroll
        for (int half = 0; half < BANDS; ++half) {
            uint32_t packed[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) packed[e] = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = r0 + (NT / 4) * half + 4 * p + i;
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
                    tq[(8 * j + e) * (kCPitch / 4) + (NT / 16) * half + p] = packed[e];
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
            for (int k = 0; k < 8 * kCT / NT; ++k) {
                const int cc = t / 8 + (NT / 8) * k;
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
                for (int k = 0; k < NT / 16; ++k) acc += psum[k][t];
                partial[(int64_t)(tile / tiles_x) * cols + pc] = acc;
            }
        }
        __syncthreads();   // tq and psum are rewritten by the next tile
    }
    block_amax_atomic<CHECK>(cm, amax_ptr, red);
}

}  // namespace fp8ln
