// Host-side dispatch of the GEMM launches: tile-row counts, size checks,
// grouping of small backward products, and the choice of the operand format
// pair's launcher (the kernels live in gemm_kernels.hpp, compiled per pair).
#include "gemm_kernels.hpp"

namespace fp8ln {

int64_t gemm_partial_rows(int64_t M, int64_t N, int64_t K) {
    return pick_tile(M, N, K, kEpiDGeluFp8) == kTile256 ? cdiv(M, 256) : cdiv(M, 128);
}

static bool gemm_fits(const GemmParams& p);

hipError_t launch_gemm_group(const GemmParams* ps, int n, hipStream_t stream) {
    for (int k = 0; k < n; ++k)
        if (!gemm_fits(ps[k])) return hipErrorInvalidValue;
    bool grouped = n >= 2 && n <= kMaxGemmGroup;
    int64_t tiles128 = 0;
    for (int k = 0; grouped && k < n; ++k) {
        const GemmParams& q = ps[k];
        const TileShape ts = q.M > 0 && q.N > 0 ? pick_tile(q.M, q.N, q.K, kEpiF32) : kTile256;
        grouped = q.epilogue == kEpiF32 && q.a_fp8 == ps[0].a_fp8 && q.b_fp8 == ps[0].b_fp8 &&
                  q.a_fp8 != kOpBf16 && q.b_fp8 != kOpBf16 && (ts == kTile64 || ts == kTile128);
        tiles128 += cdiv(q.M, 128) * cdiv(q.N, 128);
    }
    if (!grouped) {
        for (int k = 0; k < n; ++k) {
            const hipError_t e = launch_gemm(ps[k], stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // 128 x 128 tiles once the group has enough of them for half the CUs
    // (the single-product rule asks that of one product alone)
    const int bt = tiles128 >= 128 ? 128 : 64;
    GemmParams gp[kMaxGemmGroup] = {};
    int start[kMaxGemmGroup + 1];
    int total = 0;
    for (int k = 0; k < kMaxGemmGroup; ++k) {
        start[k] = total;
        if (k < n) {
            gp[k] = ps[k];
            total += (int)(cdiv(ps[k].M, bt) * cdiv(ps[k].N, bt));
        }
    }
    start[kMaxGemmGroup] = total;
    const int fa = ps[0].a_fp8, fb = ps[0].b_fp8;
    const bool t128 = bt == 128;
    if (fa == kE4M3 && fb == kE4M3) return launch_group_e4m3_e4m3(gp, start, t128, total, stream);
    if (fa == kE5M2 && fb == kE4M3) return launch_group_e5m2_e4m3(gp, start, t128, total, stream);
    if (fa == kE4M3 && fb == kE5M2) return launch_group_e4m3_e5m2(gp, start, t128, total, stream);
    return launch_group_e5m2_e5m2(gp, start, t128, total, stream);
}

// The tiles' 32-bit buffer offsets (see gemm_tile): K bytes and the h rows of
// the GELU' epilogues must keep a 256-row tile below 2^31 bytes.
static bool gemm_fits(const GemmParams& p) {
    constexpr int64_t kMaxRowBytes = 2147483647 / 256;
    const int64_t kb = (p.a_fp8 == kOpBf16 ? 2 : 1) * p.K;
    const bool reads_h = p.epilogue == kEpiDGeluF32 || p.epilogue == kEpiDGeluFp8 ||
                         p.epilogue == kEpiDGeluBf16;
    return kb <= kMaxRowBytes && (!reads_h || 2 * p.N <= kMaxRowBytes);
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    if (!gemm_fits(p)) return hipErrorInvalidValue;
    if (p.a_fp8 == kOpBf16 || p.b_fp8 == kOpBf16) {
        if (p.a_fp8 != p.b_fp8) return hipErrorInvalidValue;
        return launch_gemm_bf16_ops(p, stream);
    }
    if (p.a_fp8 == kE4M3 && p.b_fp8 == kE4M3) return launch_gemm_e4m3_e4m3(p, stream);
    if (p.a_fp8 == kE5M2 && p.b_fp8 == kE4M3) return launch_gemm_e5m2_e4m3(p, stream);
    if (p.a_fp8 == kE4M3 && p.b_fp8 == kE5M2) return launch_gemm_e4m3_e5m2(p, stream);
    return launch_gemm_e5m2_e5m2(p, stream);
}

}  // namespace fp8ln
