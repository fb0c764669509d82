// C-ABI entry points: argument validation, workspace carving and the order of
// kernel launches for each fused module step.  Nothing here computes; every step
// of the path runs in the gfx950 kernels behind launchers.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/fp8ln.h"
#include "launchers.hpp"

using namespace fp8ln;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return FP8LN_OK;
    return fail(FP8LN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FP8LN_TRY(expr, what)                       \
    do {                                            \
        int _s = hip_status((expr), (what));        \
        if (_s != FP8LN_OK) return _s;              \
    } while (0)

// Per-device gfx950 check, cached (0 unknown, 1 yes, 2 no).
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

int device_supported(int device, std::string* why) {
    if (device < 0 || device >= kMaxDevices) {
        if (why) *why = "device index out of range";
        return 0;
    }
    int cached = g_dev_ok[device].load();
    if (cached == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
            if (why) *why = "hipGetDeviceProperties failed";
            return 0;
        }
        cached = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_ok[device].store(cached);
        if (cached == 2 && why) *why = std::string("device architecture ") + prop.gcnArchName +
                                       " is not gfx950";
    }
    if (cached == 2 && why && why->empty()) *why = "device architecture is not gfx950";
    return cached == 1;
}

int check_current_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    std::string why;
    if (!device_supported(dev, &why)) return fail(FP8LN_ERR_UNSUPPORTED, "%s", why.c_str());
    return FP8LN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_recipe(const fp8ln_recipe* r) {
    if (!r) return fail(FP8LN_ERR_INVALID_ARG, "recipe is NULL");
    if (r->format < FP8LN_FORMAT_E4M3 || r->format > FP8LN_FORMAT_E5M2)
        return fail(FP8LN_ERR_INVALID_ARG, "recipe.format %d is not E4M3/HYBRID/E5M2", r->format);
    if (r->amax_history_len < 1 || r->amax_history_len > 1024)
        return fail(FP8LN_ERR_INVALID_ARG, "recipe.amax_history_len %d outside 1..1024",
                    r->amax_history_len);
    if (r->margin < 0 || r->margin > 64)
        return fail(FP8LN_ERR_INVALID_ARG, "recipe.margin %d outside 0..64", r->margin);
    if (!(std::isfinite(r->ln_eps) && r->ln_eps > 0.0f))
        return fail(FP8LN_ERR_INVALID_ARG, "recipe.ln_eps must be finite and > 0");
    if (r->activation != FP8LN_GELU_TANH && r->activation != FP8LN_GELU_ERF)
        return fail(FP8LN_ERR_INVALID_ARG, "recipe.activation %d is not GELU_TANH/GELU_ERF",
                    r->activation);
    return FP8LN_OK;
}

int check_meta(const fp8ln_meta* m, int min_slots, int kind, const char* name) {
    if (!m) return fail(FP8LN_ERR_INVALID_ARG, "%s meta is NULL", name);
    if (!m->amax_history || !m->scale || !m->scale_inv)
        return fail(FP8LN_ERR_INVALID_ARG, "%s meta has a NULL buffer", name);
    if (m->n_slots < 1 || m->n_slots > 8)
        return fail(FP8LN_ERR_INVALID_ARG, "%s meta n_slots %d outside 1..8", name, m->n_slots);
    if (m->n_slots < min_slots)
        return fail(FP8LN_ERR_INVALID_ARG, "%s meta needs %d slots, has %d", name, min_slots,
                    m->n_slots);
    if (m->kind != FP8LN_META_FORWARD && m->kind != FP8LN_META_BACKWARD)
        return fail(FP8LN_ERR_INVALID_ARG, "%s meta kind %d invalid", name, m->kind);
    if (kind >= 0 && m->kind != kind)
        return fail(FP8LN_ERR_INVALID_ARG, "%s meta has the wrong kind", name);
    return FP8LN_OK;
}

// FP8 encoding of the tensors a state block covers.
int meta_fp8(const fp8ln_recipe* r, int kind) {
    if (r->format == FP8LN_FORMAT_E4M3) return kE4M3;
    if (r->format == FP8LN_FORMAT_E5M2) return kE5M2;
    return kind == FP8LN_META_FORWARD ? kE4M3 : kE5M2;   // HYBRID
}

float fp8_max_of(int fp8) { return fp8 == kE4M3 ? 448.0f : 57344.0f; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive 256-byte aligned pieces out of a workspace.
struct Carver {
    uint8_t* base;
    size_t used = 0;
    void* take(size_t bytes) {
        void* p = base ? base + used : nullptr;
        used += align_up(bytes);
        return p;
    }
};

#define REQUIRE(cond, ...)                                      \
    do {                                                        \
        if (!(cond)) return fail(FP8LN_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, "%s is NULL", #p)
#define REQUIRE_ALIGNED(p) REQUIRE(aligned16(p), "%s is not 16-byte aligned", #p)

// Size limits of one GEMM product C[M][N] = A[M][K] . B[N][K]^T.  The tiles read
// each operand tile (up to kGemmTileRows rows of K elements) and the fused
// GELU' epilogue's h tile (up to kGemmTileRows rows of N bf16 values) through a
// buffer descriptor with a 32-bit record count and 32-bit offsets, and offsets
// at 2^31 stand for "past the tile" (read as zero), so a tile must span fewer
// than 2^31 bytes: K * element bytes <= 8388607 (about 2^23), N <= 4194303 when
// h is read.  The launch grid counts tiles in 32 bits, so M and N are bounded
// too (at most 2^22 tiles of 64 x 64).
constexpr int64_t kGemmTileRows = 256;
constexpr int64_t kGemmTileBytes = 2147483647;   // INT32_MAX
constexpr int64_t kGemmMaxTiles64 = int64_t(1) << 22;
constexpr int64_t kGemmMaxDim = int64_t(1) << 36;

int check_gemm_size(int64_t M, int64_t N, int64_t K, int64_t elem_bytes, bool reads_h,
                    const char* what) {
    if (M > kGemmMaxDim || N > kGemmMaxDim || K > kGemmMaxDim)
        return fail(FP8LN_ERR_UNSUPPORTED, "%s: a dimension exceeds 2^36", what);
    if (K * elem_bytes > kGemmTileBytes / kGemmTileRows)
        return fail(FP8LN_ERR_UNSUPPORTED,
                    "%s: contraction length %lld (%lld bytes per row) exceeds the %lld-byte "
                    "rows that 32-bit tile offsets allow",
                    what, (long long)K, (long long)(K * elem_bytes),
                    (long long)(kGemmTileBytes / kGemmTileRows));
    if (reads_h && N * 2 > kGemmTileBytes / kGemmTileRows)
        return fail(FP8LN_ERR_UNSUPPORTED, "%s: h rows of %lld bf16 values exceed 32-bit offsets",
                    what, (long long)N);
    if (((M + 63) / 64) * ((N + 63) / 64) > kGemmMaxTiles64)
        return fail(FP8LN_ERR_UNSUPPORTED, "%s: %lld x %lld output exceeds 2^22 tiles of 64 x 64",
                    what, (long long)M, (long long)N);
    return FP8LN_OK;
}

// The transposition kernels take one 64-row tile per grid row (grid y < 65536).
constexpr int64_t kMaxTransposeRows = int64_t(65535) * 64;

int check_transpose_rows(int64_t rows, const char* what) {
    if (rows > kMaxTransposeRows)
        return fail(FP8LN_ERR_UNSUPPORTED, "%s: %lld rows exceed the %lld a transposed copy allows",
                    what, (long long)rows, (long long)kMaxTransposeRows);
    return FP8LN_OK;
}

#define CHECK(expr)                 \
    do {                            \
        int _c = (expr);            \
        if (_c != FP8LN_OK) return _c; \
    } while (0)

struct LinearWs {
    uint8_t* dy_q;
    uint8_t* dy_qt;
    float* dln;
    void* cast_ws;
    void* ln_ws;
    size_t bytes;
};

LinearWs linear_ws(void* base, int64_t M, int64_t K, int64_t N) {
    Carver c{(uint8_t*)base};
    LinearWs w;
    w.dy_q = (uint8_t*)c.take((size_t)(M * N));
    w.dy_qt = (uint8_t*)c.take((size_t)(M * N));
    w.dln = (float*)c.take((size_t)(M * K) * sizeof(float));
    w.cast_ws = c.take(cast_workspace(M, N));
    w.ln_ws = c.take(ln_bwd_workspace(M, (int)K));
    w.bytes = c.used;
    return w;
}

size_t dgelu_workspace(int64_t M, int64_t N) {
    return (size_t)gemm_partial_rows_bound(M) * (size_t)N * sizeof(float);
}

struct LinearOnlyWs {
    uint8_t* dy_q;
    uint8_t* dy_qt;
    void* cast_ws;
    size_t bytes;
};

LinearOnlyWs linear_only_ws(void* base, int64_t M, int64_t K, int64_t N) {
    Carver c{(uint8_t*)base};
    LinearOnlyWs w;
    w.dy_q = (uint8_t*)c.take((size_t)(M * N));
    w.dy_qt = (uint8_t*)c.take((size_t)(M * N));
    w.cast_ws = c.take(cast_workspace(M, N));
    (void)K;
    w.bytes = c.used;
    return w;
}

// BF16 LayerNormLinear backward: transposed dy, LN output and weight, fp32 dLN.
struct LinearBf16Ws {
    void* dy_t;      // bf16 [N][M]
    void* ln_t;      // bf16 [K][M]
    void* w_t;       // bf16 [K][N]
    float* dln;      // fp32 [M][K]
    void* sum_ws;    // column-sum partials of dy
    void* ln_ws;
    size_t bytes;
};

LinearBf16Ws linear_bf16_ws(void* base, int64_t M, int64_t K, int64_t N) {
    Carver c{(uint8_t*)base};
    LinearBf16Ws w;
    w.dy_t = c.take((size_t)(M * N) * 2);
    w.ln_t = c.take((size_t)(M * K) * 2);
    w.w_t = c.take((size_t)(K * N) * 2);
    w.dln = (float*)c.take((size_t)(M * K) * sizeof(float));
    w.sum_ws = c.take(transpose_b16_workspace(M, N));
    w.ln_ws = c.take(ln_bwd_workspace(M, (int)K));
    w.bytes = c.used;
    return w;
}

// BF16 LayerNormMLP backward: transposed operands, bf16 dH, fp32 dLN.
struct MlpBf16Ws {
    void* dy_t;      // [H][M]
    void* g_t;       // [F][M]
    void* w2_t;      // [F][H]
    void* w1_t;      // [H][F]
    void* ln_t;      // [H][M]
    void* dh;        // [M][F]
    void* dh_t;      // [F][M]
    float* dln;      // fp32 [M][H]
    void* sum_ws;
    void* ln_ws;
    size_t bytes;
};

MlpBf16Ws mlp_bf16_ws(void* base, int64_t M, int64_t H, int64_t F) {
    Carver c{(uint8_t*)base};
    MlpBf16Ws w;
    w.dy_t = c.take((size_t)(M * H) * 2);
    w.g_t = c.take((size_t)(M * F) * 2);
    w.w2_t = c.take((size_t)(H * F) * 2);
    w.w1_t = c.take((size_t)(H * F) * 2);
    w.ln_t = c.take((size_t)(M * H) * 2);
    w.dh = c.take((size_t)(M * F) * 2);
    w.dh_t = c.take((size_t)(M * F) * 2);
    w.dln = (float*)c.take((size_t)(M * H) * sizeof(float));
    w.sum_ws = c.take(std::max(transpose_b16_workspace(M, H), transpose_b16_workspace(M, F)));
    w.ln_ws = c.take(ln_bwd_workspace(M, (int)H));
    w.bytes = c.used;
    return w;
}

struct MlpWs {
    uint8_t* dy_q;
    uint8_t* dy_qt;
    float* dh_part;   // column sums of dH per GEMM tile row
    uint8_t* dh_q;
    uint8_t* dh_qt;
    float* dln;
    void* cast_ws;
    void* ln_ws;
    size_t bytes;
};

MlpWs mlp_ws(void* base, int64_t M, int64_t H, int64_t F) {
    Carver c{(uint8_t*)base};
    MlpWs w;
    w.dy_q = (uint8_t*)c.take((size_t)(M * H));
    w.dy_qt = (uint8_t*)c.take((size_t)(M * H));
    w.dh_part = (float*)c.take(dgelu_workspace(M, F));
    w.dh_q = (uint8_t*)c.take((size_t)(M * F));
    w.dh_qt = (uint8_t*)c.take((size_t)(M * F));
    w.dln = (float*)c.take((size_t)(M * H) * sizeof(float));
    w.cast_ws = c.take(cast_workspace(M, H));
    w.ln_ws = c.take(ln_bwd_workspace(M, (int)H));
    w.bytes = c.used;
    return w;
}

int check_bf16_module(int64_t M, int64_t K, int64_t N, float eps) {
    REQUIRE(M >= 0, "tokens < 0");
    REQUIRE(eps > 0.0f && eps <= 3.402823466e38f, "eps must be a positive finite number");
    if (K <= 0 || K % 16 != 0 || K > 8192)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld must be a multiple of 16 in 16..8192",
                    (long long)K);
    if (N <= 0 || N % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "output width %lld must be a positive multiple of 16",
                    (long long)N);
    return FP8LN_OK;
}

GemmParams gemm_params(int64_t M, int64_t N, int64_t K, const uint8_t* A, int afmt,
                       const uint8_t* B, int bfmt, const float* sa, const float* sb,
                       int epilogue) {
    GemmParams p;
    std::memset(&p, 0, sizeof(p));
    p.M = M; p.N = N; p.K = K;
    p.A = A; p.B = B;
    p.a_fp8 = afmt; p.b_fp8 = bfmt;
    p.sinv_a = sa; p.sinv_b = sb;
    p.epilogue = epilogue;
    return p;
}

}  // namespace

namespace fp8ln {
int report_error(int status, const char* message) { return fail(status, "%s", message); }
}  // namespace fp8ln

extern "C" {

const char* fp8ln_status_string(int status) {
    switch (status) {
        case FP8LN_OK: return "ok";
        case FP8LN_ERR_INVALID_ARG: return "invalid argument";
        case FP8LN_ERR_UNSUPPORTED: return "unsupported";
        case FP8LN_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* fp8ln_last_error(void) { return g_last_error.c_str(); }

int fp8ln_check_support(int device, char* reason, size_t reason_cap) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    std::string why;
    int ok = 0;
    if (e != hipSuccess) why = std::string("no HIP device: ") + hipGetErrorString(e);
    else if (device < 0 || device >= count) why = "device index out of range";
    else ok = device_supported(device, &why);
    if (reason && reason_cap) {
        std::snprintf(reason, reason_cap, "%s", ok ? "" : why.c_str());
    }
    return ok;
}

size_t fp8ln_workspace_size(int32_t op, int64_t a, int64_t b, int64_t c) {
    if (a < 0 || b <= 0) return 0;
    switch (op) {
        case FP8LN_OP_CAST_AMAX: return cast_workspace(a, b);
        case FP8LN_OP_LAYERNORM_BWD: return ln_bwd_workspace(a, (int)b);
        case FP8LN_OP_GEMM_DGELU_FP8: return dgelu_workspace(a, b);
        case FP8LN_OP_LINEAR_BWD: return c > 0 ? linear_only_ws(nullptr, a, b, c).bytes : 0;
        case FP8LN_OP_LN_LINEAR_BWD_BF16:
            return b > 0 && c > 0 ? linear_bf16_ws(nullptr, a, b, c).bytes : 0;
        case FP8LN_OP_TRANSPOSE_BF16: return transpose_b16_workspace(a, b);
        case FP8LN_OP_LN_MLP_BWD_BF16:
            return b > 0 && c > 0 ? mlp_bf16_ws(nullptr, a, b, c).bytes : 0;
        case FP8LN_OP_LN_LINEAR_BWD: return c > 0 ? linear_ws(nullptr, a, b, c).bytes : 0;
        case FP8LN_OP_LN_MLP_BWD: return c > 0 ? mlp_ws(nullptr, a, b, c).bytes : 0;
        default: return 0;
    }
}

int fp8ln_meta_init(const fp8ln_recipe* recipe, const fp8ln_meta* meta, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    if ((s = check_meta(meta, 1, -1, "state"))) return s;
    if ((s = check_current_device())) return s;
    FP8LN_TRY(launch_meta_init(meta->amax_history, meta->scale, meta->scale_inv,
                               recipe->amax_history_len, meta->n_slots, as_stream(stream)),
              "meta_init launch");
    return FP8LN_OK;
}

int fp8ln_scaling_update(const fp8ln_recipe* recipe, const fp8ln_meta* meta, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    if ((s = check_meta(meta, 1, -1, "state"))) return s;
    if ((s = check_current_device())) return s;
    const float fmax = fp8_max_of(meta_fp8(recipe, meta->kind));
    FP8LN_TRY(launch_scaling_update(meta->amax_history, meta->scale, meta->scale_inv,
                                    recipe->amax_history_len, meta->n_slots, recipe->margin, fmax,
                                    as_stream(stream)),
              "scaling_update launch");
    return FP8LN_OK;
}

int fp8ln_scaling_update_batch(const fp8ln_recipe* recipe, const fp8ln_meta* metas, int32_t n,
                               void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    REQUIRE(n >= 0, "n < 0");
    if (n > 0) REQUIRE_PTR(metas);
    for (int32_t i = 0; i < n; ++i)
        if ((s = check_meta(metas + i, 1, -1, "state"))) return s;
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    UpdateBatch b;   // kernel arguments are copied at launch
    for (int32_t base = 0; base < n; base += kMaxUpdateBatch) {
        const int cnt = n - base < kMaxUpdateBatch ? (int)(n - base) : kMaxUpdateBatch;
        b.len = recipe->amax_history_len;
        b.margin = recipe->margin;
        for (int k = 0; k < cnt; ++k) {
            const fp8ln_meta& m = metas[base + k];
            b.job[k] = UpdateJob{m.amax_history, m.scale, m.scale_inv, m.n_slots,
                                 fp8_max_of(meta_fp8(recipe, m.kind))};
        }
        FP8LN_TRY(launch_scaling_update_batch(b, cnt, st), "scaling_update_batch launch");
    }
    return FP8LN_OK;
}

int fp8ln_ln_cast_amax(const fp8ln_recipe* recipe, int64_t rows, int64_t hidden,
                       int32_t params_dtype, const void* x, const void* gamma, const void* beta,
                       int32_t fp8_dtype, const float* scale, float* amax, uint8_t* out,
                       uint8_t* out_t, float* mean, float* rstd, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    REQUIRE(rows >= 0, "rows %lld < 0", (long long)rows);
    if (params_dtype != FP8LN_DTYPE_BF16)
        return fail(FP8LN_ERR_UNSUPPORTED, "params_dtype %d: only bf16 is supported", params_dtype);
    REQUIRE(fp8_dtype == FP8LN_E4M3 || fp8_dtype == FP8LN_E5M2, "fp8_dtype %d invalid", fp8_dtype);
    if (hidden <= 0 || hidden % 8 != 0 || hidden > 8192)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld must be a multiple of 8 in 8..8192",
                    (long long)hidden);
    if (out_t && (rows % 16 != 0 || hidden % 16 != 0))
        return fail(FP8LN_ERR_UNSUPPORTED, "a transposed output needs rows and hidden %% 16 == 0");
    REQUIRE_PTR(gamma); REQUIRE_PTR(beta); REQUIRE_PTR(scale); REQUIRE_PTR(amax);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(beta);
    if (rows > 0) {
        REQUIRE_PTR(x); REQUIRE_PTR(out);
        REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(out);
        if (out_t) REQUIRE_ALIGNED(out_t);
    }
    if (out_t) CHECK(check_transpose_rows(rows, "ln_cast_amax"));
    if ((s = check_current_device())) return s;
    if (rows == 0) return FP8LN_OK;
    hipStream_t st = as_stream(stream);
    FP8LN_TRY(launch_ln_cast_amax(rows, (int)hidden, x, gamma, beta, recipe->ln_eps, fp8_dtype,
                                  scale, amax, out, mean, rstd, st),
              "ln_cast_amax launch");
    if (out_t) FP8LN_TRY(launch_transpose_u8(rows, hidden, out, out_t, st), "transpose launch");
    return FP8LN_OK;
}

int fp8ln_cast_amax(int64_t rows, int64_t cols, int32_t in_dtype, const void* in,
                    int32_t fp8_dtype, const float* scale, float* amax, uint8_t* out,
                    uint8_t* out_t, float* colsum, void* workspace, size_t workspace_bytes,
                    void* stream) {
    REQUIRE(rows >= 0 && cols >= 0, "negative size");
    REQUIRE(in_dtype == FP8LN_DTYPE_BF16 || in_dtype == FP8LN_DTYPE_F32, "in_dtype %d invalid",
            in_dtype);
    REQUIRE(fp8_dtype == FP8LN_E4M3 || fp8_dtype == FP8LN_E5M2, "fp8_dtype %d invalid", fp8_dtype);
    if (cols % 16 != 0) return fail(FP8LN_ERR_UNSUPPORTED, "cols %lld %% 16 != 0", (long long)cols);
    if (out_t && rows % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "a transposed output needs rows %% 16 == 0");
    REQUIRE_PTR(scale); REQUIRE_PTR(amax);
    if (rows > 0 && cols > 0) {
        REQUIRE_PTR(in); REQUIRE_PTR(out);
        REQUIRE_ALIGNED(in); REQUIRE_ALIGNED(out);
        if (out_t) REQUIRE_ALIGNED(out_t);
        if (colsum) {
            REQUIRE(workspace && workspace_bytes >= cast_workspace(rows, cols),
                    "column sums need %zu bytes of workspace", cast_workspace(rows, cols));
        }
    }
    int s = check_current_device();
    if (s) return s;
    FP8LN_TRY(launch_cast_amax(rows, cols, in_dtype == FP8LN_DTYPE_F32, in, fp8_dtype, scale, amax,
                               out, out_t, colsum, workspace, as_stream(stream)),
              "cast_amax launch");
    return FP8LN_OK;
}

int fp8ln_encode_range(uint32_t start, int64_t count, int32_t fp8_dtype, uint8_t* out,
                       void* stream) {
    REQUIRE(count >= 0 && count <= (int64_t(1) << 32), "count %lld outside 0..2^32",
            (long long)count);
    REQUIRE(fp8_dtype == FP8LN_E4M3 || fp8_dtype == FP8LN_E5M2, "fp8_dtype %d invalid", fp8_dtype);
    if (count > 0) { REQUIRE_PTR(out); REQUIRE((reinterpret_cast<uintptr_t>(out) & 3) == 0, "out is not 4-byte aligned"); }
    int s = check_current_device();
    if (s) return s;
    FP8LN_TRY(launch_encode_range(start, count, fp8_dtype, out, as_stream(stream)),
              "encode_range launch");
    return FP8LN_OK;
}

int fp8ln_stream_probe(int64_t n, const void* in, uint8_t* out, void* stream) {
    REQUIRE(n >= 0 && n % 8 == 0, "n %lld must be a non-negative multiple of 8", (long long)n);
    if (n > 0) {
        REQUIRE_PTR(in); REQUIRE_PTR(out); REQUIRE_ALIGNED(in); REQUIRE_ALIGNED(out);
    }
    int s = check_current_device();
    if (s) return s;
    FP8LN_TRY(launch_stream_probe(n, in, out, as_stream(stream)), "stream probe launch");
    return FP8LN_OK;
}

int fp8ln_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
               const uint8_t* B, int32_t b_dtype, const float* sinv_a, const float* sinv_b,
               const void* bias, int32_t out_dtype, void* out, void* stream) {
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(a_dtype == FP8LN_E4M3 || a_dtype == FP8LN_E5M2, "a_dtype %d invalid", a_dtype);
    REQUIRE(b_dtype == FP8LN_E4M3 || b_dtype == FP8LN_E5M2, "b_dtype %d invalid", b_dtype);
    REQUIRE(out_dtype == FP8LN_DTYPE_BF16 || out_dtype == FP8LN_DTYPE_F32, "out_dtype %d invalid",
            out_dtype);
    if (N % 16 != 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "N and K must be multiples of 16 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    REQUIRE_PTR(sinv_a); REQUIRE_PTR(sinv_b);
    if (M > 0 && N > 0) {
        REQUIRE_PTR(out); REQUIRE_ALIGNED(out);
        if (K > 0) { REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_ALIGNED(A); REQUIRE_ALIGNED(B); }
        if (bias) REQUIRE_ALIGNED(bias);
    }
    REQUIRE(!(bias && out_dtype == FP8LN_DTYPE_F32), "bias is only applied to bf16 outputs");
    CHECK(check_gemm_size(M, N, K, 1, false, "gemm"));
    int s = check_current_device();
    if (s) return s;
    GemmParams p = gemm_params(M, N, K, A, a_dtype, B, b_dtype, sinv_a, sinv_b,
                               out_dtype == FP8LN_DTYPE_BF16 ? kEpiBf16Bias : kEpiF32);
    p.bias = (const uint16_t*)bias;
    p.out = out;
    FP8LN_TRY(launch_gemm(p, as_stream(stream)), "gemm launch");
    return FP8LN_OK;
}

int fp8ln_gemm_gelu_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
                        const uint8_t* B, int32_t b_dtype, const float* sinv_a,
                        const float* sinv_b, const void* bias, void* h_out, uint8_t* q_out,
                        uint8_t* q_out_t, int32_t q_dtype, const float* q_scale, float* q_amax,
                        int32_t activation, void* stream) {
    REQUIRE(activation == FP8LN_GELU_TANH || activation == FP8LN_GELU_ERF,
            "activation %d invalid", activation);
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(a_dtype == FP8LN_E4M3 || a_dtype == FP8LN_E5M2, "a_dtype %d invalid", a_dtype);
    REQUIRE(b_dtype == FP8LN_E4M3 || b_dtype == FP8LN_E5M2, "b_dtype %d invalid", b_dtype);
    REQUIRE(q_dtype == FP8LN_E4M3 || q_dtype == FP8LN_E5M2, "q_dtype %d invalid", q_dtype);
    if (N % 16 != 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "N and K must be multiples of 16 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (q_out_t && M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "a transposed output needs M %% 16 == 0");
    REQUIRE_PTR(sinv_a); REQUIRE_PTR(sinv_b); REQUIRE_PTR(q_scale); REQUIRE_PTR(q_amax);
    if (M > 0 && N > 0) {
        REQUIRE_PTR(q_out); REQUIRE_ALIGNED(q_out);
        if (q_out_t) REQUIRE_ALIGNED(q_out_t);
        if (h_out) REQUIRE_ALIGNED(h_out);
        if (bias) REQUIRE_ALIGNED(bias);
        if (K > 0) { REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_ALIGNED(A); REQUIRE_ALIGNED(B); }
    }
    CHECK(check_gemm_size(M, N, K, 1, false, "gemm_gelu_fp8"));
    int s = check_current_device();
    if (s) return s;
    GemmParams p = gemm_params(M, N, K, A, a_dtype, B, b_dtype, sinv_a, sinv_b, kEpiGeluFp8);
    p.bias = (const uint16_t*)bias;
    p.h_out = (uint16_t*)h_out;
    p.q_out = q_out;
    p.q_out_t = q_out_t;
    p.q_scale = q_scale;
    p.q_amax = q_amax;
    p.q_fp8 = q_dtype;
    p.gelu_erf = activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(p, as_stream(stream)), "gemm_gelu launch");
    return FP8LN_OK;
}

int fp8ln_gemm_dgelu(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
                     const uint8_t* B, int32_t b_dtype, const float* sinv_a, const float* sinv_b,
                     const void* h, float* out, int32_t activation, void* stream) {
    REQUIRE(activation == FP8LN_GELU_TANH || activation == FP8LN_GELU_ERF,
            "activation %d invalid", activation);
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(a_dtype == FP8LN_E4M3 || a_dtype == FP8LN_E5M2, "a_dtype %d invalid", a_dtype);
    REQUIRE(b_dtype == FP8LN_E4M3 || b_dtype == FP8LN_E5M2, "b_dtype %d invalid", b_dtype);
    if (N % 16 != 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "N and K must be multiples of 16 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    REQUIRE_PTR(sinv_a); REQUIRE_PTR(sinv_b);
    if (M > 0 && N > 0) {
        REQUIRE_PTR(out); REQUIRE_PTR(h); REQUIRE_ALIGNED(out); REQUIRE_ALIGNED(h);
        if (K > 0) { REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_ALIGNED(A); REQUIRE_ALIGNED(B); }
    }
    CHECK(check_gemm_size(M, N, K, 1, true, "gemm_dgelu"));
    int s = check_current_device();
    if (s) return s;
    GemmParams p = gemm_params(M, N, K, A, a_dtype, B, b_dtype, sinv_a, sinv_b, kEpiDGeluF32);
    p.h_in = (const uint16_t*)h;
    p.out = out;
    p.gelu_erf = activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(p, as_stream(stream)), "gemm_dgelu launch");
    return FP8LN_OK;
}

int fp8ln_gemm_dgelu_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
                         const uint8_t* B, int32_t b_dtype, const float* sinv_a,
                         const float* sinv_b, const void* h, int32_t q_dtype,
                         const float* q_scale, float* q_amax, uint8_t* q_out, uint8_t* q_out_t,
                         float* dbias, int32_t activation, void* workspace,
                         size_t workspace_bytes, void* stream) {
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(activation == FP8LN_GELU_TANH || activation == FP8LN_GELU_ERF,
            "activation %d invalid", activation);
    REQUIRE(a_dtype == FP8LN_E4M3 || a_dtype == FP8LN_E5M2, "a_dtype %d invalid", a_dtype);
    REQUIRE(b_dtype == FP8LN_E4M3 || b_dtype == FP8LN_E5M2, "b_dtype %d invalid", b_dtype);
    REQUIRE(q_dtype == FP8LN_E4M3 || q_dtype == FP8LN_E5M2, "q_dtype %d invalid", q_dtype);
    if (N % 16 != 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "N and K must be multiples of 16 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (q_out_t && M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "a transposed output needs M %% 16 == 0");
    REQUIRE_PTR(sinv_a); REQUIRE_PTR(sinv_b); REQUIRE_PTR(q_scale); REQUIRE_PTR(q_amax);
    if (M > 0 && N > 0) {
        REQUIRE_PTR(q_out); REQUIRE_PTR(h); REQUIRE_ALIGNED(q_out); REQUIRE_ALIGNED(h);
        if (q_out_t) REQUIRE_ALIGNED(q_out_t);
        if (K > 0) { REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_ALIGNED(A); REQUIRE_ALIGNED(B); }
    }
    if (dbias) {
        REQUIRE(workspace && workspace_bytes >= dgelu_workspace(M, N),
                "column sums need %zu bytes of workspace", dgelu_workspace(M, N));
        REQUIRE_ALIGNED(workspace);
    }
    CHECK(check_gemm_size(M, N, K, 1, true, "gemm_dgelu_fp8"));
    int s = check_current_device();
    if (s) return s;
    hipStream_t st = as_stream(stream);
    GemmParams p = gemm_params(M, N, K, A, a_dtype, B, b_dtype, sinv_a, sinv_b, kEpiDGeluFp8);
    p.h_in = (const uint16_t*)h;
    p.q_out = q_out;
    p.q_out_t = q_out_t;
    p.q_scale = q_scale;
    p.q_amax = q_amax;
    p.q_fp8 = q_dtype;
    p.col_partial = dbias ? (float*)workspace : nullptr;
    p.gelu_erf = activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(p, st), "gemm_dgelu_fp8 launch");
    if (dbias)
        FP8LN_TRY(launch_sum_partials((const float*)workspace, M > 0 ? gemm_partial_rows(M, N, K) : 0,
                                      N, dbias, nullptr, N, st),
                  "column sum launch");
    return FP8LN_OK;
}

int fp8ln_layernorm_bwd(int64_t rows, int64_t hidden, const float* dy, const void* x,
                        const float* mean, const float* rstd, const void* gamma, void* dx,
                        float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                        void* stream) {
    REQUIRE(rows >= 0, "rows < 0");
    if (hidden <= 0 || hidden % 8 != 0 || hidden > 4096)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld must be a multiple of 8 in 8..4096",
                    (long long)hidden);
    REQUIRE_PTR(gamma); REQUIRE_PTR(dgamma); REQUIRE_PTR(dbeta);
    REQUIRE_ALIGNED(gamma);
    if (rows > 0) {
        REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(mean); REQUIRE_PTR(rstd); REQUIRE_PTR(dx);
        REQUIRE_ALIGNED(dy); REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(dx);
    }
    REQUIRE(workspace && workspace_bytes >= ln_bwd_workspace(rows, (int)hidden),
            "layernorm_bwd needs %zu bytes of workspace", ln_bwd_workspace(rows, (int)hidden));
    int s = check_current_device();
    if (s) return s;
    FP8LN_TRY(launch_ln_bwd(rows, (int)hidden, dy, false, x, mean, rstd, gamma, dx, dgamma, dbeta,
                            workspace, as_stream(stream)),
              "layernorm_bwd launch");
    return FP8LN_OK;
}

// ---- BF16 path ------------------------------------------------------------------

int fp8ln_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                    const void* bias, int32_t out_dtype, void* out, void* stream) {
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    REQUIRE(out_dtype == FP8LN_DTYPE_BF16 || out_dtype == FP8LN_DTYPE_F32, "out_dtype %d invalid",
            out_dtype);
    if (N % 16 != 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "N and K must be multiples of 16 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (M > 0 && N > 0) {
        REQUIRE_PTR(out); REQUIRE_ALIGNED(out);
        if (K > 0) { REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_ALIGNED(A); REQUIRE_ALIGNED(B); }
        if (bias) REQUIRE_ALIGNED(bias);
    }
    REQUIRE(!(bias && out_dtype == FP8LN_DTYPE_F32), "bias is only applied to bf16 outputs");
    CHECK(check_gemm_size(M, N, K, 2, false, "gemm_bf16"));
    int s = check_current_device();
    if (s) return s;
    GemmParams p = gemm_params(M, N, K, (const uint8_t*)A, kOpBf16, (const uint8_t*)B, kOpBf16,
                               nullptr, nullptr,
                               out_dtype == FP8LN_DTYPE_BF16 ? kEpiBf16Bias : kEpiF32);
    p.bias = (const uint16_t*)bias;
    p.out = out;
    FP8LN_TRY(launch_gemm(p, as_stream(stream)), "gemm launch");
    return FP8LN_OK;
}

int fp8ln_gemm_gelu_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                         const void* bias, void* h_out, void* out, int32_t activation,
                         void* stream) {
    REQUIRE(activation == FP8LN_GELU_TANH || activation == FP8LN_GELU_ERF,
            "activation %d invalid", activation);
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    if (N % 16 != 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "N and K must be multiples of 16 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (M > 0 && N > 0) {
        REQUIRE_PTR(out); REQUIRE_ALIGNED(out);
        if (h_out) REQUIRE_ALIGNED(h_out);
        if (K > 0) { REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_ALIGNED(A); REQUIRE_ALIGNED(B); }
        if (bias) REQUIRE_ALIGNED(bias);
    }
    CHECK(check_gemm_size(M, N, K, 2, false, "gemm_gelu_bf16"));
    int s = check_current_device();
    if (s) return s;
    GemmParams p = gemm_params(M, N, K, (const uint8_t*)A, kOpBf16, (const uint8_t*)B, kOpBf16,
                               nullptr, nullptr, kEpiGeluBf16);
    p.bias = (const uint16_t*)bias;
    p.h_out = (uint16_t*)h_out;
    p.out = out;
    p.gelu_erf = activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(p, as_stream(stream)), "gemm launch");
    return FP8LN_OK;
}

int fp8ln_gemm_dgelu_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                          const void* h, void* out, int32_t activation, void* stream) {
    REQUIRE(activation == FP8LN_GELU_TANH || activation == FP8LN_GELU_ERF,
            "activation %d invalid", activation);
    REQUIRE(M >= 0 && N >= 0 && K >= 0, "negative size");
    if (N % 16 != 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "N and K must be multiples of 16 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    if (M > 0 && N > 0) {
        REQUIRE_PTR(out); REQUIRE_PTR(h); REQUIRE_ALIGNED(out); REQUIRE_ALIGNED(h);
        if (K > 0) { REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_ALIGNED(A); REQUIRE_ALIGNED(B); }
    }
    CHECK(check_gemm_size(M, N, K, 2, true, "gemm_dgelu_bf16"));
    int s = check_current_device();
    if (s) return s;
    GemmParams p = gemm_params(M, N, K, (const uint8_t*)A, kOpBf16, (const uint8_t*)B, kOpBf16,
                               nullptr, nullptr, kEpiDGeluBf16);
    p.h_in = (const uint16_t*)h;
    p.out = out;
    p.gelu_erf = activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(p, as_stream(stream)), "gemm launch");
    return FP8LN_OK;
}

int fp8ln_transpose_bf16(int64_t rows, int64_t cols, const void* in, void* out, float* colsum,
                         void* workspace, size_t workspace_bytes, void* stream) {
    REQUIRE(rows >= 0 && cols >= 0, "negative size");
    if (rows % 8 != 0 || cols % 8 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "rows and cols must be multiples of 8");
    if (rows > 0 && cols > 0) {
        REQUIRE_PTR(in); REQUIRE_PTR(out); REQUIRE_ALIGNED(in); REQUIRE_ALIGNED(out);
    }
    if (colsum) {
        const size_t need = transpose_b16_workspace(rows, cols);
        REQUIRE(need == 0 || (workspace && workspace_bytes >= need),
                "column sums need %zu bytes of workspace", need);
    }
    CHECK(check_transpose_rows(rows, "transpose_bf16"));
    int s = check_current_device();
    if (s) return s;
    FP8LN_TRY(launch_transpose_b16(rows, cols, in, out, colsum, workspace, as_stream(stream)),
              "transpose launch");
    return FP8LN_OK;
}

int fp8ln_ln_linear_fwd_bf16(int64_t tokens, int64_t in_features, int64_t out_features,
                             float eps, const void* x, const void* gamma, const void* beta,
                             const void* weight, const void* bias, void* out, void* ln_out,
                             float* mean, float* rstd, void* stream) {
    const int64_t M = tokens, K = in_features, N = out_features;
    int s = check_bf16_module(M, K, N, eps);
    if (s) return s;
    REQUIRE_PTR(gamma); REQUIRE_PTR(beta); REQUIRE_PTR(weight);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(beta); REQUIRE_ALIGNED(weight);
    if (bias) REQUIRE_ALIGNED(bias);
    if (M > 0) {
        REQUIRE_PTR(x); REQUIRE_PTR(out); REQUIRE_PTR(ln_out);
        REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(out); REQUIRE_ALIGNED(ln_out);
    }
    CHECK(check_gemm_size(tokens, out_features, in_features, 2, false, "ln_linear_fwd_bf16"));
    if ((s = check_current_device())) return s;
    if (M == 0) return FP8LN_OK;
    hipStream_t st = as_stream(stream);
    FP8LN_TRY(launch_ln_cast_amax(M, (int)K, x, gamma, beta, eps, kLnOutBf16, nullptr, nullptr,
                                  ln_out, mean, rstd, st),
              "layernorm launch");
    GemmParams p = gemm_params(M, N, K, (const uint8_t*)ln_out, kOpBf16, (const uint8_t*)weight,
                               kOpBf16, nullptr, nullptr, kEpiBf16Bias);
    p.bias = (const uint16_t*)bias;
    p.out = out;
    FP8LN_TRY(launch_gemm(p, st), "gemm launch");
    return FP8LN_OK;
}

int fp8ln_ln_linear_bwd_bf16(int64_t tokens, int64_t in_features, int64_t out_features,
                             const void* dy, const void* x, const void* gamma,
                             const void* weight, const void* ln_out, const float* mean,
                             const float* rstd, void* dx, float* dgamma, float* dbeta,
                             float* dweight, float* dbias, void* workspace,
                             size_t workspace_bytes, void* stream) {
    const int64_t M = tokens, K = in_features, N = out_features;
    int s = check_bf16_module(M, K, N, 1.0f);
    if (s) return s;
    if (M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "tokens %lld must be a multiple of 16", (long long)M);
    if (K > 4096)
        return fail(FP8LN_ERR_UNSUPPORTED, "in_features %lld: the backward takes at most 4096",
                    (long long)K);
    REQUIRE_PTR(gamma); REQUIRE_PTR(weight); REQUIRE_PTR(dgamma); REQUIRE_PTR(dbeta);
    REQUIRE_PTR(dweight);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(weight); REQUIRE_ALIGNED(dweight);
    if (M > 0) {
        REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(ln_out); REQUIRE_PTR(mean);
        REQUIRE_PTR(rstd); REQUIRE_PTR(dx);
        REQUIRE_ALIGNED(dy); REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(ln_out); REQUIRE_ALIGNED(dx);
    }
    const LinearBf16Ws need = linear_bf16_ws(nullptr, M, K, N);
    REQUIRE(workspace && workspace_bytes >= need.bytes,
            "ln_linear_bwd_bf16 needs %zu bytes of workspace", need.bytes);
    REQUIRE_ALIGNED(workspace);
    CHECK(check_transpose_rows(tokens, "ln_linear_bwd_bf16"));
    CHECK(check_gemm_size(tokens, in_features, out_features, 2, false, "ln_linear_bwd_bf16 dgrad"));
    CHECK(check_gemm_size(out_features, in_features, tokens, 2, false, "ln_linear_bwd_bf16 wgrad"));
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const LinearBf16Ws w = linear_bf16_ws(workspace, M, K, N);
    FP8LN_TRY(launch_transpose_b16(M, N, dy, w.dy_t, dbias, w.sum_ws, st), "dy transpose");
    FP8LN_TRY(launch_transpose_b16(N, K, weight, w.w_t, nullptr, nullptr, st), "w transpose");
    FP8LN_TRY(launch_transpose_b16(M, K, ln_out, w.ln_t, nullptr, nullptr, st), "ln transpose");
    // dgrad: dLN[M][K] = dy[M][N] . (w_t[K][N])^T
    GemmParams dg = gemm_params(M, K, N, (const uint8_t*)dy, kOpBf16, (const uint8_t*)w.w_t,
                                kOpBf16, nullptr, nullptr, kEpiF32);
    dg.out = w.dln;
    FP8LN_TRY(launch_gemm(dg, st), "dgrad launch");
    // wgrad: dW[N][K] = dy_t[N][M] . (ln_t[K][M])^T
    GemmParams wg = gemm_params(N, K, M, (const uint8_t*)w.dy_t, kOpBf16, (const uint8_t*)w.ln_t,
                                kOpBf16, nullptr, nullptr, kEpiF32);
    wg.out = dweight;
    FP8LN_TRY(launch_gemm(wg, st), "wgrad launch");
    FP8LN_TRY(launch_ln_bwd(M, (int)K, w.dln, false, x, mean, rstd, gamma, dx, dgamma, dbeta,
                            w.ln_ws, st),
              "layernorm backward launch");
    return FP8LN_OK;
}

int fp8ln_ln_mlp_fwd_bf16(int64_t tokens, int64_t hidden, int64_t ffn, float eps,
                          int32_t activation, const void* x, const void* gamma, const void* beta,
                          const void* w1, const void* b1, const void* w2, const void* b2,
                          void* out, void* ln_out, void* h, void* g, float* mean, float* rstd,
                          void* stream) {
    const int64_t M = tokens, H = hidden, F = ffn;
    int s = check_bf16_module(M, H, F, eps);
    if (s) return s;
    REQUIRE(activation == FP8LN_GELU_TANH || activation == FP8LN_GELU_ERF,
            "activation %d invalid", activation);
    REQUIRE_PTR(gamma); REQUIRE_PTR(beta); REQUIRE_PTR(w1); REQUIRE_PTR(w2);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(beta); REQUIRE_ALIGNED(w1); REQUIRE_ALIGNED(w2);
    if (b1) REQUIRE_ALIGNED(b1);
    if (b2) REQUIRE_ALIGNED(b2);
    if (M > 0) {
        REQUIRE_PTR(x); REQUIRE_PTR(out); REQUIRE_PTR(ln_out); REQUIRE_PTR(g);
        REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(out); REQUIRE_ALIGNED(ln_out); REQUIRE_ALIGNED(g);
        if (h) REQUIRE_ALIGNED(h);
    }
    CHECK(check_gemm_size(tokens, ffn, hidden, 2, false, "ln_mlp_fwd_bf16 fc1"));
    CHECK(check_gemm_size(tokens, hidden, ffn, 2, false, "ln_mlp_fwd_bf16 fc2"));
    if ((s = check_current_device())) return s;
    if (M == 0) return FP8LN_OK;
    hipStream_t st = as_stream(stream);
    FP8LN_TRY(launch_ln_cast_amax(M, (int)H, x, gamma, beta, eps, kLnOutBf16, nullptr, nullptr,
                                  ln_out, mean, rstd, st),
              "layernorm launch");
    GemmParams p1 = gemm_params(M, F, H, (const uint8_t*)ln_out, kOpBf16, (const uint8_t*)w1,
                                kOpBf16, nullptr, nullptr, kEpiGeluBf16);
    p1.bias = (const uint16_t*)b1;
    p1.h_out = (uint16_t*)h;
    p1.out = g;
    p1.gelu_erf = activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(p1, st), "fc1 launch");
    GemmParams p2 = gemm_params(M, H, F, (const uint8_t*)g, kOpBf16, (const uint8_t*)w2, kOpBf16,
                                nullptr, nullptr, kEpiBf16Bias);
    p2.bias = (const uint16_t*)b2;
    p2.out = out;
    FP8LN_TRY(launch_gemm(p2, st), "fc2 launch");
    return FP8LN_OK;
}

int fp8ln_ln_mlp_bwd_bf16(int64_t tokens, int64_t hidden, int64_t ffn, int32_t activation,
                          const void* dy, const void* x, const void* gamma, const void* w1,
                          const void* w2, const void* ln_out, const void* h, const void* g,
                          const float* mean, const float* rstd, void* dx, float* dgamma,
                          float* dbeta, float* dw1, float* db1, float* dw2, float* db2,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const int64_t M = tokens, H = hidden, F = ffn;
    int s = check_bf16_module(M, H, F, 1.0f);
    if (s) return s;
    REQUIRE(activation == FP8LN_GELU_TANH || activation == FP8LN_GELU_ERF,
            "activation %d invalid", activation);
    if (M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "tokens %lld must be a multiple of 16", (long long)M);
    if (H > 4096)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld: the backward takes at most 4096",
                    (long long)H);
    REQUIRE_PTR(gamma); REQUIRE_PTR(w1); REQUIRE_PTR(w2); REQUIRE_PTR(dgamma); REQUIRE_PTR(dbeta);
    REQUIRE_PTR(dw1); REQUIRE_PTR(dw2);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(w1); REQUIRE_ALIGNED(w2); REQUIRE_ALIGNED(dw1);
    REQUIRE_ALIGNED(dw2);
    if (M > 0) {
        REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(ln_out); REQUIRE_PTR(h); REQUIRE_PTR(g);
        REQUIRE_PTR(mean); REQUIRE_PTR(rstd); REQUIRE_PTR(dx);
        REQUIRE_ALIGNED(dy); REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(ln_out); REQUIRE_ALIGNED(h);
        REQUIRE_ALIGNED(g); REQUIRE_ALIGNED(dx);
    }
    const MlpBf16Ws need = mlp_bf16_ws(nullptr, M, H, F);
    REQUIRE(workspace && workspace_bytes >= need.bytes,
            "ln_mlp_bwd_bf16 needs %zu bytes of workspace", need.bytes);
    REQUIRE_ALIGNED(workspace);
    CHECK(check_transpose_rows(tokens, "ln_mlp_bwd_bf16"));
    CHECK(check_gemm_size(tokens, ffn, hidden, 2, true, "ln_mlp_bwd_bf16 fc2 dgrad"));
    CHECK(check_gemm_size(hidden, ffn, tokens, 2, false, "ln_mlp_bwd_bf16 wgrad"));
    CHECK(check_gemm_size(tokens, hidden, ffn, 2, false, "ln_mlp_bwd_bf16 fc1 dgrad"));
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const MlpBf16Ws w = mlp_bf16_ws(workspace, M, H, F);
    auto gemm = [&](int64_t m, int64_t n, int64_t k, const void* a, const void* b, int epi,
                    void* out) {
        GemmParams p = gemm_params(m, n, k, (const uint8_t*)a, kOpBf16, (const uint8_t*)b,
                                   kOpBf16, nullptr, nullptr, epi);
        p.out = out;
        p.h_in = (const uint16_t*)h;
        p.gelu_erf = activation == FP8LN_GELU_ERF;
        return launch_gemm(p, st);
    };
    FP8LN_TRY(launch_transpose_b16(M, H, dy, w.dy_t, db2, w.sum_ws, st), "dy transpose");
    FP8LN_TRY(launch_transpose_b16(M, F, g, w.g_t, nullptr, nullptr, st), "g transpose");
    FP8LN_TRY(launch_transpose_b16(H, F, w2, w.w2_t, nullptr, nullptr, st), "w2 transpose");
    // fc2 wgrad: dW2[H][F] = dy_t[H][M] . (g_t[F][M])^T
    FP8LN_TRY(gemm(H, F, M, w.dy_t, w.g_t, kEpiF32, dw2), "fc2 wgrad launch");
    // fc2 dgrad with GELU': dH[M][F] = (dy[M][H] . (w2_t[F][H])^T) * gelu'(h)
    FP8LN_TRY(gemm(M, F, H, dy, w.w2_t, kEpiDGeluBf16, w.dh), "fc2 dgrad launch");
    FP8LN_TRY(launch_transpose_b16(M, F, w.dh, w.dh_t, db1, w.sum_ws, st), "dH transpose");
    FP8LN_TRY(launch_transpose_b16(F, H, w1, w.w1_t, nullptr, nullptr, st), "w1 transpose");
    FP8LN_TRY(launch_transpose_b16(M, H, ln_out, w.ln_t, nullptr, nullptr, st), "ln transpose");
    // fc1 wgrad: dW1[F][H] = dh_t[F][M] . (ln_t[H][M])^T
    FP8LN_TRY(gemm(F, H, M, w.dh_t, w.ln_t, kEpiF32, dw1), "fc1 wgrad launch");
    // fc1 dgrad: dLN[M][H] = dH[M][F] . (w1_t[H][F])^T
    FP8LN_TRY(gemm(M, H, F, w.dh, w.w1_t, kEpiF32, w.dln), "fc1 dgrad launch");
    FP8LN_TRY(launch_ln_bwd(M, (int)H, w.dln, false, x, mean, rstd, gamma, dx, dgamma, dbeta,
                            w.ln_ws, st),
              "layernorm backward launch");
    return FP8LN_OK;
}

int fp8ln_layernorm_fwd(int64_t rows, int64_t hidden, float eps, const void* x,
                        const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                        void* stream) {
    REQUIRE(rows >= 0, "rows %lld < 0", (long long)rows);
    REQUIRE(eps > 0.0f && eps <= 3.402823466e38f, "eps must be a positive finite number");
    if (hidden <= 0 || hidden % 8 != 0 || hidden > 8192)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld must be a multiple of 8 in 8..8192",
                    (long long)hidden);
    REQUIRE_PTR(gamma); REQUIRE_PTR(beta);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(beta);
    if (rows > 0) {
        REQUIRE_PTR(x); REQUIRE_PTR(y);
        REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(y);
    }
    int s = check_current_device();
    if (s) return s;
    if (rows == 0) return FP8LN_OK;
    FP8LN_TRY(launch_ln_cast_amax(rows, (int)hidden, x, gamma, beta, eps, kLnOutBf16, nullptr,
                                  nullptr, y, mean, rstd, as_stream(stream)),
              "layernorm_fwd launch");
    return FP8LN_OK;
}

int fp8ln_layernorm_bwd_bf16(int64_t rows, int64_t hidden, const void* dy, const void* x,
                             const float* mean, const float* rstd, const void* gamma, void* dx,
                             float* dgamma, float* dbeta, void* workspace,
                             size_t workspace_bytes, void* stream) {
    REQUIRE(rows >= 0, "rows < 0");
    if (hidden <= 0 || hidden % 8 != 0 || hidden > 4096)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld must be a multiple of 8 in 8..4096",
                    (long long)hidden);
    REQUIRE_PTR(gamma); REQUIRE_PTR(dgamma); REQUIRE_PTR(dbeta);
    REQUIRE_ALIGNED(gamma);
    if (rows > 0) {
        REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(mean); REQUIRE_PTR(rstd); REQUIRE_PTR(dx);
        REQUIRE_ALIGNED(dy); REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(dx);
    }
    REQUIRE(workspace && workspace_bytes >= ln_bwd_workspace(rows, (int)hidden),
            "layernorm_bwd needs %zu bytes of workspace", ln_bwd_workspace(rows, (int)hidden));
    int s = check_current_device();
    if (s) return s;
    FP8LN_TRY(launch_ln_bwd(rows, (int)hidden, dy, true, x, mean, rstd, gamma, dx, dgamma, dbeta,
                            workspace, as_stream(stream)),
              "layernorm_bwd launch");
    return FP8LN_OK;
}

int fp8ln_linear_fwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                     int64_t out_features, int32_t params_dtype, const void* x,
                     const void* weight, const void* bias, void* out, const fp8ln_meta* fwd,
                     const fp8ln_linear_ctx* ctx, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    const int64_t M = tokens, K = in_features, N = out_features;
    REQUIRE(M >= 0, "tokens < 0");
    if (params_dtype != FP8LN_DTYPE_BF16)
        return fail(FP8LN_ERR_UNSUPPORTED, "params_dtype %d: only bf16 is supported", params_dtype);
    if (K <= 0 || K % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "in_features %lld must be a positive multiple of 16",
                    (long long)K);
    if (N <= 0 || N % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "out_features %lld must be a positive multiple of 16",
                    (long long)N);
    if ((s = check_meta(fwd, 2, FP8LN_META_FORWARD, "forward"))) return s;
    REQUIRE_PTR(ctx);
    REQUIRE(ctx->w_q, "ctx.w_q is required");
    REQUIRE(M == 0 || ctx->ln_q, "ctx.ln_q (the input codes) is required");
    if (ctx->ln_qt && M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "ctx.ln_qt needs tokens %% 16 == 0");
    REQUIRE(!ctx->reuse_weight_codes || ctx->w_scale_inv,
            "reuse_weight_codes needs ctx.w_scale_inv from an earlier forward");
    if (!ctx->reuse_weight_codes) { REQUIRE_PTR(weight); REQUIRE_ALIGNED(weight); }
    REQUIRE_ALIGNED(ctx->w_q);
    if (ctx->w_qt) REQUIRE_ALIGNED(ctx->w_qt);
    if (bias) REQUIRE_ALIGNED(bias);
    if (M > 0) {
        REQUIRE_PTR(x); REQUIRE_PTR(out);
        REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(out); REQUIRE_ALIGNED(ctx->ln_q);
        if (ctx->ln_qt) REQUIRE_ALIGNED(ctx->ln_qt);
    }
    CHECK(check_gemm_size(tokens, out_features, in_features, 1, false, "linear_fwd"));
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const int f = meta_fp8(recipe, FP8LN_META_FORWARD);
    float* hist = fwd->amax_history;
    if (M > 0)
        FP8LN_TRY(launch_cast_amax(M, K, false, x, f, fwd->scale + 0, hist + 0, ctx->ln_q,
                                   ctx->ln_qt, nullptr, nullptr, st),
                  "input cast launch");
    const float* w_sinv = ctx->w_scale_inv ? ctx->w_scale_inv : fwd->scale_inv + 1;
    if (!ctx->reuse_weight_codes)
        FP8LN_TRY(launch_cast_amax(N, K, false, weight, f, fwd->scale + 1, hist + 1, ctx->w_q,
                                   ctx->w_qt, nullptr, nullptr, st, fwd->scale_inv + 1,
                                   ctx->w_scale_inv),
                  "weight cast launch");
    GemmParams p = gemm_params(M, N, K, ctx->ln_q, f, ctx->w_q, f, fwd->scale_inv + 0, w_sinv,
                               kEpiBf16Bias);
    p.bias = (const uint16_t*)bias;
    p.out = out;
    FP8LN_TRY(launch_gemm(p, st), "gemm launch");
    return FP8LN_OK;
}

int fp8ln_linear_bwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                     int64_t out_features, int32_t params_dtype, const void* dy,
                     const fp8ln_linear_ctx* ctx, const fp8ln_meta* fwd, const fp8ln_meta* bwd,
                     void* dx, float* dweight, float* dbias, void* workspace,
                     size_t workspace_bytes, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    const int64_t M = tokens, K = in_features, N = out_features;
    if (params_dtype != FP8LN_DTYPE_BF16)
        return fail(FP8LN_ERR_UNSUPPORTED, "params_dtype %d: only bf16 is supported", params_dtype);
    if (M < 0 || M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "tokens %lld must be a multiple of 16", (long long)M);
    if (K <= 0 || K % 16 != 0 || N <= 0 || N % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "in/out_features must be positive multiples of 16");
    if ((s = check_meta(fwd, 2, FP8LN_META_FORWARD, "forward"))) return s;
    if ((s = check_meta(bwd, 1, FP8LN_META_BACKWARD, "backward"))) return s;
    REQUIRE_PTR(ctx);
    REQUIRE(ctx->w_qt && (M == 0 || ctx->ln_qt),
            "ctx needs ln_qt and w_qt from a training forward");
    REQUIRE_PTR(dweight);
    REQUIRE_ALIGNED(dweight); REQUIRE_ALIGNED(ctx->w_qt);
    if (M > 0) {
        REQUIRE_PTR(dy); REQUIRE_PTR(dx);
        REQUIRE_ALIGNED(dy); REQUIRE_ALIGNED(dx); REQUIRE_ALIGNED(ctx->ln_qt);
    }
    const LinearOnlyWs need = linear_only_ws(nullptr, M, K, N);
    REQUIRE(need.bytes == 0 || (workspace && workspace_bytes >= need.bytes),
            "linear_bwd needs %zu bytes of workspace", need.bytes);
    REQUIRE_ALIGNED(workspace);
    CHECK(check_gemm_size(tokens, in_features, out_features, 1, false, "linear_bwd dgrad"));
    CHECK(check_gemm_size(out_features, in_features, tokens, 1, false, "linear_bwd wgrad"));
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const LinearOnlyWs w = linear_only_ws(workspace, M, K, N);
    const int ff = meta_fp8(recipe, FP8LN_META_FORWARD);
    const int bf = meta_fp8(recipe, FP8LN_META_BACKWARD);
    FP8LN_TRY(launch_cast_amax(M, N, false, dy, bf, bwd->scale + 0, bwd->amax_history + 0, w.dy_q,
                               w.dy_qt, dbias, w.cast_ws, st),
              "grad cast launch");
    // dgrad: dx[M][K] = dy_q[M][N] . (w_qt[K][N])^T, bf16 out
    GemmParams dg = gemm_params(M, K, N, w.dy_q, bf, ctx->w_qt, ff, bwd->scale_inv + 0,
                                ctx->w_scale_inv ? ctx->w_scale_inv : fwd->scale_inv + 1,
                                kEpiBf16Bias);
    dg.out = dx;
    FP8LN_TRY(launch_gemm(dg, st), "dgrad launch");
    // wgrad: dW[N][K] = dy_qt[N][M] . (x_qt[K][M])^T
    GemmParams wg = gemm_params(N, K, M, w.dy_qt, bf, ctx->ln_qt, ff, bwd->scale_inv + 0,
                                fwd->scale_inv + 0, kEpiF32);
    wg.out = dweight;
    FP8LN_TRY(launch_gemm(wg, st), "wgrad launch");
    return FP8LN_OK;
}

// LayerNormLinear forward; with step_ws, the step-start scaling update of the
// forward state comes first (folded into the prologue launch when it runs).
static int ln_linear_fwd_impl(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                              int64_t out_features, int32_t params_dtype, const void* x,
                              const void* gamma, const void* beta, const void* weight,
                              const void* bias, void* out, const fp8ln_meta* fwd,
                              const fp8ln_linear_ctx* ctx, void* step_ws, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    const int64_t M = tokens, K = in_features, N = out_features;
    REQUIRE(M >= 0, "tokens < 0");
    if (params_dtype != FP8LN_DTYPE_BF16)
        return fail(FP8LN_ERR_UNSUPPORTED, "params_dtype %d: only bf16 is supported", params_dtype);
    if (K <= 0 || K % 16 != 0 || K > 8192)
        return fail(FP8LN_ERR_UNSUPPORTED, "in_features %lld must be a multiple of 16 in 16..8192",
                    (long long)K);
    if (N <= 0 || N % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "out_features %lld must be a positive multiple of 16",
                    (long long)N);
    if ((s = check_meta(fwd, 2, FP8LN_META_FORWARD, "forward"))) return s;
    REQUIRE_PTR(ctx);
    REQUIRE((M == 0 || ctx->ln_q) && ctx->w_q, "ctx.ln_q and ctx.w_q are required");
    if (ctx->ln_qt && M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "ctx.ln_qt needs tokens %% 16 == 0");
    REQUIRE(!ctx->reuse_weight_codes || ctx->w_scale_inv,
            "reuse_weight_codes needs ctx.w_scale_inv from an earlier forward");
    REQUIRE_PTR(gamma); REQUIRE_PTR(beta);
    if (!ctx->reuse_weight_codes) { REQUIRE_PTR(weight); REQUIRE_ALIGNED(weight); }
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(beta);
    REQUIRE_ALIGNED(ctx->w_q);
    if (ctx->w_qt) REQUIRE_ALIGNED(ctx->w_qt);
    if (bias) REQUIRE_ALIGNED(bias);
    if (M > 0) {
        REQUIRE_PTR(x); REQUIRE_PTR(out);
        REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(out); REQUIRE_ALIGNED(ctx->ln_q);
        if (ctx->ln_qt) REQUIRE_ALIGNED(ctx->ln_qt);
    }
    if (ctx->ln_qt) CHECK(check_transpose_rows(M, "ln_linear_fwd"));
    CHECK(check_gemm_size(M, N, K, 1, false, "ln_linear_fwd"));
    if (step_ws) REQUIRE_ALIGNED(step_ws);
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const int f = meta_fp8(recipe, FP8LN_META_FORWARD);
    float* hist = fwd->amax_history;
    // FP8 weight storage: reuse the codes (and their scale_inv) of an earlier
    // forward of this ctx, or cast now and record the scale_inv that goes with them
    const float* w_sinv = ctx->w_scale_inv ? ctx->w_scale_inv : fwd->scale_inv + 1;
    FusedUpdate upd{hist, fwd->scale, fwd->scale_inv, recipe->amax_history_len, fwd->n_slots,
                    recipe->margin, fp8_max_of(f), (uint32_t*)step_ws, 0, {1, 0}};
    bool fused = false;   // LayerNorm rows and weight cast in one launch (small shapes)
    if (M > 0) {
        const CastJob wj{weight, N, K, fwd->scale + 1, hist + 1, ctx->w_q, ctx->w_qt,
                         fwd->scale_inv + 1, ctx->w_scale_inv};
        FP8LN_TRY(launch_fwd_prologue(M, (int)K, x, gamma, beta, recipe->ln_eps, f,
                                      fwd->scale + 0, hist + 0, ctx->ln_q, ctx->mean, ctx->rstd,
                                      &wj, ctx->reuse_weight_codes ? 0 : 1, &fused, st,
                                      step_ws ? &upd : nullptr),
                  "forward prologue launch");
    }
    if (step_ws && !fused)   // the update as its own launch, before anything reads a scale
        FP8LN_TRY(launch_scaling_update(hist, fwd->scale, fwd->scale_inv,
                                        recipe->amax_history_len, fwd->n_slots, recipe->margin,
                                        fp8_max_of(f), st),
                  "scaling_update launch");
    if (M > 0) {
        if (!fused)
            FP8LN_TRY(launch_ln_cast_amax(M, (int)K, x, gamma, beta, recipe->ln_eps, f,
                                          fwd->scale + 0, hist + 0, ctx->ln_q, ctx->mean,
                                          ctx->rstd, st),
                      "ln_cast_amax launch");
        if (ctx->ln_qt) FP8LN_TRY(launch_transpose_u8(M, K, ctx->ln_q, ctx->ln_qt, st), "transpose");
    }
    if (!ctx->reuse_weight_codes && !fused)
        FP8LN_TRY(launch_cast_amax(N, K, false, weight, f, fwd->scale + 1, hist + 1, ctx->w_q,
                                   ctx->w_qt, nullptr, nullptr, st, fwd->scale_inv + 1,
                                   ctx->w_scale_inv),
                  "weight cast launch");
    GemmParams p = gemm_params(M, N, K, ctx->ln_q, f, ctx->w_q, f, fwd->scale_inv + 0, w_sinv,
                               kEpiBf16Bias);
    p.bias = (const uint16_t*)bias;
    p.out = out;
    if (step_ws && fused) {   // the folded update's roll, by the GEMM's first workgroup
        p.roll_hist = hist;
        p.roll_ws = (uint32_t*)step_ws;
        p.roll_len = recipe->amax_history_len;
        p.roll_slots = fwd->n_slots;
    }
    FP8LN_TRY(launch_gemm(p, st), "gemm launch");
    return FP8LN_OK;
}

int fp8ln_ln_linear_fwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                        int64_t out_features, int32_t params_dtype, const void* x,
                        const void* gamma, const void* beta, const void* weight,
                        const void* bias, void* out, const fp8ln_meta* fwd,
                        const fp8ln_linear_ctx* ctx, void* stream) {
    return ln_linear_fwd_impl(recipe, tokens, in_features, out_features, params_dtype, x, gamma,
                              beta, weight, bias, out, fwd, ctx, nullptr, stream);
}

int fp8ln_ln_linear_fwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                             int64_t out_features, int32_t params_dtype, const void* x,
                             const void* gamma, const void* beta, const void* weight,
                             const void* bias, void* out, const fp8ln_meta* fwd,
                             const fp8ln_linear_ctx* ctx, void* step_ws, void* stream) {
    REQUIRE_PTR(step_ws);
    return ln_linear_fwd_impl(recipe, tokens, in_features, out_features, params_dtype, x, gamma,
                              beta, weight, bias, out, fwd, ctx, step_ws, stream);
}

}  // extern "C"

namespace {

// The step-start scaling update of a backward state block folded into the
// gradient cast, or nothing to fold (nullopt-like: ok false).
struct BwdFold {
    bool ok;
    FusedUpdate upd;
};

BwdFold bwd_fold(const fp8ln_recipe* recipe, const fp8ln_meta* bwd, int bf, void* step_ws,
                 int64_t M) {
    BwdFold f{false, FusedUpdate{bwd->amax_history, bwd->scale, bwd->scale_inv,
                                 recipe->amax_history_len, bwd->n_slots, recipe->margin,
                                 fp8_max_of(bf), (uint32_t*)step_ws, 0, {0, 0}}};
    const int n = bwd->n_slots;
    f.ok = step_ws && M > 0 && (n & (n - 1)) == 0;
    return f;
}

// LayerNormLinear backward; with step_ws, the step-start scaling update of the
// backward state comes first (folded into the gradient cast where it can be).
int ln_linear_bwd_impl(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                       int64_t out_features, int32_t params_dtype, const void* dy,
                       const void* x, const void* gamma, const fp8ln_linear_ctx* ctx,
                       const fp8ln_meta* fwd, const fp8ln_meta* bwd, void* dx, float* dgamma,
                       float* dbeta, float* dweight, float* dbias, void* workspace,
                       size_t workspace_bytes, void* step_ws, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    const int64_t M = tokens, K = in_features, N = out_features;
    if (params_dtype != FP8LN_DTYPE_BF16)
        return fail(FP8LN_ERR_UNSUPPORTED, "params_dtype %d: only bf16 is supported", params_dtype);
    if (M < 0 || M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "tokens %lld must be a multiple of 16", (long long)M);
    if (K <= 0 || K % 16 != 0 || K > 4096)
        return fail(FP8LN_ERR_UNSUPPORTED, "in_features %lld must be a multiple of 16 in 16..4096",
                    (long long)K);
    if (N <= 0 || N % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "out_features %lld must be a positive multiple of 16",
                    (long long)N);
    if ((s = check_meta(fwd, 2, FP8LN_META_FORWARD, "forward"))) return s;
    if ((s = check_meta(bwd, 1, FP8LN_META_BACKWARD, "backward"))) return s;
    REQUIRE_PTR(ctx);
    REQUIRE(ctx->ln_qt && ctx->w_qt && ctx->mean && ctx->rstd,
            "ctx needs ln_qt, w_qt, mean and rstd from a training forward");
    REQUIRE_PTR(gamma); REQUIRE_PTR(dgamma); REQUIRE_PTR(dbeta); REQUIRE_PTR(dweight);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(dweight); REQUIRE_ALIGNED(ctx->w_qt);
    if (M > 0) {
        REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(dx);
        REQUIRE_ALIGNED(dy); REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(dx); REQUIRE_ALIGNED(ctx->ln_qt);
    }
    const LinearWs need = linear_ws(nullptr, M, K, N);
    REQUIRE(workspace && workspace_bytes >= need.bytes, "ln_linear_bwd needs %zu bytes of workspace",
            need.bytes);
    REQUIRE_ALIGNED(workspace);
    CHECK(check_gemm_size(M, K, N, 1, false, "ln_linear_bwd dgrad"));
    CHECK(check_gemm_size(N, K, M, 1, false, "ln_linear_bwd wgrad"));
    if (step_ws) REQUIRE_ALIGNED(step_ws);
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const LinearWs w = linear_ws(workspace, M, K, N);
    const int ff = meta_fp8(recipe, FP8LN_META_FORWARD);
    const int bf = meta_fp8(recipe, FP8LN_META_BACKWARD);
    SumBatch sums;   // dbias, dgamma / dbeta: one launch at the end
    const BwdFold fold = bwd_fold(recipe, bwd, bf, step_ws, M);

    if (step_ws && !fold.ok)
        FP8LN_TRY(launch_scaling_update(bwd->amax_history, bwd->scale, bwd->scale_inv,
                                        recipe->amax_history_len, bwd->n_slots, recipe->margin,
                                        fp8_max_of(bf), st),
                  "scaling_update launch");
    if (fold.ok)
        FP8LN_TRY(launch_cast_amax_step(M, N, dy, bf, fold.upd, w.dy_q, w.dy_qt, dbias, w.cast_ws,
                                        &sums, st),
                  "grad cast launch");
    else
        FP8LN_TRY(launch_cast_amax(M, N, false, dy, bf, bwd->scale + 0, bwd->amax_history + 0,
                                   w.dy_q, w.dy_qt, dbias, w.cast_ws, st, nullptr, nullptr, &sums),
                  "grad cast launch");
    // dgrad: dLN[M][K] = dy_q[M][N] . (w_qt[K][N])^T
    GemmParams dg = gemm_params(M, K, N, w.dy_q, bf, ctx->w_qt, ff, bwd->scale_inv + 0,
                                ctx->w_scale_inv ? ctx->w_scale_inv : fwd->scale_inv + 1,
                                kEpiF32);
    dg.out = w.dln;
    // wgrad: dW[N][K] = dy_qt[N][M] . (ln_qt[K][M])^T
    GemmParams wg = gemm_params(N, K, M, w.dy_qt, bf, ctx->ln_qt, ff, bwd->scale_inv + 0,
                                fwd->scale_inv + 0, kEpiF32);
    wg.out = dweight;
    // independent products: one launch when both are small
    const GemmParams grads[2] = {dg, wg};
    FP8LN_TRY(launch_gemm_group(grads, 2, st), "dgrad / wgrad launch");
    FP8LN_TRY(launch_ln_bwd(M, (int)K, w.dln, false, x, ctx->mean, ctx->rstd, gamma, dx, dgamma, dbeta,
                            w.ln_ws, st, &sums),
              "layernorm_bwd launch");
    if (fold.ok) {   // the folded update's roll, once the cast's window reads are done
        sums.roll_hist = bwd->amax_history;
        sums.roll_ws = (uint32_t*)step_ws;
        sums.roll_len = recipe->amax_history_len;
        sums.roll_slots = bwd->n_slots;
    }
    FP8LN_TRY(launch_sum_batch(sums, st), "column sums launch");
    return FP8LN_OK;
}

}  // namespace

extern "C" {

int fp8ln_ln_linear_bwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                        int64_t out_features, int32_t params_dtype, const void* dy,
                        const void* x, const void* gamma, const fp8ln_linear_ctx* ctx,
                        const fp8ln_meta* fwd, const fp8ln_meta* bwd, void* dx,
                        float* dgamma, float* dbeta, float* dweight, float* dbias,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return ln_linear_bwd_impl(recipe, tokens, in_features, out_features, params_dtype, dy, x,
                              gamma, ctx, fwd, bwd, dx, dgamma, dbeta, dweight, dbias, workspace,
                              workspace_bytes, nullptr, stream);
}

int fp8ln_ln_linear_bwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                             int64_t out_features, int32_t params_dtype, const void* dy,
                             const void* x, const void* gamma, const fp8ln_linear_ctx* ctx,
                             const fp8ln_meta* fwd, const fp8ln_meta* bwd, void* dx,
                             float* dgamma, float* dbeta, float* dweight, float* dbias,
                             void* workspace, size_t workspace_bytes, void* step_ws,
                             void* stream) {
    REQUIRE_PTR(step_ws);
    return ln_linear_bwd_impl(recipe, tokens, in_features, out_features, params_dtype, dy, x,
                              gamma, ctx, fwd, bwd, dx, dgamma, dbeta, dweight, dbias, workspace,
                              workspace_bytes, step_ws, stream);
}

// LayerNormMLP forward; with step_ws, the step-start scaling update of the
// forward state comes first (folded in when the prologue launch serves the shape).
static int ln_mlp_fwd_impl(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden,
                           int64_t ffn, int32_t params_dtype, const void* x, const void* gamma,
                           const void* beta, const void* w1, const void* b1, const void* w2,
                           const void* b2, void* out, const fp8ln_meta* fwd,
                           const fp8ln_mlp_ctx* ctx, void* step_ws, void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    const int64_t M = tokens, H = hidden, F = ffn;
    REQUIRE(M >= 0, "tokens < 0");
    if (params_dtype != FP8LN_DTYPE_BF16)
        return fail(FP8LN_ERR_UNSUPPORTED, "params_dtype %d: only bf16 is supported", params_dtype);
    if (H <= 0 || H % 16 != 0 || H > 8192)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld must be a multiple of 16 in 16..8192",
                    (long long)H);
    if (F <= 0 || F % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "ffn %lld must be a positive multiple of 16",
                    (long long)F);
    if ((s = check_meta(fwd, 4, FP8LN_META_FORWARD, "forward"))) return s;
    REQUIRE_PTR(ctx);
    REQUIRE((M == 0 || (ctx->ln_q && ctx->g_q)) && ctx->w1_q && ctx->w2_q,
            "ctx.ln_q, w1_q, w2_q and g_q are required");
    if ((ctx->ln_qt || ctx->g_qt) && M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "transposed activations need tokens %% 16 == 0");
    REQUIRE(!ctx->reuse_weight_codes || ctx->w_scale_inv,
            "reuse_weight_codes needs ctx.w_scale_inv from an earlier forward");
    REQUIRE_PTR(gamma); REQUIRE_PTR(beta);
    if (!ctx->reuse_weight_codes) {
        REQUIRE_PTR(w1); REQUIRE_PTR(w2); REQUIRE_ALIGNED(w1); REQUIRE_ALIGNED(w2);
    }
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(beta);
    REQUIRE_ALIGNED(ctx->w1_q); REQUIRE_ALIGNED(ctx->w2_q);
    if (ctx->w1_qt) REQUIRE_ALIGNED(ctx->w1_qt);
    if (ctx->w2_qt) REQUIRE_ALIGNED(ctx->w2_qt);
    if (b1) REQUIRE_ALIGNED(b1);
    if (b2) REQUIRE_ALIGNED(b2);
    if (M > 0) {
        REQUIRE_PTR(x); REQUIRE_PTR(out);
        REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(out); REQUIRE_ALIGNED(ctx->ln_q);
        REQUIRE_ALIGNED(ctx->g_q);
        if (ctx->ln_qt) REQUIRE_ALIGNED(ctx->ln_qt);
        if (ctx->g_qt) REQUIRE_ALIGNED(ctx->g_qt);
        if (ctx->h) REQUIRE_ALIGNED(ctx->h);
    }
    if (ctx->ln_qt) CHECK(check_transpose_rows(M, "ln_mlp_fwd"));
    CHECK(check_gemm_size(M, F, H, 1, false, "ln_mlp_fwd fc1"));
    CHECK(check_gemm_size(M, H, F, 1, false, "ln_mlp_fwd fc2"));
    if (step_ws) REQUIRE_ALIGNED(step_ws);
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const int f = meta_fp8(recipe, FP8LN_META_FORWARD);
    float* hist = fwd->amax_history;
    // FP8 weight storage: reuse the codes (and their scale_inv) of an earlier
    // forward of this ctx, or cast now and record the scale_inv of each
    float* wsi = ctx->w_scale_inv;
    const float* w1_sinv = wsi ? wsi + 0 : fwd->scale_inv + 1;
    const float* w2_sinv = wsi ? wsi + 1 : fwd->scale_inv + 3;
    FusedUpdate upd{hist, fwd->scale, fwd->scale_inv, recipe->amax_history_len, fwd->n_slots,
                    recipe->margin, fp8_max_of(f), (uint32_t*)step_ws, 0, {1, 3}};
    bool fused = false;   // LayerNorm rows and both weight casts in one launch (small shapes)
    if (M > 0) {
        const CastJob wj[2] = {
            {w1, F, H, fwd->scale + 1, hist + 1, ctx->w1_q, ctx->w1_qt, fwd->scale_inv + 1,
             wsi ? wsi + 0 : nullptr},
            {w2, H, F, fwd->scale + 3, hist + 3, ctx->w2_q, ctx->w2_qt, fwd->scale_inv + 3,
             wsi ? wsi + 1 : nullptr}};
        FP8LN_TRY(launch_fwd_prologue(M, (int)H, x, gamma, beta, recipe->ln_eps, f,
                                      fwd->scale + 0, hist + 0, ctx->ln_q, ctx->mean, ctx->rstd,
                                      wj, ctx->reuse_weight_codes ? 0 : 2, &fused, st,
                                      step_ws ? &upd : nullptr),
                  "forward prologue launch");
    }
    if (step_ws && !fused)   // the update as its own launch, before anything reads a scale
        FP8LN_TRY(launch_scaling_update(hist, fwd->scale, fwd->scale_inv,
                                        recipe->amax_history_len, fwd->n_slots, recipe->margin,
                                        fp8_max_of(f), st),
                  "scaling_update launch");
    // folded update: the GELU output's amax joins the others in step_ws, and the
    // fc2 GEMM's first workgroup rolls the history
    const bool roll = step_ws && fused;
    if (M > 0) {
        if (!fused)
            FP8LN_TRY(launch_ln_cast_amax(M, (int)H, x, gamma, beta, recipe->ln_eps, f,
                                          fwd->scale + 0, hist + 0, ctx->ln_q, ctx->mean,
                                          ctx->rstd, st),
                      "ln_cast_amax launch");
        if (ctx->ln_qt) FP8LN_TRY(launch_transpose_u8(M, H, ctx->ln_q, ctx->ln_qt, st), "transpose");
    }
    if (!ctx->reuse_weight_codes && !fused) {
        FP8LN_TRY(launch_cast_amax(F, H, false, w1, f, fwd->scale + 1, hist + 1, ctx->w1_q,
                                   ctx->w1_qt, nullptr, nullptr, st, fwd->scale_inv + 1,
                                   wsi ? wsi + 0 : nullptr),
                  "fc1 weight cast launch");
        FP8LN_TRY(launch_cast_amax(H, F, false, w2, f, fwd->scale + 3, hist + 3, ctx->w2_q,
                                   ctx->w2_qt, nullptr, nullptr, st, fwd->scale_inv + 3,
                                   wsi ? wsi + 1 : nullptr),
                  "fc2 weight cast launch");
    }
    GemmParams p1 = gemm_params(M, F, H, ctx->ln_q, f, ctx->w1_q, f, fwd->scale_inv + 0, w1_sinv,
                                kEpiGeluFp8);
    p1.bias = (const uint16_t*)b1;
    p1.h_out = ctx->h;
    p1.q_out = ctx->g_q;
    p1.q_out_t = ctx->g_qt;
    p1.q_scale = fwd->scale + 2;
    p1.q_amax = roll ? (float*)((uint32_t*)step_ws + 2) : hist + 2;
    p1.q_fp8 = f;
    p1.gelu_erf = recipe->activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(p1, st), "fc1 launch");
    GemmParams p2 = gemm_params(M, H, F, ctx->g_q, f, ctx->w2_q, f, fwd->scale_inv + 2, w2_sinv,
                                kEpiBf16Bias);
    p2.bias = (const uint16_t*)b2;
    p2.out = out;
    if (roll) {
        p2.roll_hist = hist;
        p2.roll_ws = (uint32_t*)step_ws;
        p2.roll_len = recipe->amax_history_len;
        p2.roll_slots = fwd->n_slots;
    }
    FP8LN_TRY(launch_gemm(p2, st), "fc2 launch");
    return FP8LN_OK;
}

int fp8ln_ln_mlp_fwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden, int64_t ffn,
                     int32_t params_dtype, const void* x, const void* gamma, const void* beta,
                     const void* w1, const void* b1, const void* w2, const void* b2, void* out,
                     const fp8ln_meta* fwd, const fp8ln_mlp_ctx* ctx, void* stream) {
    return ln_mlp_fwd_impl(recipe, tokens, hidden, ffn, params_dtype, x, gamma, beta, w1, b1, w2,
                           b2, out, fwd, ctx, nullptr, stream);
}

int fp8ln_ln_mlp_fwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden,
                          int64_t ffn, int32_t params_dtype, const void* x, const void* gamma,
                          const void* beta, const void* w1, const void* b1, const void* w2,
                          const void* b2, void* out, const fp8ln_meta* fwd,
                          const fp8ln_mlp_ctx* ctx, void* step_ws, void* stream) {
    REQUIRE_PTR(step_ws);
    return ln_mlp_fwd_impl(recipe, tokens, hidden, ffn, params_dtype, x, gamma, beta, w1, b1, w2,
                           b2, out, fwd, ctx, step_ws, stream);
}

}  // extern "C"

namespace {

// LayerNormMLP backward; with step_ws, the step-start scaling update of the
// backward state comes first (folded into the gradient cast where it can be; the
// fc1 gradient's amax is then recorded with the cast's).
int ln_mlp_bwd_impl(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden, int64_t ffn,
                    int32_t params_dtype, const void* dy, const void* x, const void* gamma,
                    const fp8ln_mlp_ctx* ctx, const fp8ln_meta* fwd, const fp8ln_meta* bwd,
                    void* dx, float* dgamma, float* dbeta, float* dw1, float* db1, float* dw2,
                    float* db2, void* workspace, size_t workspace_bytes, void* step_ws,
                    void* stream) {
    int s = check_recipe(recipe);
    if (s) return s;
    const int64_t M = tokens, H = hidden, F = ffn;
    if (params_dtype != FP8LN_DTYPE_BF16)
        return fail(FP8LN_ERR_UNSUPPORTED, "params_dtype %d: only bf16 is supported", params_dtype);
    if (M < 0 || M % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "tokens %lld must be a multiple of 16", (long long)M);
    if (H <= 0 || H % 16 != 0 || H > 4096)
        return fail(FP8LN_ERR_UNSUPPORTED, "hidden %lld must be a multiple of 16 in 16..4096",
                    (long long)H);
    if (F <= 0 || F % 16 != 0)
        return fail(FP8LN_ERR_UNSUPPORTED, "ffn %lld must be a positive multiple of 16",
                    (long long)F);
    if ((s = check_meta(fwd, 4, FP8LN_META_FORWARD, "forward"))) return s;
    if ((s = check_meta(bwd, 2, FP8LN_META_BACKWARD, "backward"))) return s;
    REQUIRE_PTR(ctx);
    REQUIRE(ctx->ln_qt && ctx->w1_qt && ctx->w2_qt && ctx->g_qt && ctx->h && ctx->mean && ctx->rstd,
            "ctx needs ln_qt, w1_qt, w2_qt, g_qt, h, mean and rstd from a training forward");
    REQUIRE_PTR(gamma); REQUIRE_PTR(dgamma); REQUIRE_PTR(dbeta); REQUIRE_PTR(dw1);
    REQUIRE_PTR(dw2);
    REQUIRE_ALIGNED(gamma); REQUIRE_ALIGNED(dw1); REQUIRE_ALIGNED(dw2);
    REQUIRE_ALIGNED(ctx->w1_qt); REQUIRE_ALIGNED(ctx->w2_qt);
    if (M > 0) {
        REQUIRE_PTR(dy); REQUIRE_PTR(x); REQUIRE_PTR(dx);
        REQUIRE_ALIGNED(dy); REQUIRE_ALIGNED(x); REQUIRE_ALIGNED(dx);
        REQUIRE_ALIGNED(ctx->ln_qt); REQUIRE_ALIGNED(ctx->g_qt); REQUIRE_ALIGNED(ctx->h);
    }
    const MlpWs need = mlp_ws(nullptr, M, H, F);
    REQUIRE(workspace && workspace_bytes >= need.bytes, "ln_mlp_bwd needs %zu bytes of workspace",
            need.bytes);
    REQUIRE_ALIGNED(workspace);
    CHECK(check_gemm_size(M, F, H, 1, true, "ln_mlp_bwd fc2 dgrad"));
    CHECK(check_gemm_size(H, F, M, 1, false, "ln_mlp_bwd wgrad"));
    CHECK(check_gemm_size(M, H, F, 1, false, "ln_mlp_bwd fc1 dgrad"));
    if (step_ws) REQUIRE_ALIGNED(step_ws);
    if ((s = check_current_device())) return s;
    hipStream_t st = as_stream(stream);
    const MlpWs w = mlp_ws(workspace, M, H, F);
    const int ff = meta_fp8(recipe, FP8LN_META_FORWARD);
    const int bf = meta_fp8(recipe, FP8LN_META_BACKWARD);
    SumBatch sums;   // db2, db1, dgamma / dbeta: one launch at the end
    const BwdFold fold = bwd_fold(recipe, bwd, bf, step_ws, M);

    if (step_ws && !fold.ok)
        FP8LN_TRY(launch_scaling_update(bwd->amax_history, bwd->scale, bwd->scale_inv,
                                        recipe->amax_history_len, bwd->n_slots, recipe->margin,
                                        fp8_max_of(bf), st),
                  "scaling_update launch");
    if (fold.ok)
        FP8LN_TRY(launch_cast_amax_step(M, H, dy, bf, fold.upd, w.dy_q, w.dy_qt, db2, w.cast_ws,
                                        &sums, st),
                  "fc2 grad cast launch");
    else
        FP8LN_TRY(launch_cast_amax(M, H, false, dy, bf, bwd->scale + 0, bwd->amax_history + 0,
                                   w.dy_q, w.dy_qt, db2, w.cast_ws, st, nullptr, nullptr, &sums),
                  "fc2 grad cast launch");
    // fc2 dgrad with the GELU derivative and the fc1 gradient cast fused:
    // dH[M][F] = dy_q[M][H] . (w2_qt[F][H])^T * gelu'(h) -> dh_q, dh_qt, amax, db1
    GemmParams dg2 = gemm_params(M, F, H, w.dy_q, bf, ctx->w2_qt, ff, bwd->scale_inv + 0,
                                 ctx->w_scale_inv ? ctx->w_scale_inv + 1 : fwd->scale_inv + 3,
                                 kEpiDGeluFp8);
    dg2.h_in = ctx->h;
    dg2.q_out = w.dh_q;
    dg2.q_out_t = w.dh_qt;
    dg2.q_scale = bwd->scale + 1;
    // folded update: the history is rolled after the last kernel, so the amax goes
    // to the step workspace as the cast's does
    dg2.q_amax = fold.ok ? (float*)((uint32_t*)step_ws + 1) : bwd->amax_history + 1;
    dg2.q_fp8 = bf;
    dg2.col_partial = db1 ? w.dh_part : nullptr;
    dg2.gelu_erf = recipe->activation == FP8LN_GELU_ERF;
    FP8LN_TRY(launch_gemm(dg2, st), "fc2 dgrad launch");
    if (db1 && !sums.add(w.dh_part, M > 0 ? gemm_partial_rows(M, F, H) : 0, F, db1, nullptr, F))
        return fail(FP8LN_ERR_INVALID_ARG, "internal: column sum batch full");
    // fc2 wgrad: dW2[H][F] = dy_qt[H][M] . (g_qt[F][M])^T
    GemmParams wg2 = gemm_params(H, F, M, w.dy_qt, bf, ctx->g_qt, ff, bwd->scale_inv + 0,
                                 fwd->scale_inv + 2, kEpiF32);
    wg2.out = dw2;
    // fc1 dgrad: dLN[M][H] = dh_q[M][F] . (w1_qt[H][F])^T
    GemmParams dg1 = gemm_params(M, H, F, w.dh_q, bf, ctx->w1_qt, ff, bwd->scale_inv + 1,
                                 ctx->w_scale_inv ? ctx->w_scale_inv + 0 : fwd->scale_inv + 1,
                                 kEpiF32);
    dg1.out = w.dln;
    // fc1 wgrad: dW1[F][H] = dh_qt[F][M] . (ln_qt[H][M])^T
    GemmParams wg1 = gemm_params(F, H, M, w.dh_qt, bf, ctx->ln_qt, ff, bwd->scale_inv + 1,
                                 fwd->scale_inv + 0, kEpiF32);
    wg1.out = dw1;
    // three independent products: one launch when all are small
    const GemmParams grads[3] = {wg2, dg1, wg1};
    FP8LN_TRY(launch_gemm_group(grads, 3, st), "fc2 wgrad / fc1 dgrad / fc1 wgrad launch");
    FP8LN_TRY(launch_ln_bwd(M, (int)H, w.dln, false, x, ctx->mean, ctx->rstd, gamma, dx, dgamma, dbeta,
                            w.ln_ws, st, &sums),
              "layernorm_bwd launch");
    if (fold.ok) {   // the folded update's roll, once the cast's window reads are done
        sums.roll_hist = bwd->amax_history;
        sums.roll_ws = (uint32_t*)step_ws;
        sums.roll_len = recipe->amax_history_len;
        sums.roll_slots = bwd->n_slots;
    }
    FP8LN_TRY(launch_sum_batch(sums, st), "column sums launch");
    return FP8LN_OK;
}

}  // namespace

extern "C" {

int fp8ln_ln_mlp_bwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden, int64_t ffn,
                     int32_t params_dtype, const void* dy, const void* x, const void* gamma,
                     const fp8ln_mlp_ctx* ctx, const fp8ln_meta* fwd, const fp8ln_meta* bwd,
                     void* dx, float* dgamma, float* dbeta, float* dw1, float* db1, float* dw2,
                     float* db2, void* workspace, size_t workspace_bytes, void* stream) {
    return ln_mlp_bwd_impl(recipe, tokens, hidden, ffn, params_dtype, dy, x, gamma, ctx, fwd, bwd,
                           dx, dgamma, dbeta, dw1, db1, dw2, db2, workspace, workspace_bytes,
                           nullptr, stream);
}

int fp8ln_ln_mlp_bwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden,
                          int64_t ffn, int32_t params_dtype, const void* dy, const void* x,
                          const void* gamma, const fp8ln_mlp_ctx* ctx, const fp8ln_meta* fwd,
                          const fp8ln_meta* bwd, void* dx, float* dgamma, float* dbeta,
                          float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                          size_t workspace_bytes, void* step_ws, void* stream) {
    REQUIRE_PTR(step_ws);
    return ln_mlp_bwd_impl(recipe, tokens, hidden, ffn, params_dtype, dy, x, gamma, ctx, fwd, bwd,
                           dx, dgamma, dbeta, dw1, db1, dw2, db2, workspace, workspace_bytes,
                           step_ws, stream);
}

}  // extern "C"
