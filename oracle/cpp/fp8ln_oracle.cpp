// CPU oracle of the FP8 delayed-scaling LayerNormLinear / LayerNormMLP step, in
// plain C++17 (TEST INFRASTRUCTURE ONLY: the test suite, the package's smoke
// check and the benchmark's CPU-baseline leg may load it; the HIP library never
// does, and this file shares no code, header or table with it).
//
// It computes what the pages describe, step by step, in float64 (binary32 where
// the recipe's own state is binary32):
//  * "Accelerating Transformer Training with NVIDIA Transformer Engine, Fused
//    Kernels, BF16, FP8, and GPU Benchmarking" (tutorial): LayerNormLinear(H, 3H)
//    and LayerNormMLP(H, 4H) with bf16 params and a DelayedScaling recipe
//    (setup listing); HYBRID or E4M3 formats, amax_history_len 16 or 1024, the
//    "max" reduction ("things to try"); the per-tensor scale vector and the 2-D
//    amax history with row 0 the newest (benchmark listing, FP8 state).
//  * "Turbo-charging your transformer training: a hands-on guide": LayerNormMLP
//    = layer norm, two linear layers and GELU ("The building blocks"); delayed
//    scaling tracks each tensor's amax and rescales it, HYBRID mixes E4M3 and
//    E5M2, activations are cast to FP8 with the scaling and gradients come back
//    in BF16/FP32 ("Playing with lower-precision formats: BF16 vs FP8").
//
// Readings where the pages are silent (the same as the Python oracle's):
//  * FP8 formats: OCP E4M3 (bias 7, no infinities, max 448) and E5M2 (bias 15,
//    max 57344); encoding = the nearest value of the decode table, ties to the
//    even code, saturating (infinities included), sign of zero kept, NaN -> 0x7F.
//  * scale = fp8_max / max(history) / 2^margin (binary32 division, then exact
//    2^-margin), kept when that is unusable; scale_inv = 1 / scale (binary32);
//    the update rolls the history down one row and zeroes row 0.
//  * LayerNorm: two-pass mean and biased variance, rstd = 1 / sqrt(var + eps).
//  * amax = binary32 rounding of max |value before scaling| (NaN wins).
//  * GEMM: C = (sum_k A[i][k] B[j][k]) * sinv_a * sinv_b + bias, on the decoded
//    codes; the sum is exact (integer multiples of the formats' smallest steps,
//    accumulated in 64- or 128-bit integers) and rounded once to float64.
//  * MLP: GELU (tanh form by default, erf form as the alternative) on the fp64
//    fc1 output h; h is stored as bf16 for the backward's GELU'.
//  * Backward: dgrad on the forward's FP8 weight codes, wgrad on the forward's
//    FP8 activation codes, bias gradients from the unquantised gradient.
//
// Loops over rows run under OpenMP when built with -fopenmp; every row's
// arithmetic is the same in any thread count.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum { kE4M3 = 0, kE5M2 = 1 };
enum { kFormatE4M3 = 0, kFormatHybrid = 1, kFormatE5M2 = 2 };
enum { kGeluTanh = 0, kGeluErf = 1 };

// One FP8 format: its decode table, the sorted finite non-negative values and
// each code's value as an integer multiple of 2^-unit_exp (the subnormal step).
struct Format {
    int ebits, mbits, bias;
    double maxv;
    int max_code;          // largest finite positive code
    int unit_exp;          // value = units * 2^-unit_exp
    double table[256];
    bool finite[256];
    int64_t units[256];
    std::vector<double> pos;   // pos[c] = value of code c, c = 0 .. max_code
};

double decode_bits(int code, int ebits, int mbits, int bias, bool is_e4m3) {
    const double sign = (code & 0x80) ? -1.0 : 1.0;
    const int e = (code >> mbits) & ((1 << ebits) - 1);
    const int m = code & ((1 << mbits) - 1);
    const int emax = (1 << ebits) - 1;
    if (is_e4m3 && e == emax && m == (1 << mbits) - 1) return std::nan("");
    if (!is_e4m3 && e == emax) return m == 0 ? sign * INFINITY : std::nan("");
    if (e == 0) return sign * std::ldexp((double)m, 1 - bias - mbits);
    return sign * std::ldexp((double)((1 << mbits) + m), e - bias - mbits);
}

Format make_format(int fmt) {
    Format F;
    const bool e4 = fmt == kE4M3;
    F.ebits = e4 ? 4 : 5;
    F.mbits = e4 ? 3 : 2;
    F.bias = e4 ? 7 : 15;
    F.unit_exp = F.bias - 1 + F.mbits;   // subnormal step 2^(1 - bias - mbits)
    for (int c = 0; c < 256; ++c) {
        F.table[c] = decode_bits(c, F.ebits, F.mbits, F.bias, e4);
        F.finite[c] = std::isfinite(F.table[c]);
        F.units[c] = F.finite[c] ? (int64_t)std::ldexp(F.table[c], F.unit_exp) : 0;
    }
    F.max_code = 0;
    for (int c = 0; c < 128; ++c)
        if (F.finite[c]) F.max_code = c;
    F.maxv = F.table[F.max_code];
    F.pos.assign(F.table, F.table + F.max_code + 1);
    return F;
}

const Format& format(int fmt) {
    static const Format e4 = make_format(kE4M3);
    static const Format e5 = make_format(kE5M2);
    return fmt == kE4M3 ? e4 : e5;
}

// The encoder: the nearest table value, ties to the even code, saturating.
uint8_t encode1(double v, const Format& F) {
    if (std::isnan(v)) return 0x7F;
    const double a = std::fabs(v);
    int mag;
    if (a >= F.maxv) {
        mag = F.max_code;
    } else {
        const int lo = (int)(std::upper_bound(F.pos.begin(), F.pos.end(), a) - F.pos.begin()) - 1;
        const int hi = lo + 1;
        const double mid = (F.pos[lo] + F.pos[hi]) * 0.5;   // exact: short binary fractions
        if (a > mid) mag = hi;
        else if (a < mid) mag = lo;
        else mag = (lo & 1) ? hi : lo;
    }
    return (uint8_t)(mag | (std::signbit(v) ? 0x80 : 0));
}

double bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
}

// float64 -> bf16 bits, one rounding to nearest even (8 significant bits, the
// subnormal spacing 2^-133 as the floor); past the largest finite value -> inf.
uint16_t bf16_round(double v) {
    if (std::isnan(v)) return 0x7FC0;
    int e = 0;
    std::frexp(v, &e);
    const int q = std::max(e - 8, -133);
    double r = std::ldexp(std::nearbyint(std::ldexp(v, -q)), q);
    const double bmax = std::ldexp(2.0 - std::ldexp(1.0, -7), 127);
    if (std::fabs(r) > bmax) r = std::copysign(INFINITY, v);
    const float f = (float)r;   // exact: r has at most 8 significant bits
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

// binary32 rounding of max |v| (NaN wins; empty -> 0).
float amax_of(const double* v, int64_t n) {
    double m = 0.0;
    bool nan = false;
    for (int64_t i = 0; i < n; ++i) {
        if (std::isnan(v[i])) nan = true;
        else m = std::max(m, std::fabs(v[i]));
    }
    return nan ? std::nanf("") : (float)m;
}

float fp8_max_f(int fmt) { return fmt == kE4M3 ? 448.0f : 57344.0f; }

}  // namespace

extern "C" {

// ---- codec ----------------------------------------------------------------------

void orc_decode_table(int fmt, double* out) {
    const Format& F = format(fmt);
    for (int c = 0; c < 256; ++c) out[c] = F.table[c];
}

void orc_encode(const double* v, int64_t n, int fmt, uint8_t* out) {
    const Format& F = format(fmt);
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) out[i] = encode1(v[i], F);
}

// out[i] = encode(binary32 with bit pattern start + i (mod 2^32)).
void orc_encode_f32_range(uint32_t start, int64_t count, int fmt, uint8_t* out) {
    const Format& F = format(fmt);
#pragma omp parallel for schedule(static) if (count > (1 << 16))
    for (int64_t i = 0; i < count; ++i) {
        const uint32_t u = start + (uint32_t)i;
        float f;
        std::memcpy(&f, &u, 4);
        out[i] = encode1((double)f, F);
    }
}

// Exhaustive check of the encoder over every binary32 input of one sign (0: +,
// 1: -): walking the patterns in value order, the code's position in value
// order never decreases (monotone), NaN patterns give 0x7F, and at every
// transition between two codes the binary32 values on either side lie on the
// correct side of the two codes' midpoint (ties to the even code).  A monotone
// step function that switches exactly at the midpoints is the nearest-value
// encoder, so this proves the encoder equal to a brute-force nearest search on
// every input.  Returns the number of violations.
int64_t orc_encode_check_sign(int fmt, int negative) {
    const Format& F = format(fmt);
    int64_t bad = 0;
    const uint32_t sbit = negative ? 0x80000000u : 0u;
    const int64_t n = int64_t(1) << 31;   // every pattern of this sign
    const int64_t chunk = int64_t(1) << 20;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad)
    for (int64_t c0 = 0; c0 < n; c0 += chunk) {
        int prev = -1;
        double prev_v = 0.0;
        for (int64_t i = c0; i < c0 + chunk + 1 && i < n; ++i) {
            const uint32_t u = sbit | (uint32_t)i;   // magnitude grows with i
            float f;
            std::memcpy(&f, &u, 4);
            const uint8_t q = encode1((double)f, F);
            if (std::isnan(f)) {
                bad += q != 0x7F;
                continue;
            }
            bad += ((q & 0x80) != 0) != (negative != 0);
            const int mag = q & 0x7F;
            if (mag > F.max_code) { ++bad; continue; }
            if (prev >= 0 && mag != prev) {
                // a transition between two adjacent finite values
                if (mag != prev + 1) { ++bad; }
                else {
                    const double a = std::fabs((double)f), pa = std::fabs(prev_v);
                    const double mid = (F.pos[prev] + F.pos[mag]) * 0.5;
                    const bool even_hi = (mag & 1) == 0;
                    // the last input that gave `prev` lies below the midpoint (or on it,
                    // when the tie goes to the lower, even code) and this one above
                    if (pa > mid || (pa == mid && even_hi)) ++bad;
                    if (a < mid || (a == mid && !even_hi)) ++bad;
                }
            }
            prev = mag;
            prev_v = (double)f;
        }
    }
    return bad;
}

void orc_bf16_decode(const uint16_t* b, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_value(b[i]);
}

void orc_bf16_round(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
}

// ---- delayed scaling --------------------------------------------------------------

// For every slot: a = max over the history column (NaN wins); when a is finite and
// > 0, scale = fp8_max / a (binary32) times 2^-margin, unless that is not a finite
// positive number; scale_inv = 1 / scale; then roll the rows down and zero row 0.
void orc_scaling_update(float* hist, float* scale, float* scale_inv, int len, int n_slots,
                        const int* fmts, int margin) {
    for (int s = 0; s < n_slots; ++s) {
        float a = 0.0f;
        bool nan = false;
        for (int i = 0; i < len; ++i) {
            const float h = hist[(int64_t)i * n_slots + s];
            if (std::isnan(h)) nan = true;
            else a = i == 0 ? h : std::max(a, h);
        }
        if (nan) a = std::nanf("");
        if (std::isfinite(a) && a > 0.0f) {
            volatile float q = fp8_max_f(fmts[s]) / a;   // one binary32 division
            const float nw = std::ldexp((float)q, -margin);
            if (std::isfinite(nw) && nw > 0.0f) scale[s] = nw;
        }
        volatile float inv = 1.0f / scale[s];
        scale_inv[s] = inv;
    }
    for (int i = len - 1; i >= 1; --i)
        std::memcpy(hist + (int64_t)i * n_slots, hist + (int64_t)(i - 1) * n_slots,
                    sizeof(float) * n_slots);
    std::memset(hist, 0, sizeof(float) * n_slots);
}

// Row 0 keeps the largest amax of the step (NaN wins).
void orc_record_amax(float* hist, int slot, float a) {
    const float cur = hist[slot];
    hist[slot] = (std::isnan(a) || std::isnan(cur)) ? std::nanf("") : std::max(cur, a);
}

// ---- LayerNorm -------------------------------------------------------------------

}  // extern "C"

namespace {

// One row: mean = sum x / H, var = sum (x - mean)^2 / H, rstd = 1 / sqrt(var + eps),
// y = (x - mean) * rstd * gamma + beta.
void layernorm_row(const double* xr, int64_t H, const double* gamma, const double* beta,
                   double eps, double* y, double* mean, double* rstd) {
    double s = 0.0;
    for (int64_t j = 0; j < H; ++j) s += xr[j];
    const double mu = s / (double)H;
    double v = 0.0;
    for (int64_t j = 0; j < H; ++j) v += (xr[j] - mu) * (xr[j] - mu);
    const double rs = 1.0 / std::sqrt(v / (double)H + eps);
    for (int64_t j = 0; j < H; ++j) y[j] = (xr[j] - mu) * rs * gamma[j] + beta[j];
    *mean = mu;
    *rstd = rs;
}

}  // namespace

extern "C" {

void orc_layernorm_fwd(const double* x, int64_t rows, int64_t H, const double* gamma,
                       const double* beta, double eps, double* y, double* mean, double* rstd) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        layernorm_row(x + r * H, H, gamma, beta, eps, y + r * H, mean + r, rstd + r);
}

// dx = rstd (g - mean(g) - xhat mean(g xhat)) with g = dy gamma; dgamma, dbeta
// are column sums of dy xhat and dy (rows in order).
void orc_layernorm_bwd(const double* dy, const double* x, const double* gamma, const double* mean,
                       const double* rstd, int64_t rows, int64_t H, double* dx, double* dgamma,
                       double* dbeta) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double c1 = 0.0, c2 = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            const double xh = (x[r * H + j] - mean[r]) * rstd[r];
            const double g = dy[r * H + j] * gamma[j];
            c1 += g;
            c2 += g * xh;
        }
        c1 /= (double)H;
        c2 /= (double)H;
        for (int64_t j = 0; j < H; ++j) {
            const double xh = (x[r * H + j] - mean[r]) * rstd[r];
            const double g = dy[r * H + j] * gamma[j];
            dx[r * H + j] = rstd[r] * (g - c1 - xh * c2);
        }
    }
    for (int64_t j = 0; j < H; ++j) { dgamma[j] = 0.0; dbeta[j] = 0.0; }
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < H; ++j) {
            const double xh = (x[r * H + j] - mean[r]) * rstd[r];
            dgamma[j] += dy[r * H + j] * xh;
            dbeta[j] += dy[r * H + j];
        }
}

// ---- FP8 cast ---------------------------------------------------------------------

// q = encode(v * scale); returns the tensor's amax (of v, before scaling).
float orc_cast_amax(const double* v, int64_t n, float scale, int fmt, uint8_t* q) {
    const Format& F = format(fmt);
    const double s = (double)scale;
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) q[i] = encode1(v[i] * s, F);
    return amax_of(v, n);
}

// ---- GEMM -------------------------------------------------------------------------

// C[i][j] = (sum_k dec(A[i][k]) dec(B[j][k])) * sinv_a * sinv_b + bias[j], A [M][K],
// B [N][K] codes.  Each code is an integer multiple of its format's smallest step,
// so the sum is accumulated exactly in integers (64-bit where E4M3 x E4M3 cannot
// overflow, 128-bit otherwise) and rounded once to float64; a NaN or infinite
// code makes that output the float64 sum of the decoded values.
void orc_fp8_gemm_tn(const uint8_t* A, int fa, const uint8_t* B, int fb, int64_t M, int64_t N,
                     int64_t K, float sinv_a, float sinv_b, const double* bias, double* C) {
    const Format& Fa = format(fa);
    const Format& Fb = format(fb);
    const int shift = Fa.unit_exp + Fb.unit_exp;
    const bool small = fa == kE4M3 && fb == kE4M3 && K <= (int64_t(1) << 20);
    const double sa = (double)sinv_a, sb = (double)sinv_b;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        const uint8_t* a = A + i * K;
        for (int64_t j = 0; j < N; ++j) {
            const uint8_t* b = B + j * K;
            bool special = false;
            double c;
            if (small) {
                int64_t acc = 0;
                for (int64_t k = 0; k < K; ++k) {
                    special |= !(Fa.finite[a[k]] && Fb.finite[b[k]]);
                    acc += Fa.units[a[k]] * Fb.units[b[k]];
                }
                c = std::ldexp((double)acc, -shift);
            } else {
                __int128 acc = 0;
                for (int64_t k = 0; k < K; ++k) {
                    special |= !(Fa.finite[a[k]] && Fb.finite[b[k]]);
                    acc += (__int128)Fa.units[a[k]] * (__int128)Fb.units[b[k]];
                }
                c = std::ldexp((double)acc, -shift);
            }
            if (special) {
                c = 0.0;
                for (int64_t k = 0; k < K; ++k) c += Fa.table[a[k]] * Fb.table[b[k]];
            }
            c = c * sa * sb;
            if (bias) c += bias[j];
            C[i * N + j] = c;
        }
    }
}

// ---- GELU ---------------------------------------------------------------------------

// tanh form: 0.5 h (1 + tanh(sqrt(2/pi) (h + 0.044715 h^3))); erf form:
// 0.5 h (1 + erf(h / sqrt 2)); and their derivatives.
double gelu1(double h, int act) {
    if (act == kGeluErf) return 0.5 * h * (1.0 + std::erf(h / std::sqrt(2.0)));
    const double c = std::sqrt(2.0 / M_PI);
    return 0.5 * h * (1.0 + std::tanh(c * (h + 0.044715 * std::pow(h, 3.0))));
}

double gelu_grad1(double h, int act) {
    if (act == kGeluErf)
        return 0.5 * (1.0 + std::erf(h / std::sqrt(2.0))) +
               h * std::exp(-0.5 * h * h) / std::sqrt(2.0 * M_PI);
    const double c = std::sqrt(2.0 / M_PI);
    const double t = std::tanh(c * (h + 0.044715 * std::pow(h, 3.0)));
    return 0.5 * (1.0 + t) + 0.5 * h * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * h * h);
}

void orc_gelu(const double* h, int64_t n, int act, double* out) {
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) out[i] = gelu1(h[i], act);
}

void orc_gelu_grad(const double* h, int64_t n, int act, double* out) {
#pragma omp parallel for schedule(static) if (n > (1 << 16))
    for (int64_t i = 0; i < n; ++i) out[i] = gelu_grad1(h[i], act);
}

// ---- module steps -------------------------------------------------------------------

// One module's FP8 state for one direction (binary32, row 0 of hist the newest).
typedef struct {
    float* hist;
    float* scale;
    float* scale_inv;
    int32_t len;
    int32_t n_slots;
} orc_meta;

}  // extern "C"

namespace {

int fwd_fmt(int recipe_format) { return recipe_format == kFormatE5M2 ? kE5M2 : kE4M3; }
int bwd_fmt(int recipe_format) { return recipe_format == kFormatE4M3 ? kE4M3 : kE5M2; }

std::vector<double> decode_bf16(const uint16_t* b, int64_t n) {
    std::vector<double> v((size_t)n);
    for (int64_t i = 0; i < n; ++i) v[(size_t)i] = bf16_value(b[i]);
    return v;
}

// [R][C] codes -> [C][R]
std::vector<uint8_t> transpose(const uint8_t* q, int64_t R, int64_t C) {
    std::vector<uint8_t> t((size_t)(R * C));
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) t[(size_t)(c * R + r)] = q[r * C + c];
    return t;
}

// Column sums over rows, in row order.
void column_sums(const double* v, int64_t R, int64_t C, double* out) {
    for (int64_t c = 0; c < C; ++c) out[c] = 0.0;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) out[c] += v[r * C + c];
}

// The weight's codes and the scale_inv they go with: a fresh cast with the slot's
// scale (its amax recorded), or the stored codes of an earlier forward (FP8
// weight storage: nothing recorded).
float weight_codes(orc_meta* m, int slot, const uint16_t* w, int64_t n, int fmt, int reuse,
                   uint8_t* w_q, float stored_sinv, float* amax_out) {
    if (reuse) {
        *amax_out = std::nanf("");   // not recorded
        return stored_sinv;
    }
    const std::vector<double> wv = decode_bf16(w, n);
    const float a = orc_cast_amax(wv.data(), n, m->scale[slot], fmt, w_q);
    orc_record_amax(m->hist, slot, a);
    *amax_out = a;
    return m->scale_inv[slot];
}

// LayerNorm of x, cast of its output with slot 0's scale, amax into slot 0.
void ln_cast_slot0(orc_meta* m, int fmt, double eps, int64_t M, int64_t H, const uint16_t* x,
                   const uint16_t* g, const uint16_t* b, uint8_t* ln_q, double* y, double* mean,
                   double* rstd, float* amax_out) {
    const std::vector<double> xv = decode_bf16(x, M * H), gv = decode_bf16(g, H),
                              bv = decode_bf16(b, H);
    orc_layernorm_fwd(xv.data(), M, H, gv.data(), bv.data(), eps, y, mean, rstd);
    const float a = orc_cast_amax(y, M * H, m->scale[0], fmt, ln_q);
    orc_record_amax(m->hist, 0, a);
    *amax_out = a;
}

}  // namespace

extern "C" {

// LayerNormLinear forward: ln_q = enc(LN(x) * scale[0]) (amax -> slot 0), w_q =
// enc(W * scale[1]) (amax -> slot 1; or reused), out = ln_q . w_q^T * sinv + bias.
// amaxes[0..1] receive the recorded amaxes (NaN where nothing was recorded);
// *w_sinv receives the scale_inv that goes with w_q.
void orc_ln_linear_fwd(int recipe_format, double eps, int64_t M, int64_t K, int64_t N,
                       const uint16_t* x, const uint16_t* gamma, const uint16_t* beta,
                       const uint16_t* w, const uint16_t* bias, orc_meta* meta, int reuse_w,
                       double* out, uint8_t* ln_q, uint8_t* w_q, float* w_sinv, double* y,
                       double* mean, double* rstd, float* amaxes) {
    const int f = fwd_fmt(recipe_format);
    ln_cast_slot0(meta, f, eps, M, K, x, gamma, beta, ln_q, y, mean, rstd, &amaxes[0]);
    *w_sinv = weight_codes(meta, 1, w, N * K, f, reuse_w, w_q, *w_sinv, &amaxes[1]);
    std::vector<double> bv;
    if (bias) bv = decode_bf16(bias, N);
    orc_fp8_gemm_tn(ln_q, f, w_q, f, M, N, K, meta->scale_inv[0], *w_sinv,
                    bias ? bv.data() : nullptr, out);
}

// Its backward for dy [M][N]: dy_q = enc(dy * bwd.scale[0]) (amax -> bwd slot 0),
// dLN = dy_q . w_q (dgrad, forward weight codes), dW = dy_q^T . ln_q (wgrad, saved
// LN codes), dbias = column sums of dy, then the LayerNorm backward.
void orc_ln_linear_bwd(int recipe_format, int64_t M, int64_t K, int64_t N, const uint16_t* dy,
                       const uint16_t* x, const uint16_t* gamma, const uint8_t* ln_q,
                       const uint8_t* w_q, float w_sinv, const double* mean, const double* rstd,
                       orc_meta* meta_fwd, orc_meta* meta_bwd, double* dx, double* dgamma,
                       double* dbeta, double* dw, double* dbias, double* dln, uint8_t* dy_q,
                       float* dy_amax) {
    const int ff = fwd_fmt(recipe_format), bf = bwd_fmt(recipe_format);
    const std::vector<double> dyv = decode_bf16(dy, M * N);
    *dy_amax = orc_cast_amax(dyv.data(), M * N, meta_bwd->scale[0], bf, dy_q);
    orc_record_amax(meta_bwd->hist, 0, *dy_amax);
    column_sums(dyv.data(), M, N, dbias);
    const std::vector<uint8_t> w_qt = transpose(w_q, N, K);     // [K][N]
    orc_fp8_gemm_tn(dy_q, bf, w_qt.data(), ff, M, K, N, meta_bwd->scale_inv[0], w_sinv, nullptr,
                    dln);
    const std::vector<uint8_t> dy_qt = transpose(dy_q, M, N);   // [N][M]
    const std::vector<uint8_t> ln_qt = transpose(ln_q, M, K);   // [K][M]
    orc_fp8_gemm_tn(dy_qt.data(), bf, ln_qt.data(), ff, N, K, M, meta_bwd->scale_inv[0],
                    meta_fwd->scale_inv[0], nullptr, dw);
    const std::vector<double> xv = decode_bf16(x, M * K), gv = decode_bf16(gamma, K);
    orc_layernorm_bwd(dln, xv.data(), gv.data(), mean, rstd, M, K, dx, dgamma, dbeta);
}

// LayerNormMLP forward: ln_q (slot 0), w1_q (slot 1), h = ln_q . w1_q^T * sinv + b1
// (fp64, stored as bf16 h_bits), g = gelu(h), g_q = enc(g * scale[2]) (slot 2),
// w2_q (slot 3), out = g_q . w2_q^T * sinv + b2.  w_sinv[0..1]: fc1, fc2 weights.
void orc_ln_mlp_fwd(int recipe_format, int activation, double eps, int64_t M, int64_t H,
                    int64_t F, const uint16_t* x, const uint16_t* gamma, const uint16_t* beta,
                    const uint16_t* w1, const uint16_t* b1, const uint16_t* w2,
                    const uint16_t* b2, orc_meta* meta, int reuse_w, double* out, uint8_t* ln_q,
                    uint8_t* w1_q, uint8_t* w2_q, float* w_sinv, double* h, uint16_t* h_bits,
                    double* g, uint8_t* g_q, double* y, double* mean, double* rstd,
                    float* amaxes) {
    const int f = fwd_fmt(recipe_format);
    ln_cast_slot0(meta, f, eps, M, H, x, gamma, beta, ln_q, y, mean, rstd, &amaxes[0]);
    w_sinv[0] = weight_codes(meta, 1, w1, F * H, f, reuse_w, w1_q, w_sinv[0], &amaxes[1]);
    w_sinv[1] = weight_codes(meta, 3, w2, H * F, f, reuse_w, w2_q, w_sinv[1], &amaxes[3]);
    std::vector<double> b1v, b2v;
    if (b1) b1v = decode_bf16(b1, F);
    if (b2) b2v = decode_bf16(b2, H);
    orc_fp8_gemm_tn(ln_q, f, w1_q, f, M, F, H, meta->scale_inv[0], w_sinv[0],
                    b1 ? b1v.data() : nullptr, h);
    orc_gelu(h, M * F, activation, g);
    orc_bf16_round(h, M * F, h_bits);
    amaxes[2] = orc_cast_amax(g, M * F, meta->scale[2], f, g_q);
    orc_record_amax(meta->hist, 2, amaxes[2]);
    orc_fp8_gemm_tn(g_q, f, w2_q, f, M, H, F, meta->scale_inv[2], w_sinv[1],
                    b2 ? b2v.data() : nullptr, out);
}

// Its backward for dy [M][H]: dy_q (bwd slot 0), db2 = column sums of dy,
// dg = dy_q . w2_q, dH = dg * gelu'(bf16 h), dh_q (bwd slot 1), db1 = column sums
// of dH, dW2 = dy_q^T . g_q, dLN = dh_q . w1_q, dW1 = dh_q^T . ln_q, LN backward.
void orc_ln_mlp_bwd(int recipe_format, int activation, int64_t M, int64_t H, int64_t F,
                    const uint16_t* dy, const uint16_t* x, const uint16_t* gamma,
                    const uint8_t* ln_q, const uint8_t* w1_q, const uint8_t* w2_q,
                    const float* w_sinv, const uint16_t* h_bits, const uint8_t* g_q,
                    const double* mean, const double* rstd, orc_meta* meta_fwd,
                    orc_meta* meta_bwd, double* dx, double* dgamma, double* dbeta, double* dw1,
                    double* db1, double* dw2, double* db2, double* dg, double* dh,
                    uint8_t* dy_q, uint8_t* dh_q, double* dln, float* amaxes) {
    const int ff = fwd_fmt(recipe_format), bf = bwd_fmt(recipe_format);
    const std::vector<double> dyv = decode_bf16(dy, M * H);
    amaxes[0] = orc_cast_amax(dyv.data(), M * H, meta_bwd->scale[0], bf, dy_q);
    orc_record_amax(meta_bwd->hist, 0, amaxes[0]);
    column_sums(dyv.data(), M, H, db2);
    const std::vector<uint8_t> w2_qt = transpose(w2_q, H, F);   // [F][H]
    orc_fp8_gemm_tn(dy_q, bf, w2_qt.data(), ff, M, F, H, meta_bwd->scale_inv[0], w_sinv[1],
                    nullptr, dg);
    const std::vector<double> hv = decode_bf16(h_bits, M * F);
    std::vector<double> gp((size_t)(M * F));
    orc_gelu_grad(hv.data(), M * F, activation, gp.data());
    for (int64_t i = 0; i < M * F; ++i) dh[i] = dg[i] * gp[(size_t)i];
    amaxes[1] = orc_cast_amax(dh, M * F, meta_bwd->scale[1], bf, dh_q);
    orc_record_amax(meta_bwd->hist, 1, amaxes[1]);
    column_sums(dh, M, F, db1);
    const std::vector<uint8_t> dy_qt = transpose(dy_q, M, H);   // [H][M]
    const std::vector<uint8_t> g_qt = transpose(g_q, M, F);     // [F][M]
    orc_fp8_gemm_tn(dy_qt.data(), bf, g_qt.data(), ff, H, F, M, meta_bwd->scale_inv[0],
                    meta_fwd->scale_inv[2], nullptr, dw2);
    const std::vector<uint8_t> w1_qt = transpose(w1_q, F, H);   // [H][F]
    orc_fp8_gemm_tn(dh_q, bf, w1_qt.data(), ff, M, H, F, meta_bwd->scale_inv[1], w_sinv[0],
                    nullptr, dln);
    const std::vector<uint8_t> dh_qt = transpose(dh_q, M, F);   // [F][M]
    const std::vector<uint8_t> ln_qt = transpose(ln_q, M, H);   // [H][M]
    orc_fp8_gemm_tn(dh_qt.data(), bf, ln_qt.data(), ff, F, H, M, meta_bwd->scale_inv[1],
                    meta_fwd->scale_inv[0], nullptr, dw1);
    const std::vector<double> xv = decode_bf16(x, M * H), gv = decode_bf16(gamma, H);
    orc_layernorm_bwd(dln, xv.data(), gv.data(), mean, rstd, M, H, dx, dgamma, dbeta);
}

// The standalone LayerNorm + FP8 cast + amax over bf16 rows (the memory-bound
// step alone): codes into q, returns the amax.
float orc_ln_cast_amax(const uint16_t* x, int64_t rows, int64_t H, const uint16_t* gamma,
                       const uint16_t* beta, double eps, float scale, int fmt, uint8_t* q,
                       double* mean, double* rstd) {
    const Format& Fm = format(fmt);
    const std::vector<double> gv = decode_bf16(gamma, H), bv = decode_bf16(beta, H);
    const double s = (double)scale;
    double amax = 0.0;
    int nan = 0;
#pragma omp parallel for schedule(static) reduction(max : amax) reduction(| : nan)
    for (int64_t r = 0; r < rows; ++r) {
        std::vector<double> xr((size_t)H), yr((size_t)H);
        for (int64_t j = 0; j < H; ++j) xr[(size_t)j] = bf16_value(x[r * H + j]);
        double mu, rs;
        layernorm_row(xr.data(), H, gv.data(), bv.data(), eps, yr.data(), &mu, &rs);
        for (int64_t j = 0; j < H; ++j) {
            const double yv = yr[(size_t)j];
            q[r * H + j] = encode1(yv * s, Fm);
            if (std::isnan(yv)) nan = 1;
            else amax = std::max(amax, std::fabs(yv));
        }
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
    return nan ? std::nanf("") : (float)amax;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

}  // extern "C"
