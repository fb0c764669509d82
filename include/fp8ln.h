/*
 * fp8ln: FP8 delayed-scaling LayerNormLinear / LayerNormMLP for AMD MI355X (gfx950).
 *
 * The operation follows two pages on NVIDIA Transformer Engine:
 *  [T] "Accelerating Transformer Training with NVIDIA Transformer Engine, Fused
 *      Kernels, BF16, FP8, and GPU Benchmarking" (tutorial), and
 *  [G] "Turbo-charging your transformer training: a hands-on guide".
 * [T] setup listing builds LayerNormLinear(H, 3H) and LayerNormMLP(H, 4H) with bf16
 * params and a DelayedScaling recipe (format HYBRID, amax_history_len 16,
 * amax_compute_algo "max"); its "things to try" list adds Format.E4M3 and
 * amax_history_len 1024; its benchmark listing reads the per-module state
 * fp8_meta["scaling_fwd"] (a per-tensor scale vector and a 2-D amax history whose
 * row 0 is the most recent).  [G] "The building blocks" describes LayerNormMLP as
 * layer norm, two linear layers and GELU; "Playing with lower-precision formats:
 * BF16 vs FP8" says delayed scaling tracks each tensor's amax and rescales it,
 * that HYBRID mixes E4M3 and E5M2, and that autocast casts activations to FP8 with
 * the scaling and returns gradients in BF16/FP32.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a device pointer unless stated otherwise, and the
 *    caller owns every buffer: inputs, outputs, saved context, FP8 state and
 *    workspace.  The library allocates no device memory (its one fixed device
 *    array, that of fp8ln_ln_linear_bwd_noalloc, comes with the loaded code) and
 *    keeps no pointer after a call returns.  Buffers must stay alive until the stream reaches the
 *    call's kernels.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and runs
 *    asynchronously.  No call synchronises the host or copies data to the host:
 *    scales stay on the device from step to step.
 *  - Arguments are validated before anything is launched.  A call that returns an
 *    error has enqueued nothing.  fp8ln_last_error() gives a message for the most
 *    recent failure on the calling host thread.
 *  - Matrices are row-major and densely packed.  bf16 values are IEEE binary32
 *    values truncated to their top 16 bits (stored as uint16).  FP8 tensors are
 *    uint8 codes in the OCP 8-bit floating point formats: E4M3 (bias 7, no
 *    infinities, largest finite 448) and E5M2 (bias 15, largest finite 57344).
 *    Encoding rounds to nearest, ties to even, saturates to the largest finite
 *    value (infinities included), keeps the sign of zero and writes every NaN as
 *    0x7F.
 *  - Only gfx950 devices are supported; on any other device every compute call
 *    returns FP8LN_ERR_UNSUPPORTED.
 */
#ifndef FP8LN_H
#define FP8LN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
typedef enum {
    FP8LN_OK = 0,
    FP8LN_ERR_INVALID_ARG = -1,   /* null pointer, bad size, bad enum value   */
    FP8LN_ERR_UNSUPPORTED = -2,   /* valid request the library does not serve */
    FP8LN_ERR_HIP = -3            /* a HIP runtime call or launch failed      */
} fp8ln_status;

/* Recipe formats ([T] setup listing: Format.HYBRID; "things to try": Format.E4M3;
 * [G] "Common pitfalls": Format.E5M2).  HYBRID casts forward tensors (LayerNorm
 * output, weights, GELU output) to E4M3 and gradients to E5M2; E4M3 and E5M2 use
 * one format for both directions. */
typedef enum {
    FP8LN_FORMAT_E4M3 = 0,
    FP8LN_FORMAT_HYBRID = 1,
    FP8LN_FORMAT_E5M2 = 2
} fp8ln_format;

/* Encoding of one FP8 tensor. */
typedef enum { FP8LN_E4M3 = 0, FP8LN_E5M2 = 1 } fp8ln_fp8_dtype;

/* params_dtype of the modules ([T] setup listing: params_dtype=torch.bfloat16).
 * FP8LN_DTYPE_F32 is accepted only as the input of fp8ln_cast_amax. */
typedef enum { FP8LN_DTYPE_BF16 = 0, FP8LN_DTYPE_F32 = 1 } fp8ln_dtype;

/* Direction of one FP8 state block (the tutorial's fp8_meta["scaling_fwd"] and its
 * backward counterpart). */
typedef enum { FP8LN_META_FORWARD = 0, FP8LN_META_BACKWARD = 1 } fp8ln_meta_kind;

/* LayerNormMLP activation: GELU with the tanh approximation (the default), or the
 * exact erf form of the plain-PyTorch mirror block's nn.GELU() ([T] model
 * listing). */
typedef enum { FP8LN_GELU_TANH = 0, FP8LN_GELU_ERF = 1 } fp8ln_activation;

/* DelayedScaling recipe ([T] setup listing) plus the module settings the steps
 * need.  amax_compute_algo is always "max".
 *   format            fp8ln_format
 *   amax_history_len  1 .. 1024
 *   margin            0 .. 64; scale = fp8_max / max(history) / 2^margin
 *   ln_eps            LayerNorm epsilon, finite and > 0 (1e-5 by default)
 *   activation        fp8ln_activation of LayerNormMLP */
typedef struct {
    int32_t format;
    int32_t amax_history_len;
    int32_t margin;
    float ln_eps;
    int32_t activation;
} fp8ln_recipe;

/* One direction's FP8 state of one module, all device buffers owned by the caller:
 *   amax_history  float [amax_history_len][n_slots], row 0 = newest
 *   scale         float [n_slots]; must hold finite positive values
 *   scale_inv     float [n_slots]
 *   n_slots       1 .. 8
 *   kind          fp8ln_meta_kind; picks the FP8 format of every slot
 * Slots: LayerNormLinear forward {0: LN output, 1: weight}, backward {0: output
 * gradient}.  LayerNormMLP forward {0: LN output, 1: fc1 weight, 2: GELU output,
 * 3: fc2 weight}, backward {0: fc2 output gradient, 1: fc1 output gradient}. */
typedef struct {
    float* amax_history;
    float* scale;
    float* scale_inv;
    int32_t n_slots;
    int32_t kind;
} fp8ln_meta;

/* What LayerNormLinear's forward saves for its backward (device buffers).
 * M = tokens, K = in_features, N = out_features.
 *   ln_q   uint8 [M][K]  FP8 LayerNorm output (forward format)
 *   ln_qt  uint8 [K][M]  its transpose; may be NULL for a forward-only call
 *   w_q    uint8 [N][K]  FP8 weight
 *   w_qt   uint8 [K][N]  its transpose; may be NULL for a forward-only call
 *   mean   float [M]     row means
 *   rstd   float [M]     row 1/sqrt(var + eps)
 *   w_scale_inv  float [1]  the scale_inv the w_q codes were made with: every
 *                forward that casts the weight writes it, and the GEMMs on w_q /
 *                w_qt dequantise with it.  May be NULL (then the forward meta's
 *                scale_inv is used, which is the same value in a normal step).
 *   reuse_weight_codes  FP8 weight storage ([T] "things to try next": FP8 model
 *                init): 1 = the weight has not changed since a forward of this
 *                ctx wrote w_q (w_qt) and w_scale_inv, so the weight cast is
 *                skipped and those codes are used as they are; that step records
 *                no weight amax.  Needs w_scale_inv.  0 = cast the weight. */
typedef struct {
    uint8_t* ln_q;
    uint8_t* ln_qt;
    uint8_t* w_q;
    uint8_t* w_qt;
    float* mean;
    float* rstd;
    float* w_scale_inv;
    int32_t reuse_weight_codes;
} fp8ln_linear_ctx;

/* What LayerNormMLP's forward saves for its backward (device buffers).
 * M = tokens, H = hidden, F = ffn.
 *   ln_q [M][H], ln_qt [H][M], w1_q [F][H], w1_qt [H][F], w2_q [H][F],
 *   w2_qt [F][H], g_q [M][F] (FP8 GELU output), g_qt [F][M]: uint8
 *   h     uint16 (bf16) [M][F]: fc1 output before GELU
 *   mean, rstd float [M]
 *   w_scale_inv float [2]: scale_inv of the w1 and w2 codes (as for
 *   fp8ln_linear_ctx); reuse_weight_codes: skip both weight casts (as for
 *   fp8ln_linear_ctx).
 * The *_qt transposes and h may be NULL for a forward-only call. */
typedef struct {
    uint8_t* ln_q;
    uint8_t* ln_qt;
    uint8_t* w1_q;
    uint8_t* w1_qt;
    uint8_t* w2_q;
    uint8_t* w2_qt;
    uint16_t* h;
    uint8_t* g_q;
    uint8_t* g_qt;
    float* mean;
    float* rstd;
    float* w_scale_inv;
    int32_t reuse_weight_codes;
} fp8ln_mlp_ctx;

/* Workspace kinds for fp8ln_workspace_size. */
typedef enum {
    FP8LN_OP_CAST_AMAX = 0,        /* a = rows, b = cols (column sums requested) */
    FP8LN_OP_LAYERNORM_BWD = 1,    /* a = rows, b = hidden */
    FP8LN_OP_LN_LINEAR_BWD = 2,    /* a = tokens, b = in_features, c = out_features */
    FP8LN_OP_LN_MLP_BWD = 3,       /* a = tokens, b = hidden, c = ffn */
    FP8LN_OP_GEMM_DGELU_FP8 = 4,   /* a = M, b = N (column sums requested) */
    FP8LN_OP_LINEAR_BWD = 5,       /* a = tokens, b = in_features, c = out_features */
    FP8LN_OP_LN_LINEAR_BWD_BF16 = 6, /* a = tokens, b = in_features, c = out_features */
    FP8LN_OP_TRANSPOSE_BF16 = 7,   /* a = rows, b = cols (column sums requested) */
    FP8LN_OP_LN_MLP_BWD_BF16 = 8   /* a = tokens, b = hidden, c = ffn */
} fp8ln_op;

/* ---- library ------------------------------------------------------------ */

/* Text for a status code (static storage). */
const char* fp8ln_status_string(int status);

/* Message for the most recent failed call on this host thread ("" if none). */
const char* fp8ln_last_error(void);

/* Whether `device` can run this library: 1 = yes, 0 = no (reason written to
 * `reason`, a host buffer of `reason_cap` bytes, may be NULL), < 0 = error.
 * The counterpart of the tutorial's capability probe ([T] setup listing). */
int fp8ln_check_support(int device, char* reason, size_t reason_cap);

/* Bytes of workspace that op needs (see fp8ln_op); 0 for bad arguments. */
size_t fp8ln_workspace_size(int32_t op, int64_t a, int64_t b, int64_t c);

/* ---- delayed-scaling state ([T] benchmark listing; [G] "Playing with
 *      lower-precision formats") ------------------------------------------ */

/* Start a module's state: history = 0, scale = scale_inv = 1. */
int fp8ln_meta_init(const fp8ln_recipe* recipe, const fp8ln_meta* meta, void* stream);

/* Step start: for every slot, a = max over all history rows; if a is finite and
 * > 0, scale = fp8_max / a / 2^margin (binary32 division, then exact scaling by
 * 2^-margin) unless that is not a finite positive number; otherwise the scale is
 * kept.  scale_inv = 1 / scale.  Then every history row moves down one row (the
 * oldest falls off) and row 0 is set to zero; the step's kernels record their
 * amaxes into row 0.  fp8_max is 448 for E4M3 slots and 57344 for E5M2 slots. */
int fp8ln_scaling_update(const fp8ln_recipe* recipe, const fp8ln_meta* meta, void* stream);

/* fp8ln_scaling_update for n state blocks of one recipe (a host array of n
 * fp8ln_meta; each block keeps its own kind and slot count), with the same
 * results, in one launch per 64 blocks: a model updates every module's forward
 * and backward state at the start of its step (the recipe's update touches only
 * a block's own history, so its order among the blocks does not matter). */
int fp8ln_scaling_update_batch(const fp8ln_recipe* recipe, const fp8ln_meta* metas, int32_t n,
                               void* stream);

/* ---- fused LayerNorm + FP8 cast + amax ([T] setup listing, LayerNormLinear;
 *      [G] "The building blocks") ------------------------------------------ */

/* For each of `rows` rows of x (bf16 [rows][hidden]):
 *   mean, var (biased) of the row; rstd = 1 / sqrt(var + recipe->ln_eps);
 *   y = (x - mean) * rstd * gamma + beta         (gamma, beta: bf16 [hidden])
 *   out[r][j] = encode(y * (*scale))              (uint8 [rows][hidden])
 *   out_t[j][r] = out[r][j]                       (optional, may be NULL)
 *   *amax = max(*amax, max |y|)  (NaN, if any y is NaN, wins)
 *   mean[r], rstd[r] saved if the pointers are not NULL.
 * amax usually points into history row 0 of the owning slot.  hidden must be a
 * multiple of 8 and at most 8192; params_dtype must be FP8LN_DTYPE_BF16; rows may
 * be 0 (nothing is launched). */
int fp8ln_ln_cast_amax(const fp8ln_recipe* recipe, int64_t rows, int64_t hidden,
                       int32_t params_dtype, const void* x, const void* gamma,
                       const void* beta, int32_t fp8_dtype, const float* scale,
                       float* amax, uint8_t* out, uint8_t* out_t, float* mean,
                       float* rstd, void* stream);

/* Cast a [rows][cols] tensor (bf16 or fp32, in_dtype) to FP8:
 *   out[r][c] = encode(in[r][c] * (*scale)); out_t[c][r] = out[r][c] (optional);
 *   *amax = max(*amax, max |in|); colsum[c] = sum over rows of in[r][c] (optional,
 *   fp32, needs workspace of fp8ln_workspace_size(FP8LN_OP_CAST_AMAX, rows, cols)).
 * cols must be a multiple of 16. */
int fp8ln_cast_amax(int64_t rows, int64_t cols, int32_t in_dtype, const void* in,
                    int32_t fp8_dtype, const float* scale, float* amax, uint8_t* out,
                    uint8_t* out_t, float* colsum, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Encode `count` consecutive binary32 bit patterns start, start+1, ... (mod 2^32)
 * with the same device encoder the kernels use: out[i] = encode(float(start + i)).
 * Lets a caller check the encoder against every binary32 input. */
int fp8ln_encode_range(uint32_t start, int64_t count, int32_t fp8_dtype, uint8_t* out,
                       void* stream);

/* Streaming-bandwidth probe (measurement): out[i] = the high byte of the 16-bit
 * word in[i] for n elements, i.e. the memory traffic of fp8ln_ln_cast_amax (2
 * bytes read and 1 written per element, non-temporal accesses) without its
 * arithmetic; its rate on a device is the practical ceiling of that step there.
 * n: multiple of 8; in (2n bytes) and out (n bytes) 16-byte aligned. */
int fp8ln_stream_probe(int64_t n, const void* in, uint8_t* out, void* stream);

/* ---- FP8 GEMM ([G] "Playing with lower-precision formats"; [T] intro, FP8
 *      tensor cores) ------------------------------------------------------- */

/* out[m][n] = (sum_k A[m][k] * B[n][k]) * (*sinv_a) * (*sinv_b) + bias[n]
 * A: uint8 [M][K] codes in a_dtype; B: uint8 [N][K] codes in b_dtype (both keep
 * the contraction index last); bias: bf16 [N] or NULL; out_dtype FP8LN_DTYPE_BF16
 * or FP8LN_DTYPE_F32 (out is [M][N]).  K and N must be multiples of 16. */
int fp8ln_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
               const uint8_t* B, int32_t b_dtype, const float* sinv_a, const float* sinv_b,
               const void* bias, int32_t out_dtype, void* out, void* stream);

/* The fc1 step of LayerNormMLP ([G] "The building blocks": linear, GELU, linear)
 * as its own call:
 *   h = (sum_k A[m][k] B[n][k]) * (*sinv_a) * (*sinv_b) + bias[n]   (fp32)
 *   h_out[m][n] = bf16(h)                          (optional, may be NULL)
 *   g = gelu(h) (activation: fp8ln_activation); q_out[m][n] = encode(g * (*q_scale))
 *   q_out_t[n][m] = q_out[m][n]                    (optional, needs M % 16 == 0)
 *   *q_amax = max(*q_amax, max |g|)
 * bias is bf16 [N] or NULL.  K and N must be multiples of 16. */
int fp8ln_gemm_gelu_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
                        const uint8_t* B, int32_t b_dtype, const float* sinv_a,
                        const float* sinv_b, const void* bias, void* h_out, uint8_t* q_out,
                        uint8_t* q_out_t, int32_t q_dtype, const float* q_scale, float* q_amax,
                        int32_t activation, void* stream);

/* The fc2 dgrad step of the LayerNormMLP backward with the GELU derivative:
 *   out[m][n] = (sum_k A[m][k] B[n][k]) * (*sinv_a) * (*sinv_b) * gelu'(h[m][n])
 * (gelu of the given fp8ln_activation).
 * h is the bf16 [M][N] fc1 output saved by the forward; out is fp32 [M][N].
 * K and N must be multiples of 16. */
int fp8ln_gemm_dgelu(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
                     const uint8_t* B, int32_t b_dtype, const float* sinv_a, const float* sinv_b,
                     const void* h, float* out, int32_t activation, void* stream);

/* The same product with the gradient cast of the fc1 output fused in, which is
 * how the LayerNormMLP backward runs it (HYBRID: gradients in E5M2):
 *   d = (sum_k A[m][k] B[n][k]) * (*sinv_a) * (*sinv_b) * gelu'(h[m][n])   (fp32)
 *   q_out[m][n] = encode(d * (*q_scale)) in q_dtype, from the exact product
 *   q_out_t[n][m] = q_out[m][n]                    (optional, needs M % 16 == 0)
 *   *q_amax = max(*q_amax, max |d|)
 *   dbias[n] = sum_m d[m][n]                       (optional; fixed summation order)
 * The d values and codes equal those of fp8ln_gemm_dgelu followed by
 * fp8ln_cast_amax on its output.  dbias needs a workspace of
 * fp8ln_workspace_size(FP8LN_OP_GEMM_DGELU_FP8, M, N) bytes.  K and N must be
 * multiples of 16. */
int fp8ln_gemm_dgelu_fp8(int64_t M, int64_t N, int64_t K, const uint8_t* A, int32_t a_dtype,
                         const uint8_t* B, int32_t b_dtype, const float* sinv_a,
                         const float* sinv_b, const void* h, int32_t q_dtype,
                         const float* q_scale, float* q_amax, uint8_t* q_out, uint8_t* q_out_t,
                         float* dbias, int32_t activation, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ---- LayerNorm backward ---------------------------------------------------- */

/* With xhat = (x - mean) * rstd and g = dy * gamma per row:
 *   dx = rstd * (g - mean_j g - xhat * mean_j(g * xhat))        (bf16 [rows][hidden])
 *   dgamma = sum over rows of dy * xhat, dbeta = sum over rows of dy (fp32 [hidden])
 * dy is fp32 [rows][hidden]; x, gamma bf16; mean, rstd fp32 [rows] as saved by the
 * forward.  Workspace: fp8ln_workspace_size(FP8LN_OP_LAYERNORM_BWD, rows, hidden). */
int fp8ln_layernorm_bwd(int64_t rows, int64_t hidden, const float* dy, const void* x,
                        const float* mean, const float* rstd, const void* gamma, void* dx,
                        float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ---- BF16 path ([G] "Playing with lower-precision formats: BF16 vs FP8"; [T]
 *      benchmark listing and results: the same modules without FP8) ---------- */

/* The modules without FP8: every GEMM multiplies bf16 values on the bf16 matrix
 * cores with fp32 accumulation; there are no scales, amaxes or histories.
 *
 * out[m][n] = sum_k A[m][k] * B[n][k] + bias[n]
 * A bf16 [M][K], B bf16 [N][K] (contraction index last), bias bf16 [N] or NULL,
 * out [M][N] in out_dtype (bf16, or fp32 without bias).  N, K: multiples of 16. */
int fp8ln_gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                    const void* bias, int32_t out_dtype, void* out, void* stream);

/* h = A . B^T + bias (fp32); h_out = bf16(h) when h_out is not NULL;
 * out = bf16(gelu(h)) with gelu of the given activation form.  Shapes as above. */
int fp8ln_gemm_gelu_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                         const void* bias, void* h_out, void* out, int32_t activation,
                         void* stream);

/* out = bf16((A . B^T) * gelu'(h)) with h bf16 [M][N] and gelu' of the given
 * activation form (the fc2 dgrad of the BF16 LayerNormMLP).  Shapes as above. */
int fp8ln_gemm_dgelu_bf16(int64_t M, int64_t N, int64_t K, const void* A, const void* B,
                          const void* h, void* out, int32_t activation, void* stream);

/* out[c][r] = in[r][c] for bf16 [rows][cols] (rows, cols multiples of 8), and
 * colsum[c] = sum over r of in[r][c] in fp32 when colsum is not NULL (workspace:
 * fp8ln_workspace_size(FP8LN_OP_TRANSPOSE_BF16, rows, cols)). */
int fp8ln_transpose_bf16(int64_t rows, int64_t cols, const void* in, void* out, float* colsum,
                         void* workspace, size_t workspace_bytes, void* stream);

/* BF16 LayerNormLinear forward: ln_out = bf16(LN(x)) (as fp8ln_layernorm_fwd;
 * mean, rstd written when not NULL), out = ln_out . W^T + bias in bf16.
 * x bf16 [tokens][in], W bf16 [out][in], bias bf16 [out] or NULL, ln_out bf16
 * [tokens][in] (kept for the backward).  in: multiple of 16 up to 8192; out:
 * multiple of 16. */
int fp8ln_ln_linear_fwd_bf16(int64_t tokens, int64_t in_features, int64_t out_features,
                             float eps, const void* x, const void* gamma, const void* beta,
                             const void* weight, const void* bias, void* out, void* ln_out,
                             float* mean, float* rstd, void* stream);

/* Its backward for dy bf16 [tokens][out]:
 *   dLN = dy . W (fp32), dW = dy^T . ln_out (fp32 [out][in]), dbias = column sums
 *   of dy (fp32, or NULL), then the LayerNorm backward gives dx (bf16), dgamma and
 *   dbeta (fp32).
 * tokens: multiple of 16; in at most 4096.  Workspace:
 * fp8ln_workspace_size(FP8LN_OP_LN_LINEAR_BWD_BF16, tokens, in, out). */
int fp8ln_ln_linear_bwd_bf16(int64_t tokens, int64_t in_features, int64_t out_features,
                             const void* dy, const void* x, const void* gamma,
                             const void* weight, const void* ln_out, const float* mean,
                             const float* rstd, void* dx, float* dgamma, float* dbeta,
                             float* dweight, float* dbias, void* workspace,
                             size_t workspace_bytes, void* stream);

/* BF16 LayerNormMLP forward: ln_out = bf16(LN(x)); h = ln_out . W1^T + b1 (fp32,
 * stored as bf16 when h is not NULL); g = bf16(gelu(h)) [tokens][ffn];
 * out = g . W2^T + b2 in bf16.  W1 bf16 [ffn][hidden], W2 bf16 [hidden][ffn]. */
int fp8ln_ln_mlp_fwd_bf16(int64_t tokens, int64_t hidden, int64_t ffn, float eps,
                          int32_t activation, const void* x, const void* gamma, const void* beta,
                          const void* w1, const void* b1, const void* w2, const void* b2,
                          void* out, void* ln_out, void* h, void* g, float* mean, float* rstd,
                          void* stream);

/* Backward of fp8ln_ln_mlp_fwd_bf16 for dy bf16 [tokens][hidden], from the
 * forward's ln_out, h and g (all bf16) and mean, rstd:
 *   dW2 = dy^T . g, db2 = column sums of dy
 *   dH = (dy . W2) * gelu'(h) (bf16), dW1 = dH^T . ln_out, db1 = column sums of dH
 *   dLN = dH . W1 (fp32), then the LayerNorm backward gives dx, dgamma, dbeta.
 * dW1, dW2, db1, db2, dgamma, dbeta fp32; db1 / db2 may be NULL.  tokens: multiple
 * of 16; hidden at most 4096.  Workspace:
 * fp8ln_workspace_size(FP8LN_OP_LN_MLP_BWD_BF16, tokens, hidden, ffn). */
int fp8ln_ln_mlp_bwd_bf16(int64_t tokens, int64_t hidden, int64_t ffn, int32_t activation,
                          const void* dy, const void* x, const void* gamma, const void* w1,
                          const void* w2, const void* ln_out, const void* h, const void* g,
                          const float* mean, const float* rstd, void* dx, float* dgamma,
                          float* dbeta, float* dw1, float* db1, float* dw2, float* db2,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- LayerNorm ([T] setup listing, module tour: te.LayerNorm) --------------- */

/* The plain LayerNorm module (no FP8 output): per row of x bf16 [rows][hidden],
 *   mean = sum x / hidden, var = sum (x - mean)^2 / hidden (biased),
 *   rstd = 1 / sqrt(var + eps), y = (x - mean) * rstd * gamma + beta
 * computed in fp32 and rounded to bf16 (nearest-even) into y [rows][hidden].
 * mean and rstd (fp32 [rows]) are written when not NULL; the backward needs them.
 * hidden: multiple of 8, at most 8192.  x, y, gamma, beta: 16-byte aligned. */
int fp8ln_layernorm_fwd(int64_t rows, int64_t hidden, float eps, const void* x,
                        const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                        void* stream);

/* fp8ln_layernorm_bwd for a bf16 dy [rows][hidden] (the gradient that reaches a
 * plain LayerNorm module); same outputs, limits and workspace. */
int fp8ln_layernorm_bwd_bf16(int64_t rows, int64_t hidden, const void* dy, const void* x,
                             const float* mean, const float* rstd, const void* gamma, void* dx,
                             float* dgamma, float* dbeta, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---- Linear ([T] setup listing, module tour: te.Linear) --------------------- */

/* out = x W^T + bias with FP8 operands (a Linear layer without the LayerNorm), for
 * x bf16 [tokens][in_features], W bf16 [out_features][in_features], bias bf16
 * [out_features] or NULL, out bf16 [tokens][out_features]:
 *   x_q = encode(x * scale[0]), amax -> history[0][0]   (stored in ctx->ln_q,
 *         its transpose in ctx->ln_qt when set)
 *   w_q = encode(W * scale[1]), amax -> history[0][1]   (or reused, see
 *         fp8ln_linear_ctx.reuse_weight_codes)
 *   out = (x_q . w_q^T) * scale_inv[0] * w_scale_inv + bias
 * ctx->mean and ctx->rstd are not used.  in_features, out_features: multiples of
 * 16; when ctx->ln_qt is set tokens must be a multiple of 16. */
int fp8ln_linear_fwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                     int64_t out_features, int32_t params_dtype, const void* x,
                     const void* weight, const void* bias, void* out, const fp8ln_meta* fwd,
                     const fp8ln_linear_ctx* ctx, void* stream);

/* Backward of fp8ln_linear_fwd for dy bf16 [tokens][out_features]:
 *   dy_q = encode(dy * bwd.scale[0]) in the backward format, amax -> bwd history
 *   dx = (dy_q . w_q) * bwd.scale_inv[0] * w_scale_inv          (bf16 [tokens][in])
 *   dW = (dy_q^T . x_q) * bwd.scale_inv[0] * fwd.scale_inv[0]   (fp32 [out][in])
 *   dbias = column sums of dy (fp32 [out], or NULL)
 * ctx must hold ln_qt (the input codes' transpose) and w_qt.  tokens: multiple of 16.
 * Workspace: fp8ln_workspace_size(FP8LN_OP_LINEAR_BWD, tokens, in, out). */
int fp8ln_linear_bwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                     int64_t out_features, int32_t params_dtype, const void* dy,
                     const fp8ln_linear_ctx* ctx, const fp8ln_meta* fwd, const fp8ln_meta* bwd,
                     void* dx, float* dweight, float* dbias, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ---- LayerNormLinear ([T] setup listing: te.LayerNormLinear(H, 3*H)) ------- */

/* out = LN(x) W^T + bias with FP8 operands, for x bf16 [tokens][in_features],
 * W bf16 [out_features][in_features] (torch.nn.Linear layout), bias bf16
 * [out_features] or NULL, out bf16 [tokens][out_features]:
 *   ln_q = encode(LN(x) * scale[0]), amax -> history[0][0]
 *   w_q  = encode(W * scale[1]),     amax -> history[0][1]
 *   out  = (ln_q . w_q^T) * scale_inv[0] * scale_inv[1] + bias
 * fwd is the module's forward state (2 slots, kind FORWARD), already advanced by
 * fp8ln_scaling_update for this step.  ctx receives what the backward needs.
 * in_features: multiple of 16, at most 8192; out_features: multiple of 16; when
 * ctx->ln_qt is set tokens must be a multiple of 16. */
int fp8ln_ln_linear_fwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                        int64_t out_features, int32_t params_dtype, const void* x,
                        const void* gamma, const void* beta, const void* weight,
                        const void* bias, void* out, const fp8ln_meta* fwd,
                        const fp8ln_linear_ctx* ctx, void* stream);

/* Bytes of the step workspace of the *_step entry points. */
#define FP8LN_STEP_WS_BYTES 64

/* One forward step of LayerNormLinear: fp8ln_scaling_update(recipe, fwd) followed
 * by fp8ln_ln_linear_fwd with the same arguments, with identical results (history,
 * scale, scale_inv, ctx contents and out, bit for bit).  The delayed recipe knows
 * the step's scales before it sees the step's data ("Turbo-charging your
 * transformer training", "Playing with lower-precision formats"; tutorial
 * "Accelerating Transformer Training with NVIDIA Transformer Engine ...", FP8
 * recipe setup: amax history, max reduction), so the update needs no launch of
 * its own: where the forward's first launch (LayerNorm rows and weight cast side
 * by side) serves the shape, each of its workgroups forms its scale from the
 * history window itself and the GEMM's first workgroup then rolls the history
 * (the pages' "fused" operations: fewer launches, "Turbo-charging ...", "What
 * does 'fused' really mean?").  Otherwise the update runs as its own launch first.
 * step_ws: device buffer of FP8LN_STEP_WS_BYTES, 16-byte aligned, all zero
 * before the first call; every call leaves it zero.  Calls that share a step_ws
 * or a state block must not overlap (the same stream orders them). */
int fp8ln_ln_linear_fwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                             int64_t out_features, int32_t params_dtype, const void* x,
                             const void* gamma, const void* beta, const void* weight,
                             const void* bias, void* out, const fp8ln_meta* fwd,
                             const fp8ln_linear_ctx* ctx, void* step_ws, void* stream);

/* Backward of fp8ln_ln_linear_fwd for the output gradient dy bf16
 * [tokens][out_features]:
 *   dy_q = encode(dy * bwd.scale[0]) in the backward format, amax -> bwd history
 *   dLN = (dy_q . w_q) * bwd.scale_inv[0] * fwd.scale_inv[1]           (dgrad)
 *   dW  = (dy_q^T . ln_q) * bwd.scale_inv[0] * fwd.scale_inv[0]        (wgrad)
 *   dbias = column sums of dy; dx, dgamma, dbeta from the LayerNorm backward.
 * dx bf16 [tokens][in]; dgamma, dbeta fp32 [in]; dweight fp32 [out][in]; dbias
 * fp32 [out] or NULL.  ctx must hold ln_qt and w_qt.  tokens: multiple of 16.
 * Workspace: fp8ln_workspace_size(FP8LN_OP_LN_LINEAR_BWD, tokens, in, out). */
int fp8ln_ln_linear_bwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                        int64_t out_features, int32_t params_dtype, const void* dy,
                        const void* x, const void* gamma, const fp8ln_linear_ctx* ctx,
                        const fp8ln_meta* fwd, const fp8ln_meta* bwd, void* dx,
                        float* dgamma, float* dbeta, float* dweight, float* dbias,
                        void* workspace, size_t workspace_bytes, void* stream);

/* One backward step of LayerNormLinear: fp8ln_scaling_update(recipe, bwd)
 * followed by fp8ln_ln_linear_bwd with the same arguments, with identical results
 * (backward history, scale, scale_inv and every output, bit for bit).  As in the
 * forward step, the delayed recipe knows the step's gradient scale from earlier
 * steps' amaxes alone, so the update rides in the gradient cast: each of its
 * workgroups forms the scales from the history window, records the amax in
 * step_ws, and the backward's last launch (its column sums) rolls the history
 * ("Turbo-charging your transformer training", "What does 'fused' really
 * mean?": fewer launches).  With no tokens, or when bwd->n_slots is not 1, 2, 4
 * or 8, the update runs as its own launch first.  step_ws as for
 * fp8ln_ln_linear_fwd_step (a step's forward and backward may share one, in
 * stream order). */
int fp8ln_ln_linear_bwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                             int64_t out_features, int32_t params_dtype, const void* dy,
                             const void* x, const void* gamma, const fp8ln_linear_ctx* ctx,
                             const fp8ln_meta* fwd, const fp8ln_meta* bwd, void* dx,
                             float* dgamma, float* dbeta, float* dweight, float* dbias,
                             void* workspace, size_t workspace_bytes, void* step_ws,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): fp8ln_ln_linear_bwd
 * without the workspace argument.  The same kernels run with their workspace in
 * a 32 MiB (33554432-byte) device array that the library holds on each GPU it
 * runs on until the process ends; it calls no allocator.  Sizes whose workspace
 * (fp8ln_workspace_size(FP8LN_OP_LN_LINEAR_BWD, tokens, in, out)) exceeds 32 MiB
 * return FP8LN_ERR_UNSUPPORTED before anything is enqueued (2048 tokens at
 * 768 -> 2304 need about 19 MB).  All calls on one GPU share its array: calls
 * that overlap on a GPU (other streams, other threads) race and must be
 * ordered by the caller.  Arguments, outputs and errors are otherwise those of
 * fp8ln_ln_linear_bwd. */
int fp8ln_ln_linear_bwd_noalloc(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                                int64_t out_features, int32_t params_dtype, const void* dy,
                                const void* x, const void* gamma, const fp8ln_linear_ctx* ctx,
                                const fp8ln_meta* fwd, const fp8ln_meta* bwd, void* dx,
                                float* dgamma, float* dbeta, float* dweight, float* dbias,
                                void* stream);

/* ---- LayerNormMLP ([T] setup listing: te.LayerNormMLP(H, 4*H); [G] "The
 *      building blocks") ------------------------------------------------------ */

/* out = fc2(GELU(fc1(LN(x)))) with FP8 operands, GELU in its tanh form:
 *   ln_q = encode(LN(x) * scale[0])                         amax -> slot 0
 *   w1_q = encode(W1 * scale[1]), w2_q = encode(W2 * scale[3])  slots 1, 3
 *   h = (ln_q . w1_q^T) * scale_inv[0] * scale_inv[1] + b1   (saved as bf16)
 *   g = gelu(h) from the fp32 h; g_q = encode(g * scale[2])  amax -> slot 2
 *   out = (g_q . w2_q^T) * scale_inv[2] * scale_inv[3] + b2
 * x bf16 [tokens][hidden]; W1 bf16 [ffn][hidden]; b1 bf16 [ffn] or NULL;
 * W2 bf16 [hidden][ffn]; b2 bf16 [hidden] or NULL; out bf16 [tokens][hidden].
 * hidden: multiple of 16, at most 8192; ffn: multiple of 16; when transposes are
 * requested in ctx, tokens must be a multiple of 16. */
int fp8ln_ln_mlp_fwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden,
                     int64_t ffn, int32_t params_dtype, const void* x, const void* gamma,
                     const void* beta, const void* w1, const void* b1, const void* w2,
                     const void* b2, void* out, const fp8ln_meta* fwd,
                     const fp8ln_mlp_ctx* ctx, void* stream);

/* One forward step of LayerNormMLP: fp8ln_scaling_update(recipe, fwd) followed by
 * fp8ln_ln_mlp_fwd with the same arguments, with identical results, the update
 * folded into the forward's launches as in fp8ln_ln_linear_fwd_step (the GELU
 * output's amax is recorded with the others and the fc2 GEMM rolls the history).
 * step_ws as for fp8ln_ln_linear_fwd_step. */
int fp8ln_ln_mlp_fwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden,
                          int64_t ffn, int32_t params_dtype, const void* x, const void* gamma,
                          const void* beta, const void* w1, const void* b1, const void* w2,
                          const void* b2, void* out, const fp8ln_meta* fwd,
                          const fp8ln_mlp_ctx* ctx, void* step_ws, void* stream);

/* Backward of fp8ln_ln_mlp_fwd for dy bf16 [tokens][hidden]:
 *   dy_q = encode(dy * bwd.scale[0]); db2 = column sums of dy
 *   dH = (dy_q . w2_q) * bwd.scale_inv[0] * fwd.scale_inv[3] * gelu'(h)
 *   dh_q = encode(dH * bwd.scale[1]); db1 = column sums of dH
 *   dW2 = (dy_q^T . g_q) * bwd.scale_inv[0] * fwd.scale_inv[2]
 *   dLN = (dh_q . w1_q) * bwd.scale_inv[1] * fwd.scale_inv[1]
 *   dW1 = (dh_q^T . ln_q) * bwd.scale_inv[1] * fwd.scale_inv[0]
 *   dx, dgamma, dbeta from the LayerNorm backward.
 * dx bf16 [tokens][hidden]; dgamma, dbeta, db2 fp32 [hidden]; dw1 fp32
 * [ffn][hidden]; db1 fp32 [ffn]; dw2 fp32 [hidden][ffn]; db1, db2 may be NULL.
 * ctx must hold every transpose and h.  tokens: multiple of 16.
 * Workspace: fp8ln_workspace_size(FP8LN_OP_LN_MLP_BWD, tokens, hidden, ffn). */
int fp8ln_ln_mlp_bwd(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden,
                     int64_t ffn, int32_t params_dtype, const void* dy, const void* x,
                     const void* gamma, const fp8ln_mlp_ctx* ctx, const fp8ln_meta* fwd,
                     const fp8ln_meta* bwd, void* dx, float* dgamma, float* dbeta,
                     float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                     size_t workspace_bytes, void* stream);

/* One backward step of LayerNormMLP: fp8ln_scaling_update(recipe, bwd) followed
 * by fp8ln_ln_mlp_bwd with the same arguments, with identical results, the
 * update folded in as in fp8ln_ln_linear_bwd_step (the fc1 gradient's amax,
 * from the fc2 dgrad's fused cast, is recorded in step_ws with the output
 * gradient's).  step_ws as for fp8ln_ln_linear_fwd_step. */
int fp8ln_ln_mlp_bwd_step(const fp8ln_recipe* recipe, int64_t tokens, int64_t hidden,
                          int64_t ffn, int32_t params_dtype, const void* dy, const void* x,
                          const void* gamma, const fp8ln_mlp_ctx* ctx, const fp8ln_meta* fwd,
                          const fp8ln_meta* bwd, void* dx, float* dgamma, float* dbeta,
                          float* dw1, float* db1, float* dw2, float* db2, void* workspace,
                          size_t workspace_bytes, void* step_ws, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8LN_H */
