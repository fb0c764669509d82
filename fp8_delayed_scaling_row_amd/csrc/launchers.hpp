// Host-side launchers of the gfx950 kernels.  Each enqueues its kernels on
// `stream` and returns the launch status; arguments are validated by the C-ABI
// layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8ln {

// Records `message` as the calling thread's last error (fp8ln_last_error) and
// returns `status` (api.cpp).
int report_error(int status, const char* message);

// FP8 encodings (same values as fp8ln_fp8_dtype).
enum Fp8Kind : int { kE4M3 = 0, kE5M2 = 1 };

// scaling.hip
hipError_t launch_meta_init(float* hist, float* scale, float* scale_inv, int len, int n_slots,
                            hipStream_t stream);
// Up to kMaxUpdateBatch state blocks updated in one launch (same recipe).
constexpr int kMaxUpdateBatch = 64;
struct UpdateJob {
    float* hist;
    float* scale;
    float* scale_inv;
    int n_slots;
    float fp8_max;
};
struct UpdateBatch {
    UpdateJob job[kMaxUpdateBatch];
    int len, margin;
};
hipError_t launch_scaling_update_batch(const UpdateBatch& b, int n, hipStream_t stream);
hipError_t launch_scaling_update(float* hist, float* scale, float* scale_inv, int len,
                                 int n_slots, int margin, float fp8_max, hipStream_t stream);

// layernorm.hip.  fp8 = kLnOutBf16 selects the plain LayerNorm (bf16 output,
// scale and amax unused).
constexpr int kLnOutBf16 = 2;
hipError_t launch_ln_cast_amax(int64_t rows, int hidden, const void* x, const void* gamma,
                               const void* beta, float eps, int fp8, const float* scale,
                               float* amax, void* out, float* mean, float* rstd,
                               hipStream_t stream);
size_t ln_bwd_workspace(int64_t rows, int hidden);
struct SumBatch;
hipError_t launch_ln_bwd(int64_t rows, int hidden, const void* dy, bool dy_bf16, const void* x,
                         const float* mean, const float* rstd, const void* gamma, void* dx,
                         float* dgamma, float* dbeta, void* workspace, hipStream_t stream,
                         SumBatch* sums = nullptr);

// prologue.hip: the LayerNorm + cast + amax of the rows and up to two weight
// casts (bf16 [rows][cols] -> codes, optional transposed copy, amax, scale_inv
// copy as in launch_cast_amax) in one launch.  Launches only when every workgroup
// fits on the GPU at once and hidden <= 2048; *launched says whether it did (the
// caller otherwise launches the kernels one by one).
constexpr int kMaxPrologueCasts = 2;
struct CastJob {
    const void* in;
    int64_t rows, cols;
    const float* scale;
    float* amax;
    uint8_t* out;
    uint8_t* out_t;
    const float* copy_src;
    float* copy_dst;
};
// The step-start scaling update folded into the prologue (upd non-null): every
// workgroup forms its own slot's scale from the history window (the update's
// arithmetic) and records its amax into ws instead of the history; workgroup 0
// writes every slot's scale and scale_inv, and the first workgroup of the
// forward's last GEMM rolls the history with row 0 = the recorded amaxes (0 for
// slots the step does not cast) and clears ws.
// ws: kStepWsWords words, zero on entry, zero again when the step ends.
constexpr int kStepWsWords = 16;
constexpr int kMaxMetaSlots = 8;
struct FusedUpdate {
    float* hist;        // [len][n_slots]
    float* scale;       // [n_slots]
    float* scale_inv;   // [n_slots]
    int len, n_slots, margin;
    float fp8_max;
    uint32_t* ws;       // [0, n_slots): amax bits per slot
    int ln_slot;
    int cast_slot[kMaxPrologueCasts];
};
hipError_t launch_fwd_prologue(int64_t rows, int hidden, const void* x, const void* gamma,
                               const void* beta, float eps, int fp8, const float* scale,
                               float* amax, uint8_t* out, float* mean, float* rstd,
                               const CastJob* casts, int n_casts, bool* launched,
                               hipStream_t stream, const FusedUpdate* upd = nullptr);

// cast.hip
size_t cast_workspace(int64_t rows, int64_t cols);
// copy_src / copy_dst: when given, *copy_dst = *copy_src is done by the cast
// kernel (the scale_inv that goes with the codes it writes).
// sums: when given, the column sums are added to it instead of launched.
hipError_t launch_cast_amax(int64_t rows, int64_t cols, bool in_f32, const void* in, int fp8,
                            const float* scale, float* amax, uint8_t* out, uint8_t* out_t,
                            float* colsum, void* workspace, hipStream_t stream,
                            const float* copy_src = nullptr, float* copy_dst = nullptr,
                            SumBatch* sums = nullptr);
// The same cast of bf16 [rows][cols] (rows > 0) with the step's scaling update
// folded in: every workgroup forms the scales from the history window (the cast
// uses slot u.cast_slot[0]'s) and records the amax into u.ws; workgroup 0 writes
// every slot's scale and scale_inv; a later launch rolls the history.
hipError_t launch_cast_amax_step(int64_t rows, int64_t cols, const void* in, int fp8,
                                 const FusedUpdate& u, uint8_t* out, uint8_t* out_t,
                                 float* colsum, void* workspace, SumBatch* sums,
                                 hipStream_t stream);
// out[j] = sum over r < nrows of partial[r][j] in a fixed order; columns j < split
// go to out0[j], the others to out1[j - split].
struct SumJob {
    const float* partial;
    int64_t nrows, width;
    float* out0;
    float* out1;
    int64_t split;
};
hipError_t launch_sum_partials(const float* partial, int64_t nrows, int64_t width, float* out0,
                               float* out1, int64_t split, hipStream_t stream);
// Column sums gathered from several kernels (launchers given a SumBatch add their
// job instead of launching it) and run as one launch, each with the order of its
// own launch; roll_hist (optional): the folded scaling update's history roll
// (roll_history), done by the launch's first workgroup.
constexpr int kMaxSumJobs = 4;
struct SumBatch {
    SumJob job[kMaxSumJobs];
    int n = 0;
    float* roll_hist = nullptr;
    uint32_t* roll_ws = nullptr;
    int roll_len = 0, roll_slots = 0;
    bool add(const float* partial, int64_t nrows, int64_t width, float* out0, float* out1,
             int64_t split);   // false when full
};
hipError_t launch_sum_batch(const SumBatch& b, hipStream_t stream);
// in [rows][cols] -> out [cols][rows] bytes (rows, cols % 16 == 0).
hipError_t launch_transpose_u8(int64_t rows, int64_t cols, const uint8_t* in, uint8_t* out,
                               hipStream_t stream);
hipError_t launch_encode_range(uint32_t start, int64_t count, int fp8, uint8_t* out,
                               hipStream_t stream);
// bf16 [rows][cols] -> [cols][rows] (rows, cols % 8 == 0); colsum (optional) gets
// the fp32 column sums and needs transpose_b16_workspace bytes of workspace.
size_t transpose_b16_workspace(int64_t rows, int64_t cols);
hipError_t launch_transpose_b16(int64_t rows, int64_t cols, const void* in, void* out,
                                float* colsum, void* workspace, hipStream_t stream);

// stream.hip: out[i] = high byte of the 16-bit in[i] for n elements (n % 8 == 0),
// non-temporal; the LayerNorm + cast step's traffic without its arithmetic.
hipError_t launch_stream_probe(int64_t n, const void* in, uint8_t* out, hipStream_t stream);

// gemm.hip
enum GemmEpilogue : int {
    kEpiBf16Bias = 0,   // out bf16 = acc * alpha + bias
    kEpiF32 = 1,        // out fp32 = acc * alpha
    kEpiGeluFp8 = 2,    // h = acc * alpha + bias -> h bf16; g = gelu(h) -> FP8 (+T), amax
    kEpiDGeluF32 = 3,   // out fp32 = acc * alpha * gelu'(h)
    kEpiDGeluFp8 = 4,   // d = acc * alpha * gelu'(h) -> FP8 (+T), amax, column partial sums
    kEpiGeluBf16 = 5,   // h = acc * alpha + bias -> h bf16 (optional); out bf16 = gelu(h)
    kEpiDGeluBf16 = 6,  // out bf16 = acc * alpha * gelu'(h)
};

// GEMM operand kind besides the FP8 formats: bf16 values.  Both operands of a
// product are then bf16 (K counts elements, not bytes), and the epilogues are
// kEpiBf16Bias, kEpiF32, kEpiGeluBf16, kEpiDGeluF32 and kEpiDGeluBf16.
constexpr int kOpBf16 = 2;

struct GemmParams {
    int64_t M, N, K;
    const uint8_t* A;       // [M][K] codes (or bf16 values)
    const uint8_t* B;       // [N][K]
    int a_fp8, b_fp8;       // kE4M3, kE5M2, or kOpBf16 for both
    const float* sinv_a;    // device scalars; alpha = *sinv_a * *sinv_b
    const float* sinv_b;
    const uint16_t* bias;   // bf16 [N] or null
    void* out;              // [M][N], bf16 or fp32
    // kEpiGeluFp8
    uint16_t* h_out;        // bf16 [M][N] or null
    uint8_t* q_out;         // [M][N]
    uint8_t* q_out_t;       // [N][M] or null
    const float* q_scale;   // scale of the FP8 output
    float* q_amax;          // amax of gelu(h)
    int q_fp8;
    // kEpiDGeluF32, kEpiDGeluBf16, kEpiDGeluFp8 (which also uses q_out, q_out_t, q_scale,
    // q_amax, q_fp8)
    const uint16_t* h_in;   // bf16 [M][N]
    float* col_partial;     // kEpiDGeluFp8: [ceil(M / tile rows)][N] column sums, or null
    int gelu_erf;           // GELU epilogues: 0 = tanh form, 1 = erf form
    int epilogue;
    // The step's history roll when the scaling update was folded into the
    // forward (see FusedUpdate): workgroup 0 moves every row of roll_hist
    // [roll_len][roll_slots] down by one, sets row 0 to the amax bits recorded in
    // roll_ws and clears them.  Null roll_hist: no roll.
    float* roll_hist;
    uint32_t* roll_ws;
    int roll_len, roll_slots;
};

// Rows of the col_partial array launch_gemm writes for an M-row product (its
// tile height), and an upper bound for workspace sizing.
int64_t gemm_partial_rows(int64_t M, int64_t N, int64_t K);
inline int64_t gemm_partial_rows_bound(int64_t M) { return (M + 127) / 128; }

hipError_t launch_gemm(const GemmParams& p, hipStream_t stream);
// n (<= kMaxGemmGroup) independent products in one launch when all of them are
// small fp32-output FP8 products of the same operand formats (their tiles then
// share the GPU); otherwise one launch_gemm after the other.  Results are those
// of launch_gemm either way.
constexpr int kMaxGemmGroup = 3;
hipError_t launch_gemm_group(const GemmParams* ps, int n, hipStream_t stream);

}  // namespace fp8ln
