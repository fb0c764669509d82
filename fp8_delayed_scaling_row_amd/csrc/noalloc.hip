// The LayerNormLinear backward for callers that cannot allocate device memory:
// code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc.  It runs exactly the kernels of fp8ln_ln_linear_bwd; the only
// difference is where their workspace lives: in `scratch`, a file-scope device
// array of kScratchBytes that each GPU the library runs on holds until the
// process ends, instead of a buffer the caller brings.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is ever handed to the kernels.
//
// Every call on one GPU uses that GPU's one array, so calls that overlap on a
// GPU (on different streams, or from different threads without ordering) race
// on it.  The array keeps the last call's contents; nothing in this backward
// needs it zeroed: the gradient codes and their transpose, the fp32 dLN and the
// column-sum and dgamma / dbeta partials are each written in full before they
// are read.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/fp8ln.h"
#include "launchers.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxScratchDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];   // device address of `scratch`, per device

// The current device's address of `scratch` (looked up on its first use there).
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    char msg[256];
    if (e != hipSuccess) {
        std::snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
        return fp8ln::report_error(FP8LN_ERR_HIP, msg);
    }
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fp8ln::report_error(FP8LN_ERR_UNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s",
                          hipGetErrorString(e));
            return fp8ln::report_error(FP8LN_ERR_HIP, msg);
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FP8LN_OK;
}

}  // namespace

extern "C" {

int fp8ln_ln_linear_bwd_noalloc(const fp8ln_recipe* recipe, int64_t tokens, int64_t in_features,
                                int64_t out_features, int32_t params_dtype, const void* dy,
                                const void* x, const void* gamma, const fp8ln_linear_ctx* ctx,
                                const fp8ln_meta* fwd, const fp8ln_meta* bwd, void* dx,
                                float* dgamma, float* dbeta, float* dweight, float* dbias,
                                void* stream) {
    const size_t need = fp8ln_workspace_size(FP8LN_OP_LN_LINEAR_BWD, tokens, in_features,
                                             out_features);
    if (need > kScratchBytes) {
        char msg[256];
        std::snprintf(msg, sizeof(msg),
                      "ln_linear_bwd_noalloc: %lld tokens x %lld -> %lld needs %zu bytes of "
                      "scratch; the library holds %zu",
                      (long long)tokens, (long long)in_features, (long long)out_features, need,
                      kScratchBytes);
        return fp8ln::report_error(FP8LN_ERR_UNSUPPORTED, msg);
    }
    if (need == 0)   // invalid sizes: the full entry point names the problem
        return fp8ln_ln_linear_bwd(recipe, tokens, in_features, out_features, params_dtype, dy,
                                   x, gamma, ctx, fwd, bwd, dx, dgamma, dbeta, dweight, dbias,
                                   nullptr, 0, stream);
    void* ws = nullptr;
    const int s = scratch_address(&ws);
    if (s != FP8LN_OK) return s;
    return fp8ln_ln_linear_bwd(recipe, tokens, in_features, out_features, params_dtype, dy, x,
                               gamma, ctx, fwd, bwd, dx, dgamma, dbeta, dweight, dbias, ws,
                               kScratchBytes, stream);
}

}  // extern "C"
