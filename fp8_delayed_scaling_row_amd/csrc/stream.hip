// Streaming-bandwidth probe: the memory traffic of the LayerNorm + FP8 cast step
// (2 bytes read, 1 byte written per element, non-temporal, 16-byte loads and
// 8-byte stores) with no arithmetic beyond picking a byte, so its rate is what
// HBM delivers to that access pattern on the running device.  The benchmark
// reports it beside the 8 TB/s of the spec sheet.
#include "device_common.hpp"
#include "launchers.hpp"

namespace fp8ln {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamRow = 2048;                 // elements per row: 4 KB in, 2 KB out
constexpr int kStreamCpl = kStreamRow / 8 / kWave;   // 16-byte chunks per lane and row

__device__ __forceinline__ uint2 high_bytes(const uint4& w) {
    return make_uint2(__builtin_amdgcn_perm(w.y, w.x, 0x07050301u),
                      __builtin_amdgcn_perm(w.w, w.z, 0x07050301u));
}

// out[i] = the high byte of the 16-bit word in[i].  The access pattern is the
// LayerNorm kernel's at hidden 2048: one wave per 4 KB row, lane l owning the
// row's 16-byte chunks l, l + 64, ..., the next row's loads issued before the
// current row is stored; the last partial row (n % 2048 elements) is done by
// whole 8-element groups.
__global__ __launch_bounds__(kStreamThreads) void stream_probe_kernel(
    const uint4* __restrict__ in, uint2* __restrict__ out, int64_t n16) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t waves = (int64_t)gridDim.x * (kStreamThreads / kWave);
    const int64_t rows = n16 / (kStreamRow / 8);
    int64_t row = (int64_t)blockIdx.x * (kStreamThreads / kWave) + threadIdx.x / kWave;
    uint4 cur[kStreamCpl];
    auto load = [&](int64_t r) {
        const uint4* src = in + (r < rows ? r : rows - 1) * (kStreamRow / 8);
#pragma unroll
        for (int i = 0; i < kStreamCpl; ++i) cur[i] = load_nt(src + lane + i * kWave);
    };
    if (rows > 0) load(row);
    for (; row < rows; row += waves) {
        uint4 w[kStreamCpl];
#pragma unroll
        for (int i = 0; i < kStreamCpl; ++i) w[i] = cur[i];
        __builtin_amdgcn_sched_barrier(0);
        load(row + waves);
        uint2* dst = out + row * (kStreamRow / 8);
#pragma unroll
        for (int i = 0; i < kStreamCpl; ++i) store_nt(dst + lane + i * kWave, high_bytes(w[i]));
    }
    const int64_t t = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    for (int64_t i = rows * (kStreamRow / 8) + t; i < n16;
         i += (int64_t)gridDim.x * kStreamThreads)
        store_nt(out + i, high_bytes(load_nt(in + i)));
}

}  // namespace

hipError_t launch_stream_probe(int64_t n, const void* in, uint8_t* out, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    static int resident = 0;
    if (resident == 0) {
        int nb = 0, dev = 0, cus = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, stream_probe_kernel,
                                                                    kStreamThreads, 0);
        if (e != hipSuccess) return e;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
            hipSuccess)
            return e;
        resident = (nb > 0 ? nb : 1) * cus;
    }
    const int64_t n16 = n / 8;
    const int64_t want = (n16 + kStreamThreads - 1) / kStreamThreads;
    const int blocks = (int)(want < resident ? want : resident);
    hipLaunchKernelGGL(stream_probe_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream,
                       (const uint4*)in, (uint2*)out, n16);
    return hipGetLastError();
}

}  // namespace fp8ln
