// w12_probe.hip -- w12_read_probe: a plain streaming read of a device
// buffer, the reference a weight-streaming GEMM is measured against.  The
// pages tune kernels against the memory-bandwidth limit (AI Radar summary
// of SpecPilot, English edition, opening paragraph); the published HBM peak
// is not reachable by any kernel, so the benchmark also reports the rate of
// this kernel on a buffer of the weight's size.
//
// Each wave reads its own contiguous run of the buffer with eight 16-byte
// non-temporal loads in flight per lane (the pattern that measured fastest
// among grid-stride and per-wave runs with 4-16 loads in flight and 4-32
// waves per CU), folds the words with xor, and writes one word only if the
// fold equals a fixed value, so nothing but the read reaches memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w12.h"

namespace w12 {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kInFlight = 8;
constexpr int kWavesPerCu = 32;
constexpr int kCus = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ p,
                                                                   int64_t n16, int64_t per_wave,
                                                                   uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
    const int64_t beg = wave * per_wave;
    const int64_t end = beg + per_wave < n16 ? beg + per_wave : n16;
    uint32_t acc = 0;
    for (int64_t i = beg + lane; i < end; i += 64 * kInFlight) {
        u32x4_t v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            int64_t j = i + 64 * u;
            j = j < end ? j : end - 1;   // i < end, so end - 1 >= beg
            v[u] = __builtin_nontemporal_load(p + j);
        }
        // past the end the load repeats the last word: it must not count
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            if (i + 64 * u < end) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace
}  // namespace w12

extern "C" int w12_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (buf == nullptr || sink == nullptr) return W12_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || bytes % 16 != 0 ||
        (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return W12_ERR_ALIGN;
    if (bytes == 0) return W12_ERR_SHAPE;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t waves = (int64_t)w12::kCus * w12::kWavesPerCu;
    int64_t per_wave = (n16 + waves - 1) / waves;
    per_wave = (per_wave + 63) / 64 * 64;
    const int64_t waves_used = (n16 + per_wave - 1) / per_wave;   // at most `waves`
    const int64_t blocks = (waves_used * 64 + w12::kProbeThreads - 1) / w12::kProbeThreads;
    hipLaunchKernelGGL(w12::read_probe_kernel, dim3((unsigned)blocks), dim3(w12::kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const w12::u32x4_t*>(buf), n16,
                       per_wave, sink);
    return hipGetLastError() == hipSuccess ? W12_OK : W12_ERR_HIP;
}
