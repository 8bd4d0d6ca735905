// w12_exc.hip -- the exception list: the escape path that keeps a W12
// container lossless when a group holds an element below its window.
//
// The pages call the format lossless (AI Radar summary of SpecPilot, English
// edition, "Reasons"; HotRepo digest of StargazerX0/SpecPilot, project
// introduction).  Each allocation stores 16 exponents per group (W12-v1:
// {0, 1} and 14 above an even base; W12-b: {0} and 15 above any base); an
// element outside them is written to the planes as the window floor (the
// group is flagged) and, here, also as one exception entry (format in
// w12.h): grouped by (tile, group) block in block order, inside a block in
// the order the tiled layout stores the weights (piece, dword, element).
// Three launches build the list: a count per block, one scan over the
// blocks (whose exclusive sums are the block offsets), and a write pass in
// which each wave places its block's entries at the scanned offset, lanes in
// piece order.
#include <hip/hip_runtime.h>

#include "w12_internal.hpp"

namespace w12 {
namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// The lane's 32 weights of block blk (lane L = 16 q + c: row 16 T + c,
// k = 128 g + 32 b + 8 q + e, bit 8 b + e of the mask) and the bits of those
// below the group's window.  Every lane of the wave must call this (the
// group maximum is shared through shuffles).
struct LaneWeights {
    uint32_t v[16];
    uint32_t mask;
    uint32_t beta;
    int64_t n;
    int64_t kbase;  // k of bit 0: 128 g + 8 q
};

template <int FMT>
__device__ __forceinline__ LaneWeights lane_weights(const uint16_t* __restrict__ w, int64_t N,
                                                    int64_t K, int64_t blk, int lane) {
    LaneWeights r;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int64_t G = K / 128;
    r.n = (blk / G) * 16 + c;
    const int64_t g = blk % G;
    r.kbase = 128 * g + 8 * q;
    const bool valid = r.n < N;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint4 d = make_uint4(0, 0, 0, 0);
        if (valid) d = *reinterpret_cast<const uint4*>(w + r.n * K + 128 * g + 32 * b + 8 * q);
        r.v[4 * b + 0] = d.x;
        r.v[4 * b + 1] = d.y;
        r.v[4 * b + 2] = d.z;
        r.v[4 * b + 3] = d.w;
    }
    uint32_t emax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        emax = max_u32(emax, (r.v[i] >> 7) & 0xFFu);
        emax = max_u32(emax, (r.v[i] >> 23) & 0xFFu);
    }
    emax = max_u32(emax, (uint32_t)__shfl_xor((int)emax, 16));
    emax = max_u32(emax, (uint32_t)__shfl_xor((int)emax, 32));
    // the group base and the lowest stored normal exponent: W12-v1
    // [2 beta + 2, 2 beta + 15] (E <= 1 always stored), W12-b [b + 1, b + 15]
    // (E = 0 always stored)
    const uint32_t beta = FMT == kFmtB ? (emax <= 15u ? 0u : emax - 15u)
                                       : (emax <= 15u ? 0u : (emax - 14u) >> 1);
    const uint32_t floor_e = FMT == kFmtB ? beta + 1u : 2u * beta + 2u;
    const uint32_t low_e = FMT == kFmtB ? 1u : 2u;
    r.beta = beta;
    r.mask = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t word = (r.v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const uint32_t ex = (word >> 7) & 0xFFu;
        if (ex >= low_e && ex < floor_e) r.mask |= 1u << i;
    }
    return r;
}

__device__ __forceinline__ uint32_t word_of(const LaneWeights& r, int i) {
    return (r.v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
}

// Sum over the 64 lanes of a wave (fixed xor tree).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v += (uint32_t)__shfl_xor((int)v, d);
    return v;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void exc_count_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                             int64_t K, int64_t nblocks,
                                                             uint32_t* __restrict__ cnt) {
    const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (blk >= nblocks) return;  // whole waves only
    const int lane = threadIdx.x & 63;
    const LaneWeights r = lane_weights<FMT>(w, N, K, blk, lane);
    const uint32_t total = wave_sum((uint32_t)__popc(r.mask));
    if (lane == 0) cnt[blk] = total;
}

// One workgroup: exclusive scan of the block counts in place, in chunks of
// kScanThreads with a running carry; then the block offsets and the total.
__global__ __launch_bounds__(kScanThreads) void exc_scan_kernel(uint32_t* __restrict__ cnt,
                                                                int64_t nblocks,
                                                                uint32_t* __restrict__ offsets,
                                                                uint32_t* __restrict__ total) {
    __shared__ uint32_t buf[kScanThreads];
    __shared__ uint32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < nblocks; base += kScanThreads) {
        const int64_t i = base + threadIdx.x;
        const uint32_t v = i < nblocks ? cnt[i] : 0u;
        buf[threadIdx.x] = v;
        __syncthreads();
        // Hillis-Steele inclusive scan over the chunk.
        for (int d = 1; d < kScanThreads; d <<= 1) {
            const uint32_t add = threadIdx.x >= (unsigned)d ? buf[threadIdx.x - d] : 0u;
            __syncthreads();
            buf[threadIdx.x] += add;
            __syncthreads();
        }
        const uint32_t c0 = carry;
        if (i < nblocks) cnt[i] = c0 + buf[threadIdx.x] - v;  // exclusive
        __syncthreads();
        if (threadIdx.x == kScanThreads - 1) carry = c0 + buf[threadIdx.x];
        __syncthreads();
    }
    for (int64_t t = threadIdx.x; t < nblocks; t += kScanThreads) offsets[t] = cnt[t];
    if (threadIdx.x == 0) {
        offsets[nblocks] = carry;
        *total = carry;
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void exc_write_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                             int64_t K, int64_t nblocks,
                                                             const uint32_t* __restrict__ off,
                                                             uint32_t* __restrict__ entries,
                                                             int64_t capacity) {
    const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const int lane = threadIdx.x & 63;
    const LaneWeights r = lane_weights<FMT>(w, N, K, blk, lane);
    // Exclusive prefix of the lane counts in lane (= piece) order.
    const uint32_t mine = (uint32_t)__popc(r.mask);
    uint32_t incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t up = (uint32_t)__shfl_up((int)incl, d);
        if (lane >= d) incl += up;
    }
    int64_t idx = (int64_t)off[blk] + (incl - mine);
    const uint32_t c = (uint32_t)(lane & 15);
    // ascending bit = ascending (b, e); a static index keeps v[] in registers
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if (r.mask & (1u << i)) {
            if (idx < capacity) {
                const int64_t k = r.kbase + 32 * (i >> 3) + (i & 7);
                entries[2 * idx] = (c << 24) | (uint32_t)k;
                entries[2 * idx + 1] = (r.beta << 16) | word_of(r, i);
            }
            ++idx;
        }
    }
}

__global__ __launch_bounds__(kThreads) void exc_apply_kernel(const uint32_t* __restrict__ offsets,
                                                             const uint32_t* __restrict__ entries,
                                                             int64_t N, int64_t K,
                                                             uint16_t* __restrict__ w) {
    // tile t: blocks t * G .. t * G + G - 1, entries of consecutive blocks
    // are consecutive
    const int64_t t = blockIdx.x;
    const int64_t G = K / 128;
    const uint32_t beg = offsets[t * G], end = offsets[(t + 1) * G];
    for (uint32_t i = beg + threadIdx.x; i < end; i += kThreads) {
        const uint32_t pos = entries[2 * (int64_t)i];
        const int64_t n = 16 * t + (pos >> 24);
        const int64_t k = pos & 0xFFFFFFu;
        if (n < N && k < K) w[n * K + k] = (uint16_t)(entries[2 * (int64_t)i + 1] & 0xFFFFu);
    }
}

template <int FMT>
hipError_t exceptions_fmt(const uint16_t* w, int64_t N, int64_t K, uint32_t* ws, uint32_t* offsets,
                          uint32_t* entries, int64_t capacity, uint32_t* total, hipStream_t s) {
    const int64_t nb = (N + 15) / 16 * (K / 128);
    const int64_t grid = (nb + 3) / 4;
    hipLaunchKernelGGL(exc_count_kernel<FMT>, dim3((unsigned)grid), dim3(kThreads), 0, s, w, N, K,
                       nb, ws);
    hipLaunchKernelGGL(exc_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, ws, nb, offsets, total);
    if (entries != nullptr && capacity > 0)
        hipLaunchKernelGGL(exc_write_kernel<FMT>, dim3((unsigned)grid), dim3(kThreads), 0, s, w, N,
                           K, nb, ws, entries, capacity);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_exceptions(int fmt, const uint16_t* w, int64_t N, int64_t K, uint32_t* ws,
                             uint32_t* offsets, uint32_t* entries, int64_t capacity,
                             uint32_t* total, hipStream_t s) {
    return fmt == kFmtB ? exceptions_fmt<kFmtB>(w, N, K, ws, offsets, entries, capacity, total, s)
                        : exceptions_fmt<kFmtV1>(w, N, K, ws, offsets, entries, capacity, total, s);
}

hipError_t launch_apply_exceptions(const uint32_t* offsets, const uint32_t* entries, int64_t N,
                                   int64_t K, uint16_t* w, hipStream_t s) {
    const int64_t ntiles = (N + 15) / 16;
    hipLaunchKernelGGL(exc_apply_kernel, dim3((unsigned)ntiles), dim3(kThreads), 0, s, offsets,
                       entries, N, K, w);
    return hipGetLastError();
}

}  // namespace w12
