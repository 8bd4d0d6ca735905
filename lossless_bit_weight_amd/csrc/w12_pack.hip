// w12_pack.hip -- W12 encoders (pack), streaming decoders (unpack) for both
// bit allocations (W12-v1 and the arbitrary-base W12-b), and the BF16
// control layout (bf16_tile).
//
// Format: see w12.h.  The pages say only that BF16 is split into three 4-bit
// planes and that the format is lossless (AI Radar summary of SpecPilot,
// English edition, "Reasons"); the group/base rule and the tiled layout are
// this library's W12-v1.
//
// Work split: one wave per (16-row tile T, 128-weight group g).  Lane
// L = 16 q + c owns row n = 16 T + c and the 32 weights
// k = 128 g + 32 b + 8 q + e (b, e = 0..3, 0..7) -- exactly the 16-byte
// piece L of the block in each plane, so every plane store of a wave is one
// contiguous 1 KB.  The four lanes of a row (q = 0..3) form the group and
// agree on its base through two xor shuffles.  Rows >= N (padding of the
// last tile) are encoded as zeros.
#include "w12_decode.hpp"
#include "w12_internal.hpp"

namespace w12 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int FMT>
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                        int64_t K, int64_t nblocks,
                                                        uint4* __restrict__ p0,
                                                        uint4* __restrict__ p1,
                                                        uint4* __restrict__ p2,
                                                        uint8_t* __restrict__ meta,
                                                        uint32_t* __restrict__ bad_count) {
    const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (blk >= nblocks) return;  // whole waves only
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int64_t G = K / 128;
    const int64_t n = (blk / G) * 16 + c;
    const int64_t g = blk % G;
    const bool valid = n < N;

    uint32_t v[16];  // block b: v[4b .. 4b+3] = 8 BF16 words, natural order
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint4 d = make_uint4(0, 0, 0, 0);
        if (valid) d = *reinterpret_cast<const uint4*>(w + n * K + 128 * g + 32 * b + 8 * q);
        v[4 * b + 0] = d.x;
        v[4 * b + 1] = d.y;
        v[4 * b + 2] = d.z;
        v[4 * b + 3] = d.w;
    }

    // Largest biased exponent of the group (its 4 lanes).
    uint32_t emax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        emax = max_u32(emax, (v[i] >> 7) & 0xFFu);
        emax = max_u32(emax, (v[i] >> 23) & 0xFFu);
    }
    emax = max_u32(emax, (uint32_t)__shfl_xor((int)emax, 16));
    emax = max_u32(emax, (uint32_t)__shfl_xor((int)emax, 32));
    // W12-v1: even base 2 beta, window [2 beta + 2, 2 beta + 15] plus E <= 1.
    // W12-b: base b, window [b + 1, b + 15] plus E = 0.
    const uint32_t beta = FMT == kFmtB ? (emax <= 15u ? 0u : emax - 15u)
                                       : (emax <= 15u ? 0u : (emax - 14u) >> 1);
    const uint32_t floor_e = FMT == kFmtB ? beta + 1u : 2u * beta + 2u;

    // Per weight: lo = the byte that becomes planes P1:P0, code = the P2
    // nibble.  W12-v1: the BF16 low byte and sign<<3 | h.  W12-b: sign<<7 |
    // mantissa and the exponent offset c.
    uint32_t lo[32], code[32];
    uint32_t bad = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t word = (v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const uint32_t ex = (word >> 7) & 0xFFu;
        const uint32_t s = word >> 15;
        if constexpr (FMT == kFmtB) {
            uint32_t m = word & 0x7Fu;
            uint32_t c;
            if (ex == 0u) {
                c = 0u;
            } else if (ex >= floor_e) {
                c = ex - beta;
            } else {  // below the window: store the window floor, flag the group
                c = 1u;
                m = 0u;
                bad = 1u;
            }
            lo[i] = (s << 7) | m;
            code[i] = c;
        } else {
            uint32_t l = word & 0xFFu;
            uint32_t h;
            if (ex <= 1u) {
                h = 0u;
            } else if (ex >= floor_e) {
                h = (ex >> 1) - beta;
            } else {  // below the window: store the window floor, flag the group
                h = 1u;
                l = 0u;
                bad = 1u;
            }
            lo[i] = l;
            code[i] = (s << 3) | h;
        }
    }

    // Split-nibble order: dword b holds weights 8b..8b+7 of the lane; byte j
    // carries weight j (low nibble) and j+4 (high nibble).
    uint32_t o0[4], o1[4], o2[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t a0 = 0, a1 = 0, a2 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e0 = 8 * b + j, e1 = 8 * b + j + 4;
            a0 |= ((lo[e0] & 0xFu) | ((lo[e1] & 0xFu) << 4)) << (8 * j);
            a1 |= ((lo[e0] >> 4) | ((lo[e1] >> 4) << 4)) << (8 * j);
            a2 |= (code[e0] | (code[e1] << 4)) << (8 * j);
        }
        o0[b] = a0;
        o1[b] = a1;
        o2[b] = a2;
    }
    bad |= (uint32_t)__shfl_xor((int)bad, 16);
    bad |= (uint32_t)__shfl_xor((int)bad, 32);

    p0[blk * 64 + lane] = make_uint4(o0[0], o0[1], o0[2], o0[3]);
    p1[blk * 64 + lane] = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    p2[blk * 64 + lane] = make_uint4(o2[0], o2[1], o2[2], o2[3]);
    // W12-b's base needs all 8 bits: its groups are flagged through the count
    if (q == 0) meta[blk * 16 + c] = (uint8_t)(FMT == kFmtB ? beta : (beta | (bad << 7)));

    // One atomic per wave: the flagged groups of this block.
    const uint64_t flagged = __ballot(q == 0 && valid && bad);
    if (bad_count != nullptr && lane == 0 && flagged != 0)
        atomicAdd(bad_count, (uint32_t)__popcll(flagged));
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint4* __restrict__ p0,
                                                          const uint4* __restrict__ p1,
                                                          const uint4* __restrict__ p2,
                                                          const uint8_t* __restrict__ meta,
                                                          int64_t N, int64_t K, int64_t nblocks,
                                                          uint16_t* __restrict__ w) {
    const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int64_t G = K / 128;
    const int64_t n = (blk / G) * 16 + c;
    const int64_t g = blk % G;
    const uint4 a = p0[blk * 64 + lane], b4 = p1[blk * 64 + lane], c4 = p2[blk * 64 + lane];
    const uint32_t mb = meta[blk * 16 + c];
    const Lut t = make_lut(mb & 0x7Fu);
    const uint32_t base4 = mb * 0x01010101u;
    if (n >= N) return;
    const uint32_t pa[4] = {a.x, a.y, a.z, a.w};
    const uint32_t pb[4] = {b4.x, b4.y, b4.z, b4.w};
    const uint32_t pc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t o[4];
        if constexpr (FMT == kFmtB)
            decode8b(pa[b], pb[b], pc[b], base4, o);
        else
            decode8(pa[b], pb[b], pc[b], t, o);
        *reinterpret_cast<uint4*>(w + n * K + 128 * g + 32 * b + 8 * q) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Row-major BF16 [N, K] -> control layout: block (T, g) of 2048 words, 1 KB
// sub-block b, lane L's 8 words k = 128 g + 32 b + 8 q + e.
__global__ __launch_bounds__(kThreads) void bf16_tile_kernel(const uint16_t* __restrict__ w,
                                                             int64_t N, int64_t K, int64_t nblocks,
                                                             uint4* __restrict__ out) {
    const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (blk >= nblocks) return;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int64_t G = K / 128;
    const int64_t n = (blk / G) * 16 + c;
    const int64_t g = blk % G;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint4 d = make_uint4(0, 0, 0, 0);
        if (n < N) d = *reinterpret_cast<const uint4*>(w + n * K + 128 * g + 32 * b + 8 * q);
        out[(blk * 4 + b) * 64 + lane] = d;
    }
}

int64_t blocks_of(int64_t N, int64_t K) { return (N + 15) / 16 * (K / 128); }

}  // namespace

hipError_t launch_pack(int fmt, const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1,
                       void* p2, uint8_t* meta, uint32_t* bad, hipStream_t s) {
    const int64_t nb = blocks_of(N, K);
    const int64_t grid = (nb + 3) / 4;
    if (fmt == kFmtB)
        hipLaunchKernelGGL(pack_kernel<kFmtB>, dim3((unsigned)grid), dim3(kThreads), 0, s, w, N, K,
                           nb, reinterpret_cast<uint4*>(p0), reinterpret_cast<uint4*>(p1),
                           reinterpret_cast<uint4*>(p2), meta, bad);
    else
        hipLaunchKernelGGL(pack_kernel<kFmtV1>, dim3((unsigned)grid), dim3(kThreads), 0, s, w, N, K,
                           nb, reinterpret_cast<uint4*>(p0), reinterpret_cast<uint4*>(p1),
                           reinterpret_cast<uint4*>(p2), meta, bad);
    return hipGetLastError();
}

hipError_t launch_unpack(int fmt, const void* p0, const void* p1, const void* p2,
                         const uint8_t* meta, int64_t N, int64_t K, uint16_t* w, hipStream_t s) {
    const int64_t nb = blocks_of(N, K);
    const int64_t grid = (nb + 3) / 4;
    if (fmt == kFmtB)
        hipLaunchKernelGGL(unpack_kernel<kFmtB>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                           reinterpret_cast<const uint4*>(p0), reinterpret_cast<const uint4*>(p1),
                           reinterpret_cast<const uint4*>(p2), meta, N, K, nb, w);
    else
        hipLaunchKernelGGL(unpack_kernel<kFmtV1>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                           reinterpret_cast<const uint4*>(p0), reinterpret_cast<const uint4*>(p1),
                           reinterpret_cast<const uint4*>(p2), meta, N, K, nb, w);
    return hipGetLastError();
}

hipError_t launch_bf16_tile(const uint16_t* w, int64_t N, int64_t K, uint16_t* out, hipStream_t s) {
    const int64_t nb = blocks_of(N, K);
    const int64_t grid = (nb + 3) / 4;
    hipLaunchKernelGGL(bf16_tile_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, w, N, K, nb,
                       reinterpret_cast<uint4*>(out));
    return hipGetLastError();
}

}  // namespace w12
