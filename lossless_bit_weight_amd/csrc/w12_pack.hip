// w12_pack.hip -- W12-v1 encoder (pack) and streaming decoder (unpack).
//
// Format: see w12.h.  The pages say only that BF16 is split into three 4-bit
// planes and that the format is lossless (AI Radar summary of SpecPilot,
// English edition, "Reasons"); the group/base rule and the layout are this
// library's W12-v1.
//
// Work split: one thread owns 32 consecutive weights of the row-major
// tensor, i.e. one 16-byte slice of each plane and a quarter of a 128-weight
// group; 4 neighbouring lanes of a wave form one group.  Because K % 128 == 0
// a group never straddles rows, so the flat index is all a thread needs.
// Both kernels are single streaming passes: 64 B read + 48 B written per
// thread (pack), 48 B + 1 B read and 64 B written (unpack).
#include "w12_decode.hpp"
#include "w12_internal.hpp"

namespace w12 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

__global__ __launch_bounds__(kThreads) void pack_kernel(const uint4* __restrict__ w,
                                                        int64_t slices,
                                                        uint4* __restrict__ p0,
                                                        uint4* __restrict__ p1,
                                                        uint4* __restrict__ p2,
                                                        uint8_t* __restrict__ meta,
                                                        uint32_t* __restrict__ bad_count) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const bool active = i < slices;

    uint32_t v[16];  // 32 BF16 words, two per dword, natural order
    if (active) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 d = w[4 * i + q];
            v[4 * q + 0] = d.x;
            v[4 * q + 1] = d.y;
            v[4 * q + 2] = d.z;
            v[4 * q + 3] = d.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = 0;
    }

    // Largest biased exponent over the group (4 lanes x 32 weights).
    uint32_t emax = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        emax = max_u32(emax, (v[q] >> 7) & 0xFFu);
        emax = max_u32(emax, (v[q] >> 23) & 0xFFu);
    }
    emax = max_u32(emax, (uint32_t)__shfl_xor((int)emax, 1));
    emax = max_u32(emax, (uint32_t)__shfl_xor((int)emax, 2));
    const uint32_t beta = emax <= 15u ? 0u : (emax - 14u) >> 1;
    const uint32_t floor_e = 2u * beta + 2u;

    // Per weight: low byte kept, high byte -> sign<<3 | h.
    uint32_t lo[32], code[32];
    uint32_t bad = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const uint32_t word = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const uint32_t ex = (word >> 7) & 0xFFu;
        const uint32_t s = word >> 15;
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
        lo[e] = l;
        code[e] = (s << 3) | h;
    }

    // Split-nibble order: dword b of a plane holds weights 8b..8b+7; byte j
    // carries weight 8b+j (low nibble) and 8b+j+4 (high nibble).
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

    bad |= (uint32_t)__shfl_xor((int)bad, 1);
    bad |= (uint32_t)__shfl_xor((int)bad, 2);

    if (active) {
        p0[i] = make_uint4(o0[0], o0[1], o0[2], o0[3]);
        p1[i] = make_uint4(o1[0], o1[1], o1[2], o1[3]);
        p2[i] = make_uint4(o2[0], o2[1], o2[2], o2[3]);
        if ((i & 3) == 0) meta[i >> 2] = (uint8_t)(beta | (bad << 7));
    }

    // One atomic per wave: the number of flagged groups led by this wave.
    const uint64_t leaders = __ballot(active && (i & 3) == 0 && bad);
    if (bad_count != nullptr && (threadIdx.x & 63) == 0 && leaders != 0)
        atomicAdd(bad_count, (uint32_t)__popcll(leaders));
}

__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint4* __restrict__ p0,
                                                          const uint4* __restrict__ p1,
                                                          const uint4* __restrict__ p2,
                                                          const uint8_t* __restrict__ meta,
                                                          int64_t slices,
                                                          uint4* __restrict__ w) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= slices) return;
    const uint4 a = p0[i], b = p1[i], c = p2[i];
    const Lut t = make_lut(meta[i >> 2] & 0x7Fu);
    const uint32_t pa[4] = {a.x, a.y, a.z, a.w};
    const uint32_t pb[4] = {b.x, b.y, b.z, b.w};
    const uint32_t pc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t o[4];
        decode8(pa[q], pb[q], pc[q], t, o);
        w[4 * i + q] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

hipError_t launch_pack(const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1, void* p2,
                       uint8_t* meta, uint32_t* bad, hipStream_t s) {
    const int64_t slices = N * K / 32;
    const int64_t blocks = (slices + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint4*>(w), slices,
                       reinterpret_cast<uint4*>(p0), reinterpret_cast<uint4*>(p1),
                       reinterpret_cast<uint4*>(p2), meta, bad);
    return hipGetLastError();
}

hipError_t launch_unpack(const void* p0, const void* p1, const void* p2, const uint8_t* meta,
                         int64_t N, int64_t K, uint16_t* w, hipStream_t s) {
    const int64_t slices = N * K / 32;
    const int64_t blocks = (slices + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint4*>(p0), reinterpret_cast<const uint4*>(p1),
                       reinterpret_cast<const uint4*>(p2), meta, slices,
                       reinterpret_cast<uint4*>(w));
    return hipGetLastError();
}

}  // namespace w12
