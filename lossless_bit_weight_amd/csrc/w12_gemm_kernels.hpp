// w12_gemm_kernels.hpp -- kernel templates of the small-M decode GEMM
// y = x . W^T for gfx950; W is fetched either from a W12 container (rebuilt
// to BF16 in registers) or from the BF16 control layout.  Instantiated per x
// height by w12_gemm_inst.hip and launched through w12_gemm.hip.
//
// The pages: in single-request decoding every step reads all target weights
// while only a few tokens are accepted, and kernels are tuned against the
// memory-bandwidth limit (AI Radar summary of SpecPilot, English edition,
// opening paragraph); W12 is rebuilt bit-exactly inside the GEMM at batch
// 1-32 (HotRepo digest of StargazerX0/SpecPilot, project introduction).  So
// the kernel is a weight stream -- 1.5 B per weight for W12, 2 B for BF16 --
// with x small enough to sit in LDS.
//
// Structure shared by both variants and both weight fetches:
//   * both weight layouts are tiled: one (16-row tile, 128-weight group)
//     block is 1 KB per plane (W12) or 4 x 1 KB (BF16), stored in lane
//     order, so every load instruction of a wave reads 1 KB of contiguous
//     memory.  Lane L = 16 q + col holds row col of the tile and the 32
//     weights k = 128 g + 32 b + 8 q + e; its 8-weight block b is ready as
//     4 dwords of BF16 pairs after decode;
//   * a workgroup (4, 8 or 16 waves) owns R tiles per row-wave over one K slice
//     (grid y; the whole K unless K is split across workgroups); KW of its
//     waves split the slice's groups (group g0 + i goes to K-wave i % KW)
//     and add their partial sums through LDS in a fixed order;
//   * with K split over S workgroups: S = 2 (up to 32 rows) publishes each
//     output with one atomic exchange and the second arriver adds the two
//     slices in slice order; S > 2 writes the slices' fp32 sums to a
//     workspace and the last of a row block to finish (an atomic counter)
//     adds them in slice order -- so the result never depends on which
//     workgroup finishes last, and no workgroup waits for another;
//   * each lane keeps D groups in flight in a register ring unrolled at
//     compile time; every ring load is issued unconditionally (indices are
//     clamped to valid memory), so the compiler waits only for the oldest
//     group instead of draining the ring;
//   * x lives in LDS (the columns of the workgroup's K slice).  If they fit
//     they are loaded once, before the ring is primed, so the prologue
//     barrier waits for x only.  Otherwise they are double-buffered in
//     chunks of KC columns loaded one chunk ahead (chunks 0 and 1 both
//     before the ring is primed), one barrier per chunk, between ring
//     windows.  In x-direct mode each ring slot carries its group's x values
//     instead and there is no x barrier at all;
// GEMV (M <= 8; the default at M = 1): v_dot2c_f32_bf16 into fp32, x[m]
// read as a broadcast (all 16 lanes of a quarter read the same 16 bytes);
// the 4 quarter sums of a row are added with a fixed xor butterfly.
// MFMA (M <= 32; the default from M = 2): v_mfma_f32_16x16x32_bf16; block b
// of lane (col, q) is the B fragment of MFMA b, which therefore contracts the
// K set {32 b + 8 q + e}; the A fragment (x row col) is read with the same
// permutation, so the four MFMAs of a group cover its 128 K exactly once.
// The W12 and BF16 fetches feed identical operands in identical order, so
// for W = unpack(pack(W)) both return bitwise equal y.
// An exception list (the escape path that keeps every group lossless) adds,
// for each listed weight, x * (original - clamp) as (acc - x * clamp) +
// x * original, in list order: prepared by an extra wave in the x-direct
// kernels, applied group by group inside the main loop in the LDS-staged
// MFMA kernels up to 32 rows, walked after the loop elsewhere.
#pragma once

#include <type_traits>

#include "w12_decode.hpp"
#include "w12_internal.hpp"

namespace w12 {
namespace kern {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
}

// Every lane takes the value of quad position b of its own quad (DPP
// quad_perm [b, b, b, b]); b is 0..3 after unrolling.
__device__ __forceinline__ uint32_t quad_bcast1(uint32_t v, int b) {
    switch (b) {
        case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, true);
        case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, true);
        case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, true);
        default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, true);
    }
}
__device__ __forceinline__ uint4 quad_bcast(const uint4& v, int b) {
    return make_uint4(quad_bcast1(v.x, b), quad_bcast1(v.y, b), quad_bcast1(v.z, b), quad_bcast1(v.w, b));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void store_y(const GemmArgs& g, int m, int64_t n, float v) {
    if (g.y_f32)
        reinterpret_cast<float*>(g.y)[(int64_t)m * g.ldy + n] = v;
    else
        reinterpret_cast<uint16_t*>(g.y)[(int64_t)m * g.ldy + n] = f32_to_bf16_rne(v);
}

// A finished sum of one K slice: y itself when K is not split, else the
// slice's partial sum ws[s][m][n] (Np = N rounded up to 16 columns), stored
// with device scope (written through to the device coherence point, so no
// cache maintenance is needed to publish it).
__device__ __forceinline__ void out_value(const GemmArgs& g, int m, int64_t n, float v) {
    if (gridDim.y == 1) {
        store_y(g, m, n, v);
    } else {
        const int64_t np = (g.N + 15) / 16 * 16;
        __hip_atomic_store(g.ws + ((int64_t)blockIdx.y * g.M + m) * np + n, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

// K split in exactly two slices (MFMA and GEMV tiles up to 32 rows): each
// output is published with ONE 64-bit atomic exchange of (kPairTag << 32 |
// its fp32 bits) into its slot, ws64[m][n] (Np columns; the slots occupy the
// bytes the two slices' partial sums would).  The workgroup that gets its
// partner's tagged value back adds the two in slice order -- slice 0's sum
// plus slice 1's, whichever arrives second, so y never depends on the order
// of arrival -- stores y and clears the slot; the other gets back anything
// else and is done.  One memory round trip per output batch, against the
// store, completion wait, counter round trip and reload of split_finish.
// The tag is a word no fp32 partial sum of BF16 products can be (a NaN
// whose low 16 payload bits are ones: NaNs from BF16 operands carry zero
// low bits, NaNs made by invalid operations are the default quiet NaN), so
// the partial sums that other launches leave in the workspace (three or
// more slices, or 64- and 128-row tiles) never read as a published slot,
// and a zero-filled workspace starts with every slot empty.
constexpr uint32_t kPairTag = 0xFFFFFFFFu;
__device__ __forceinline__ uint64_t pair_publish(const GemmArgs& g, int m, int64_t n, float v) {
    const int64_t np = (g.N + 15) / 16 * 16;
    uint64_t* slot = reinterpret_cast<uint64_t*>(g.ws) + (int64_t)m * np + n;
    return __hip_atomic_exchange(slot, ((uint64_t)kPairTag << 32) | __builtin_bit_cast(uint32_t, v),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void pair_complete(const GemmArgs& g, int m, int64_t n, float v,
                                              uint64_t old) {
    if ((uint32_t)(old >> 32) != kPairTag) return;   // the partner finishes this output
    const float o = __builtin_bit_cast(float, (uint32_t)old);
    store_y(g, m, n, blockIdx.y == 0 ? v + o : o + v);
    const int64_t np = (g.N + 15) / 16 * 16;
    __hip_atomic_store(reinterpret_cast<uint64_t*>(g.ws) + (int64_t)m * np + n, (uint64_t)0,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Split-K epilogue for three or more slices, run by every thread of a
// workgroup after its partial sums are stored.  The workgroups of one row block count themselves in
// cnt[block]; the last one to arrive adds the S partial sums of the block in
// slice order 0, 1, ..., S-1 (the same order whichever workgroup is last, so
// y is deterministic) and resets the counter to zero for the next launch.
// No workgroup waits for another.
//
// Publication without whole-cache maintenance: partial sums are written and
// read with device-scope accesses (they bypass the per-XCD caches), each
// wave waits until its own stores have completed before the workgroup
// barrier, and only then does one thread bump the device-scope counter.  A
// workgroup that sees the count reach S - 1 therefore reads complete sums.
// (A release/acquire fence here would write back and invalidate the whole
// L2 of the XCD once per workgroup, which serialised the launch.)
template <int kTilesPerWG, int NT>
__device__ __forceinline__ void split_finish(const GemmArgs& g) {
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial-sum stores are complete
    __syncthreads();
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(g.cnt + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == gridDim.y - 1;
    __syncthreads();
    if (!last) return;
    constexpr int kRows = kTilesPerWG * 16;
    const int64_t np = (g.N + 15) / 16 * 16;
    const int64_t n0 = (int64_t)blockIdx.x * kRows;
    const int64_t slice = (int64_t)g.M * np;
    for (int i = threadIdx.x; i < kRows * g.M; i += NT) {
        const int m = i / kRows;
        const int64_t n = n0 + i % kRows;
        if (n >= g.N) continue;
        const float* p = g.ws + (int64_t)m * np + n;
        float v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int s = 1; s < (int)gridDim.y; ++s)
            v += __hip_atomic_load(p + s * slice, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        store_y(g, m, n, v);
    }
    if (threadIdx.x == 0) __hip_atomic_store(g.cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same protocol for the 64- and 128-row MFMA tiles, whose workgroups
// hold up to 16K outputs: split_arrive counts the workgroup in (true in every
// thread of the last one, which also resets the counter), and split_sum then
// lets each lane finish the outputs it stored itself, taking its own slice
// from registers and issuing the loads of the other slices together instead
// of one output (and one memory round trip) after another.  (In the 16- and
// 32-row kernels this form measured slower than split_finish.)
__device__ __forceinline__ bool split_arrive(const GemmArgs& g) {
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial-sum stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const bool l = __hip_atomic_fetch_add(g.cnt + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) == gridDim.y - 1;
        // all S workgroups have counted: nothing else touches the counter in
        // this launch
        if (l) __hip_atomic_store(g.cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = l;
    }
    __syncthreads();
    return last;
}

// Output (m, n) of y held in a lane's register i; ok = false: no output.
struct OutPos {
    int m;
    bool ok;
    int64_t n;
};

// In the last workgroup of a row block: v[i] holds this slice's sum of the
// output pos(i) (an OutPos); it becomes the sum of the S slices' partial sums, added in slice order
// 0, 1, ..., S-1 (the same order whichever workgroup is last, so y is
// deterministic).  This slice's term comes from v itself; the loads of the
// other slices are issued kP slices x kC outputs at a time, so that they
// are in flight together.
template <int NO, class Pos>
__device__ __forceinline__ void split_sum(const GemmArgs& g, float (&v)[NO], Pos pos) {
    constexpr int kC = NO < 32 ? NO : 32;
    constexpr int kP = kC <= 16 ? 2 : 1;
    static_assert(NO % kC == 0, "outputs come in whole chunks");
    const int S = (int)gridDim.y;
    const int me = (int)blockIdx.y;
    const int64_t np = (g.N + 15) / 16 * 16;
    const int64_t slice = (int64_t)g.M * np;
#pragma unroll
    for (int c0 = 0; c0 < NO; c0 += kC) {
        float acc[kC];
        for (int s0 = 0; s0 < S; s0 += kP) {
            float t[kP][kC];
#pragma unroll
            for (int p = 0; p < kP; ++p) {
                const int s = s0 + p;
#pragma unroll
                for (int i = 0; i < kC; ++i) {
                    const OutPos o = pos(c0 + i);
                    if (s == me)
                        t[p][i] = v[c0 + i];
                    else if (s < S && o.ok)
                        t[p][i] = __hip_atomic_load(g.ws + s * slice + (int64_t)o.m * np + o.n,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        t[p][i] = 0.f;
                }
            }
#pragma unroll
            for (int p = 0; p < kP; ++p)
#pragma unroll
                for (int i = 0; i < kC; ++i)
                    if (s0 + p < S) acc[i] = s0 + p == 0 ? t[p][i] : acc[i] + t[p][i];
        }
#pragma unroll
        for (int i = 0; i < kC; ++i) v[c0 + i] = acc[i];
    }
}

// Exception corrections (W12 containers with an exception list): the main
// loop multiplied each exception element's stored clamp (sign | window floor:
// 2^(2 beta + 2 - 127) in W12-v1, 2^(b + 1 - 127) in W12-b); for every entry of `tile` whose group lies in this
// workgroup's K slice [g0, g0 + gn), the sum first takes back x[m][k] * clamp
// and then adds x[m][k] * original (two fused multiply-adds; a precomputed
// difference would round away originals far below the clamp).
//
// Entries are handled 64 at a time by one wave: lane i loads entry i and the
// x[m][k] it needs (all loads of a batch in flight together), stages them in
// the wave's LDS area, and then every lane walks, in list order, only the
// entries of its own row (col == c; found with one ballot per row).  The
// per-wave area holds 64 x (original, clamp) words, a spare word, and
// XR x 64 BF16 x values.
__device__ __forceinline__ float bf16_to_f32(uint32_t v) { return __builtin_bit_cast(float, v << 16); }

template <int XR>
struct ExcStage {
    static constexpr int kBytes = 64 * 3 * 4 + XR * 64 * 2;
};
// x rows one pass of the corrections stages: all of them for the GEMV and
// MFMA tiles up to 32 rows, 16 at a time above (so that eight staging areas
// fit beside a 128 KB x double buffer).
__host__ __device__ constexpr int exc_rows(bool mfma, int mr) {
    return !mfma || mr <= 32 ? mr : 16;
}

// The walk over one staged batch: lane i of the batch holds the entry of row
// c_i (-1: none); its original and clamp are at area+256 / area+512 and its
// x values at area+768, 64 per x row.  Each lane applies, in list order,
// only the entries of its own row (col).
template <class Apply>
__device__ __forceinline__ void exc_walk(int lane, int col, const uint8_t* area, int c, Apply apply) {
    const float* orig = reinterpret_cast<const float*>(area + 256);
    const float* clamp = reinterpret_cast<const float*>(area + 512);
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(area + 768);
    // LDS accesses of one wave complete in order; keep the compiler from
    // moving the reads below above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // The batch entries of this lane's row, as a lane mask (list order =
    // ascending bit); each lane then walks only its own entries.
    uint64_t mine = 0;
#pragma unroll 1
    for (int cc = 0; cc < 16; ++cc) {
        const uint64_t b = __ballot(c == cc);
        if (col == cc) mine = b;
    }
    while (mine != 0) {
        const int j = __ffsll((unsigned long long)mine) - 1;
        mine &= mine - 1;
        apply(orig[j], clamp[j], [&](int m) { return bf16_to_f32(xs[m * 64 + j]); });
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    (void)lane;
}

// apply(j, orig, clamp, xs) runs on the lanes of entry j's row; xs(m) reads
// that entry's x[mb + m][k] from LDS (XR rows from row mb < M).
// F::clamp_word(entry word 1) gives the BF16 clamp the planes hold for the
// entry.  The entries walked are [beg, end) of the list (by default the
// slice's blocks of `tile`).
// With `use_first` the lane's entry of the first batch (entry beg + lane,
// when it exists) is `first` instead of being loaded.
template <class F, int XR, class Apply>
__device__ __forceinline__ void exc_corrections(const GemmArgs& g, int64_t tile, int g0, int gn,
                                                int lane, int col, uint8_t* area, int mb,
                                                Apply apply, int64_t beg_in = -1,
                                                int64_t end_in = -1, bool use_first = false,
                                                uint2 first = {0u, 0u}) {
    float* orig = reinterpret_cast<float*>(area + 256);
    float* clamp = reinterpret_cast<float*>(area + 512);
    uint16_t* xs = reinterpret_cast<uint16_t*>(area + 768);
    // the entries of the slice's blocks (tile, g0) .. (tile, g0 + gn - 1)
    uint32_t beg, end;
    if (beg_in >= 0) {
        beg = (uint32_t)beg_in;
        end = (uint32_t)end_in;
    } else {
        const int64_t blk0 = tile * (g.K / 128) + g0;
        beg = g.exc_off[blk0];
        end = g.exc_off[blk0 + gn];
    }
    for (uint32_t base = beg; base < end; base += 64) {
        const uint32_t i = base + (uint32_t)lane;
        int c = -1;
        float o = 0.f, cl = 0.f;
        int64_t k = 0;
        if (i < end) {
            const bool pre = use_first && base == beg;
            const uint32_t pos = pre ? first.x : g.exc_ent[2 * (int64_t)i];
            const uint32_t val = pre ? first.y : g.exc_ent[2 * (int64_t)i + 1];
            k = pos & 0xFFFFFFu;
            const int grp = (int)(k >> 7);
            if (grp >= g0 && grp < g0 + gn) {
                c = (int)(pos >> 24);
                o = bf16_to_f32(val & 0xFFFFu);
                cl = bf16_to_f32(F::clamp_word(val));
            }
        }
        orig[lane] = o;
        clamp[lane] = cl;
        // x[m][k] for the batch, sixteen rows of loads in flight at a time;
        // rows past M and lanes without an entry store zero (a zero x adds
        // nothing, so the consumers need no row test)
        // a per-lane running row pointer, from row mb
        const uint16_t* px = g.x + (int64_t)mb * g.ldx + (c >= 0 ? k : 0);
        const uint32_t keep = c >= 0 ? 0xFFFFu : 0u;
        constexpr int kRound = XR < 16 ? XR : 16;
#pragma unroll 1
        for (int m0 = 0; m0 < XR; m0 += kRound) {
            uint16_t xv[kRound];
#pragma unroll
            for (int d = 0; d < kRound; ++d) {
                xv[d] = *px;
                px += mb + m0 + d + 1 < g.M ? g.ldx : 0;   // stays on the last row of x
            }
            const int valid = g.M - mb - m0;
#pragma unroll
            for (int d = 0; d < kRound; ++d)
                xs[(m0 + d) * 64 + lane] = (uint16_t)(d < valid ? xv[d] & keep : 0u);
        }
        exc_walk(lane, col, area, c, apply);
    }
}

// ---- weight fetch policies ------------------------------------------------
// Weights are read once per GEMM, so their 16-byte loads are non-temporal
// (the `nt` cache policy: streamed through the caches without displacing x
// or the exception data).  Measured on MI355X: a plain streaming read of
// 55 MB ran at 5.5 TB/s with ordinary loads and 5.85 TB/s with `nt`; the
// QKV GEMV at M = 1 went from 12.55 to 11.28 us.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// load(): the 32 weights lane `lane` owns in block `blk` (= tile * G + group)
// into raw registers; block(): its 8-weight block b (0..3) as 4 dwords of
// BF16 pairs in natural k order.

struct FetchW12 {
    // kHasExceptions: the container may carry an exception list, whose
    // corrections are added to the sums.  kExcWave (W12-v1 with a list): in
    // the kernels that read x directly an extra wave of the workgroup
    // prepares those corrections while the others stream the weights; the
    // LDS-staged MFMA kernels up to 32 rows apply them inside the main loop;
    // every other kernel walks the list after the main loop.
    static constexpr bool kHasExceptions = false;
    static constexpr bool kExcWave = false;
    static constexpr bool kHasMeta = true;
    struct Raw {
        uint4 a, b, c;
        // the meta byte as loaded: widened only where a group is computed,
        // so no arithmetic on it is placed right after its load (in the
        // x-staged kernels that put a wait for the whole primed ring before
        // the first x barrier)
        uint8_t beta;
    };
    // Wave-uniform part of the addresses of tile `tile` (all groups); the
    // lane part is added per load.
    struct Base {
        const uint8_t *p0, *p1, *p2, *meta;
    };
    __device__ __forceinline__ static Base base(const GemmArgs& g, int64_t tile) {
        const int64_t blk0 = tile * (g.K / 128);
        return Base{g.p0 + blk0 * 1024, g.p1 + blk0 * 1024, g.p2 + blk0 * 1024, g.meta + blk0 * 16};
    }
    __device__ __forceinline__ static void load(const Base& b, int grp, int lane, Raw& r) {
        const uint32_t off = (uint32_t)grp * 1024u + 16u * (uint32_t)lane;
        r.a = load_stream(b.p0 + off);
        r.b = load_stream(b.p1 + off);
        r.c = load_stream(b.p2 + off);
    }
    // The meta byte of row (lane & 15) in group grp (each quarter of a wave
    // may ask for a different group).
    __device__ __forceinline__ static uint8_t load_meta(const Base& b, int grp, int lane) {
        return b.meta[(uint32_t)grp * 16u + (uint32_t)(lane & 15)];
    }
    __device__ __forceinline__ static void block(const Raw& r, int b, uint32_t out[4]) {
        const Lut t = make_lut(r.beta & 0x7Fu);
        const uint32_t pa = b == 0 ? r.a.x : b == 1 ? r.a.y : b == 2 ? r.a.z : r.a.w;
        const uint32_t pb = b == 0 ? r.b.x : b == 1 ? r.b.y : b == 2 ? r.b.z : r.b.w;
        const uint32_t pc = b == 0 ? r.c.x : b == 1 ? r.c.y : b == 2 ? r.c.z : r.c.w;
        decode8(pa, pb, pc, t, out);
    }
    // Exception entry word 1 = beta << 16 | original: the clamp is the
    // window floor 2^(2 beta + 2 - 127) with the original's sign.
    __device__ __forceinline__ static uint32_t clamp_word(uint32_t val) {
        return (val & 0x8000u) | ((2u * ((val >> 16) & 0x7Fu) + 2u) << 7);
    }
};

// W12-v1 with an exception list (the same planes and decode).
struct FetchW12X : FetchW12 {
    static constexpr bool kHasExceptions = true;
    static constexpr bool kExcWave = true;
};

// The arbitrary-base allocation W12-b: same planes and loads, the meta byte
// is the base b itself (0..240), decode8b rebuilds E = b + c.
struct FetchW12B : FetchW12 {
    static constexpr bool kHasExceptions = true;
    __device__ __forceinline__ static void block(const Raw& r, int b, uint32_t out[4]) {
        const uint32_t pa = b == 0 ? r.a.x : b == 1 ? r.a.y : b == 2 ? r.a.z : r.a.w;
        const uint32_t pb = b == 0 ? r.b.x : b == 1 ? r.b.y : b == 2 ? r.b.z : r.b.w;
        const uint32_t pc = b == 0 ? r.c.x : b == 1 ? r.c.y : b == 2 ? r.c.z : r.c.w;
        decode8b(pa, pb, pc, (r.beta & 0xFFu) * 0x01010101u, out);
    }
    // Entry word 1 = b << 16 | original: the clamp is 2^(b + 1 - 127).
    __device__ __forceinline__ static uint32_t clamp_word(uint32_t val) {
        return (val & 0x8000u) | ((((val >> 16) & 0xFFu) + 1u) << 7);
    }
};

struct FetchBF16 {
    static constexpr bool kHasExceptions = false;
    static constexpr bool kExcWave = false;
    static constexpr bool kHasMeta = false;
    struct Raw {
        uint4 q[4];
        uint32_t beta;   // unused
    };
    struct Base {
        const uint8_t* w;
    };
    __device__ __forceinline__ static Base base(const GemmArgs& g, int64_t tile) {
        return Base{reinterpret_cast<const uint8_t*>(g.w) + tile * (g.K / 128) * 4096};
    }
    __device__ __forceinline__ static void load(const Base& b, int grp, int lane, Raw& r) {
        const uint32_t off = (uint32_t)grp * 4096u + 16u * (uint32_t)lane;
#pragma unroll
        for (int i = 0; i < 4; ++i) r.q[i] = load_stream(b.w + off + 1024u * i);
    }
    __device__ __forceinline__ static void block(const Raw& r, int b, uint32_t out[4]) {
        out[0] = r.q[b].x;
        out[1] = r.q[b].y;
        out[2] = r.q[b].z;
        out[3] = r.q[b].w;
    }
};

// ---- x staging ----------------------------------------------------------------
// x[0:MROWS][k0:k0+KC] -> LDS in 16-byte units (8 BF16); rows >= M and
// columns >= K are zero.  Layout::phys(row, unit) is the LDS slot.

template <int MROWS, int KC, int NT>
struct XChunk {
    static constexpr int kUnitsPerRow = KC / 8;
    static constexpr int kUnits = MROWS * kUnitsPerRow;
    static constexpr int kPerThread = (kUnits + NT - 1) / NT;
    uint4 v[kPerThread];

    // Every lane issues every load (addresses clamped into x), and values
    // outside x are zeroed afterwards: unpredicated loads let the compiler
    // count outstanding loads exactly instead of draining the weight ring.
    __device__ __forceinline__ void load(const GemmArgs& g, int64_t k0) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int id = threadIdx.x + NT * j;
            const int m = id / kUnitsPerRow;
            const int64_t k = k0 + 8 * (id % kUnitsPerRow);
            const bool ok = id < kUnits && m < g.M && k < g.K;
            const int mc = m < g.M ? m : g.M - 1;
            const int64_t kc = k < g.K ? k : g.K - 8;
            const uint4 v0 = *reinterpret_cast<const uint4*>(g.x + (int64_t)mc * g.ldx + kc);
            v[j] = ok ? v0 : make_uint4(0, 0, 0, 0);
        }
    }
    template <class Layout>
    __device__ __forceinline__ void store(uint4* buf) const {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int id = threadIdx.x + NT * j;
            if (id < kUnits) buf[Layout::phys(id / kUnitsPerRow, id % kUnitsPerRow)] = v[j];
        }
    }
};

// Whole-x staging when all of x fits (at most kSingleBytes): loaded into
// registers before the weight ring is primed, stored to LDS after it, so
// waiting for x never waits for weights.  The registers die after the store.
constexpr int kSingleBytes = 40 * 1024;   // a multiple of 16 * 512

template <int NT>
struct XAll {
    static constexpr int kSingleUnits = (kSingleBytes / 16 + NT - 1) / NT;  // per thread
    uint4 v[kSingleUnits];
    int units, units_per_row;

    // Columns [k0, k0 + 8 * upr) of rows 0..mrows-1 (mrows * upr <=
    // kSingleUnits * NT, checked on the host).
    __device__ __forceinline__ void load(const GemmArgs& g, int mrows, int64_t k0, int upr) {
        units_per_row = upr;
        units = mrows * units_per_row;
#pragma unroll
        for (int j = 0; j < kSingleUnits; ++j) {
            // The guard is uniform over the workgroup (it depends on j and
            // the shape only), so the loads of a round are all issued or all
            // skipped and the count of later loads stays known.
            if (NT * j < units) {
                const int id = threadIdx.x + NT * j;
                const int m = id / units_per_row;
                const int64_t k = k0 + 8 * (int64_t)(id % units_per_row);
                const bool ok = id < units && m < g.M;
                const int mc = m < g.M ? m : g.M - 1;
                const uint4 v0 = *reinterpret_cast<const uint4*>(g.x + (int64_t)mc * g.ldx + k);
                v[j] = ok ? v0 : make_uint4(0, 0, 0, 0);
            }
        }
    }
    template <class Layout>
    __device__ __forceinline__ void store(uint4* buf) const {
#pragma unroll
        for (int j = 0; j < kSingleUnits; ++j) {
            const int id = threadIdx.x + NT * j;
            if (id < units)
                buf[Layout::phys(id / units_per_row, id % units_per_row, units_per_row)] = v[j];
        }
    }
};

// x layout in LDS: row m, 16-byte unit u at slot m * units_per_row +
// (u ^ (m & 7)).  The MFMA reads one unit of rows m = 0..15 per instruction
// and the xor spreads them over 8 different 16-byte bank slots; the GEMV
// reads the same unit of a row from all lanes of a quarter (a broadcast).
struct XLayout {
    __device__ __forceinline__ static int phys(int m, int u, int units_per_row) {
        return m * units_per_row + (u ^ (m & 7));
    }
};

template <class L, int UPR>
struct FixedLayout {
    __device__ __forceinline__ static int phys(int m, int u) { return L::phys(m, u, UPR); }
};

// ---- compile-time chunk sizes ---------------------------------------------------
// Chunked mode double-buffers KC columns of x.  KC is a multiple of one ring
// window of the workgroup (D slices of each of the KW K-waves), so chunk
// transitions fall between ring windows.

__host__ __device__ constexpr int gemv_kc(int M, int KW, int D) {
    const int base = M <= 1 ? 8192 : M <= 2 ? 4096 : M <= 4 ? 2048 : 1024;
    const int window = 128 * KW * D;
    return base < window ? window : base;
}
__host__ __device__ constexpr int mfma_kc(int MT, int KW, int D) {
    const int base = MT == 16 ? 512 : 256;
    const int window = 128 * KW * D;
    return base < window ? window : base;
}
// A chunked variant is built only if each thread stages at most 8 x 16
// bytes of a chunk (x rows * KC <= 64 * threads) and the double buffer
// stays within 128 KB of LDS (of the 160 KB a workgroup may hold): 64 KB
// for 256 threads, 128 KB for 512 and 1024.
__host__ __device__ constexpr bool chunk_ok(int rows, int kc, int nw) {
    return rows * kc <= 4096 * (nw < 8 ? nw : 8);
}
__host__ __device__ constexpr int kc_of(bool mfma, int rows, int KW, int D) {
    return mfma ? mfma_kc(rows, KW, D) : gemv_kc(rows, KW, D);
}

// Compile-time loops for the ring's tails: f(integral_constant<int, i>) for
// i = I .. N - 1, and f(integral_constant<int, v>) for the runtime v in
// [I, N) (nothing for any other v).
template <int I, int N, class F>
__device__ __forceinline__ void w12_static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        w12_static_for<I + 1, N>(f);
    }
}
template <int I, int N, class F>
__device__ __forceinline__ void w12_select(int v, F&& f) {
    if constexpr (I < N) {
        if (v == I)
            f(std::integral_constant<int, I>{});
        else
            w12_select<I + 1, N>(v, f);
    }
}

// The main loop shared by both variants.  `fetch(j, ring[d], d)` loads wave
// slice j (clamped to the wave's last slice, so it always issues the same
// loads), `compute(ring[d], j, d)` consumes it, `correct(j)` follows the
// refill of its slot, `xbuf` is the LDS chunk base.
// Ring slot d always holds slice jb + d, so the compiler sees straight-line
// loads and waits exactly for the oldest slice.  The last window is peeled
// off the loop and refills only the slices that remain: a load issued past
// the wave's last slice would never be consumed, yet its destination
// registers are reused by the epilogue, which then has to wait a full
// memory round trip for it (measured: 1.8 us of a 15 us launch at M = 16).
#define W12_CHUNK_STEP(CHUNKED, L, nchunks, xr, store_next)                             \
    if constexpr (CHUNKED) {                                                              \
        if (jb < (J) && jb == next_boundary) {                                            \
            store_next();                                                                 \
            __syncthreads();                                                              \
            ++c;                                                                          \
            next_boundary += (L);                                                         \
            if (c + 1 < (nchunks)) xr.load(g, kbase + (int64_t)(c + 1) * KC);             \
        }                                                                                 \
    }

#define W12_RING_LOOP(D, CHUNKED, J, L, nchunks, xr, store_next, fetch, compute)          \
    {                                                                                     \
        int jb = 0;                                                                       \
        /* windows after which at least one more full window follows: every */          \
        /* refill is a live group, and the loads are unconditional */                     \
        for (; jb + 2 * (D) <= (J); jb += (D)) {                                          \
            W12_CHUNK_STEP(CHUNKED, L, nchunks, xr, store_next)                           \
            _Pragma("unroll") for (int d = 0; d < (D); ++d) {                             \
                compute(ring[d], jb + d, d);                                              \
                fetch(jb + d + (D), ring[d], d);                                          \
                correct(jb + d);                                                          \
                /* keep the next slot's arithmetic below this slot's loads */             \
                __builtin_amdgcn_sched_barrier(0);                                        \
            }                                                                             \
        }                                                                                 \
        /* the last window refills only the groups that remain, so no load */            \
        /* is left in flight after the loop; then the final partial window. */           \
        /* With D = 2 up to 32 rows each count of groups left (J - jb < 4) */           \
        /* has a tail */                                                                  \
        /* of its own in which every load is unconditional: with the loads */             \
        /* predicated the compiler could not count them and waited for all of */          \
        /* them -- the refill just issued included -- before each remaining */            \
        /* group, a memory round trip at the end of every wave. */                        \
        auto w12_tail = [&](auto rem_c) {                                                 \
            constexpr int rem = decltype(rem_c)::value;                                   \
            W12_CHUNK_STEP(CHUNKED, L, nchunks, xr, store_next)                           \
            w12_static_for<0, (D)>([&](auto d_c) {                                        \
                constexpr int d = decltype(d_c)::value;                                   \
                if constexpr (d < rem) compute(ring[d], jb + d, d);                       \
                if constexpr (d + (D) < rem) fetch(jb + d + (D), ring[d], d);             \
                if constexpr (d < rem) correct(jb + d);                                   \
                __builtin_amdgcn_sched_barrier(0);                                        \
            });                                                                           \
            if constexpr (rem > (D)) {                                                    \
                jb += (D);                                                                \
                W12_CHUNK_STEP(CHUNKED, L, nchunks, xr, store_next)                       \
                w12_static_for<0, (D)>([&](auto d_c) {                                    \
                    constexpr int d = decltype(d_c)::value;                               \
                    if constexpr (d + (D) < rem) {                                        \
                        compute(ring[d], jb + d, d);                                      \
                        correct(jb + d);                                                  \
                    }                                                                     \
                });                                                                       \
            }                                                                             \
            /* The tails end in different blocks, and where the sums are */              \
            /* matrix-core results read right after the join the compiler did */           \
            /* not always put the wait states such a read needs (measured: */              \
            /* stale sums in the BF16 control at 16 rows, two K-waves, x direct). */       \
            /* 24 wait states at the end of every tail cover any MFMA here. */            \
            if constexpr (MFMA) {                                                         \
                __builtin_amdgcn_sched_barrier(0);                                        \
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");                              \
                __builtin_amdgcn_sched_barrier(0);                                        \
            }                                                                             \
        };                                                                                \
        if constexpr ((D) <= 2 && MR <= 32) {                                             \
            w12_select<1, 2 * (D)>((J) - jb, w12_tail);                                   \
        } else if (jb < (J)) {                                                            \
            W12_CHUNK_STEP(CHUNKED, L, nchunks, xr, store_next)                           \
            _Pragma("unroll") for (int d = 0; d < (D); ++d) {                             \
                if (jb + d < (J)) compute(ring[d], jb + d, d);                            \
                if (jb + d + (D) < (J)) fetch(jb + d + (D), ring[d], d);                  \
                if (jb + d < (J)) correct(jb + d);                                        \
                __builtin_amdgcn_sched_barrier(0);                                        \
            }                                                                             \
            jb += (D);                                                                    \
            W12_CHUNK_STEP(CHUNKED, L, nchunks, xr, store_next)                           \
            _Pragma("unroll") for (int d = 0; d < (D); ++d) {                             \
                if (jb + d < (J)) {                                                       \
                    compute(ring[d], jb + d, d);                                          \
                    correct(jb + d);                                                      \
                }                                                                         \
            }                                                                             \
        }                                                                                 \
        /* Every thread stages its share of every x chunk, so a wave that ran */         \
        /* out of slices still performs the chunk transitions it did not reach. */        \
        if constexpr (CHUNKED) {                                                          \
            while (c + 1 < (nchunks)) {                                                   \
                store_next();                                                             \
                __syncthreads();                                                          \
                ++c;                                                                      \
                if (c + 1 < (nchunks)) xr.load(g, kbase + (int64_t)(c + 1) * KC);         \
            }                                                                             \
        }                                                                                 \
    }

// Bytes of LDS a launch needs (x buffers of one K slice of gs groups; the
// reductions reuse them).
template <bool MFMA, int MR, int R, int KW, int D, bool CHUNKED, bool XD, int NW>
__host__ __device__ size_t lds_bytes(int gs) {
    const size_t x = XD ? 0
                     : CHUNKED ? 2 * (size_t)MR * kc_of(MFMA, MR, KW, D) * 2
                               : (size_t)MR * gs * 128 * 2;
    const size_t red = KW == 1 ? 0
                       : MFMA ? (size_t)(KW - 1) * (NW / KW) * 64 * R * (MR / 16) * 16
                              : (size_t)(KW - 1) * (NW / KW) * 16 * R * MR * 4;
    const size_t m = x > red ? x : red;
    return (m + 15) / 16 * 16;
}
// With an exception list the owner waves also stage correction batches
// after the main loop.
template <bool MFMA, int MR, int KW, int NW>
__host__ __device__ constexpr size_t exc_lds_bytes() {
    return (size_t)(NW / KW) * ExcStage<exc_rows(MFMA, MR)>::kBytes;
}
// Where those batches go: with x staged in LDS and several K-waves the walk
// runs after the barrier that ends every read of x, so they reuse the x
// buffers after the reduction partials when they fit there (a separate area
// took the 32-row two-K-wave kernel past half the LDS, one workgroup per CU
// instead of two); otherwise they go after everything else.  `extra` = the
// LDS the launch must add for them.
template <bool MFMA, int MR, int R, int KW, int D, bool CHUNKED, bool XD, int NW>
__host__ __device__ size_t walk_base(int gs, size_t* extra) {
    const size_t x = XD ? 0
                     : CHUNKED ? 2 * (size_t)MR * kc_of(MFMA, MR, KW, D) * 2
                               : (size_t)MR * gs * 128 * 2;
    const size_t red = KW == 1 ? 0
                       : MFMA ? (size_t)(KW - 1) * (NW / KW) * 64 * R * (MR / 16) * 16
                              : (size_t)(KW - 1) * (NW / KW) * 16 * R * MR * 4;
    const size_t redr = (red + 15) / 16 * 16;
    const size_t need = exc_lds_bytes<MFMA, MR, KW, NW>();
    if (!XD && KW > 1 && redr + need <= x) {
        *extra = 0;
        return redr;
    }
    *extra = need;
    return lds_bytes<MFMA, MR, R, KW, D, CHUNKED, XD, NW>(gs);
}
// With a correction wave (F::kExcWave, x read directly): its one staging
// area, then the two correction sums of every output of the workgroup's
// tiles -- [tile of the workgroup][row in tile][x row][2] fp32.
template <int MR, int R, int KW, int NW>
__host__ __device__ constexpr size_t excwave_lds_bytes() {
    return (size_t)ExcStage<MR>::kBytes + (size_t)(NW / KW) * R * 16 * MR * 2 * 4;
}


// ---- the kernel ----------------------------------------------------------------------
// MFMA = false: GEMV, MR = M (1..8).  MFMA = true: MR = 16 or 32 (x rows,
// zero padded).

// XD: x is not staged in LDS; each ring slot also carries the x values of
// its group, loaded straight from memory (x is small and stays in L1/L2), so
// there is no x barrier at all and each wave waits only for its own loads.
// GEMV: one 16-byte load per x row and group, spread so that each quad of
// lanes holds the four pieces its quarter needs; block b's piece is then
// broadcast within the quad (DPP).  MFMA: each lane loads its own A
// fragments (row 16 mt + col); rows past M repeat row M - 1 instead of being
// zero -- they only feed output rows that are never stored.
template <class F, bool MFMA, int MR, int R, int KW, int D, bool CHUNKED, bool XD, int NW>
__global__ __launch_bounds__(NW * 64 + (F::kExcWave && XD ? 64 : 0)) void gemm_kernel(GemmArgs g) {
    static_assert(!(XD && CHUNKED), "direct x is never chunked");
    constexpr int KC = kc_of(MFMA, MR, KW, D);
    constexpr int kRowWaves = NW / KW;
    constexpr int kBuf = MR * KC / 8;                 // uint4 per x chunk buffer
    constexpr int L = KC / (128 * KW);                // wave groups per chunk (multiple of D)
    constexpr int kMT = MR / 16;                      // MFMA: 16-row tiles of x
    using Raw = typename F::Raw;
    extern __shared__ uint4 lds[];

    const int lane = threadIdx.x & 63;
    // wave-uniform by construction; readfirstlane tells the compiler, so the
    // loop bounds derived from it stay scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int col = lane & 15;   // weight row in the tile; A row for the MFMA
    const int q = lane >> 4;     // quarter: weights 8q..8q+7 of each 32
    const int kw = wave % KW;
    const int nw = wave / KW;
    const int64_t G = g.K / 128;
    const int64_t ntiles = (g.N + 15) / 16;
    // the correction wave's area (after the x buffers / reductions) and the
    // post-loop walk's (see walk_base)
    const size_t exc_base = lds_bytes<MFMA, MR, R, KW, D, CHUNKED, XD, NW>(g.gs);
    size_t walk_extra;
    const size_t walk_b = walk_base<MFMA, MR, R, KW, D, CHUNKED, XD, NW>(g.gs, &walk_extra);
    (void)walk_extra;
    const int64_t tile0 = ((int64_t)blockIdx.x * kRowWaves + nw) * R;  // tile r: tile0 + r

    int64_t tload[R];  // tiles past the end are clamped for loading
#pragma unroll
    for (int r = 0; r < R; ++r) tload[r] = tile0 + r < ntiles ? tile0 + r : ntiles - 1;

    // K slice of this workgroup: groups g0 .. g0 + gn - 1 (gn >= 1).
    const int g0 = (int)blockIdx.y * g.gs;
    const int gn = G - g0 < g.gs ? (int)(G - g0) : g.gs;
    const int64_t kbase = (int64_t)g0 * 128;
    const int J = gn > kw ? (gn - kw + KW - 1) / KW : 0;  // this wave's groups
    const int Jlast = J > 0 ? J - 1 : 0;
    const int units_per_row = CHUNKED ? KC / 8 : gn * 16;
    const int64_t nchunks = CHUNKED ? ((int64_t)gn * 128 + KC - 1) / KC : 1;
    int c = 0;
    int next_boundary = CHUNKED && nchunks > 1 ? L : 1 << 30;

    typename F::Base wbase[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wbase[r] = F::base(g, tload[r]);
    const int glast = g0 + gn - 1;

    // Exception list applied in or after the main loop (no correction
    // wave): the entry range of each tile's blocks in this K slice is read
    // here, before
    // any other load, through the scalar cache (uniform addresses; these
    // loads neither wait behind nor delay the vector loads), and once the
    // ring is primed every wave loads the first 64 entries of each range,
    // one per lane (exc_pre): the in-loop corrections take them from there,
    // and the walk after the loop starts with its entries in registers (one
    // memory round trip fewer); the entry loads are older than every ring
    // load the loop waits for.
    // Without a list the offsets read the first words of plane 0 and the
    // range stays empty.
    uint32_t exc_b[R], exc_e[R];
    uint2 exc_pre[R];
    if constexpr (F::kHasExceptions && !(F::kExcWave && XD)) {
        const bool has = g.exc_off != nullptr;
        const __attribute__((address_space(4))) uint32_t* off4 =
            (const __attribute__((address_space(4))) uint32_t*)(has ? g.exc_off
                                                                     : reinterpret_cast<const uint32_t*>(g.p0));
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t blk0 = has ? tload[r] * G + g0 : 0;
            exc_b[r] = off4[blk0];
            exc_e[r] = off4[has ? blk0 + gn : 0];
        }
    }
    // The entry loads (after the ring is primed): a lane past the range
    // reads its own tile's first plane-0 words instead (valid, and spread
    // over the tiles rather than one hot word), so the load is issued
    // unconditionally and the loop's wait counts stay exact.
    // In-loop corrections: W12-v1 with a list (that fetch is only launched
    // with one), MFMA, x staged in LDS, up to 32 x rows.
    constexpr bool kInLoop = F::kExcWave && MFMA && !XD && MR <= 32;
    auto exc_prefetch = [&]() {
        if constexpr (F::kHasExceptions && !(F::kExcWave && XD)) {
            const uint2* ent = reinterpret_cast<const uint2*>(g.exc_ent);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t i = exc_b[r] + (uint32_t)lane;
                const uint2* p = i < exc_e[r] ? ent + i
                                              : reinterpret_cast<const uint2*>(wbase[r].p0) + lane;
                exc_pre[r] = *p;
            }
        }
    };
    // In-loop corrections (MFMA kernels with x staged in LDS and a list):
    // the first 64 entries of each tile's slice (exc_pre, usually all of
    // them) are applied inside the main loop, each by the lanes of its row
    // right after the products of its group, with x read from the LDS copy;
    // entries past the first 64 are walked after the loop.  exc_grp is each
    // lane's entry's group (-1: none).  The entries are waited for once
    // before the loop: a first use inside the loop made the compiler wait
    // for them -- and for every load issued behind them -- on every pass.
    int exc_grp[R];
    auto exc_inloop_ready = [&]() {
        if constexpr (kInLoop) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t pos = exc_pre[r].x, val = exc_pre[r].y;
                asm volatile("" : "+v"(pos), "+v"(val));
                exc_pre[r] = make_uint2(pos, val);
                exc_grp[r] = exc_b[r] + (uint32_t)lane < exc_e[r] ? (int)((pos & 0xFFFFFFu) >> 7) : -1;
            }
        }
    };

    // The correction wave (exception list, x read directly): wave NW of the
    // workgroup walks the entries of every tile of the workgroup -- block
    // offsets, entries, the x values they need: three dependent memory round
    // trips, taken while the other waves stream the weights -- and leaves,
    // for each output, the sum of x[m][k] * clamp and the sum of
    // x[m][k] * original over its entries (list order, fp32) in LDS.  The
    // owner waves read them after the K-wave reduction barrier and form
    // (y - sum clamp) + sum original, so that a one-hot x row returns an
    // original word exactly.  The wave then takes part in exactly the
    // barriers the other waves still execute (the reduction, or its stand-in
    // with one K-wave; the two of a split-K finish of three or more slices).
    constexpr bool kExcWave = F::kExcWave && XD;
    float* exc_corr = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(lds) + exc_base +
                                               ExcStage<MR>::kBytes);
    if constexpr (kExcWave) {
        if (wave == NW) {
            // T tiles; the x values of TB tiles' entries are loaded in one
            // round (at most 64 values per lane)
            constexpr int T = kRowWaves * R;
            constexpr int TB = 64 / MR < 1 ? 1 : (64 / MR > T ? T : 64 / MR);
            uint8_t* area = reinterpret_cast<uint8_t*>(lds) + exc_base;
            const int64_t tbase = (int64_t)blockIdx.x * T;
            // 1. the block offsets of every tile's slice: uniform addresses,
            // so scalar loads, which do not queue behind the vector loads of
            // the weight streams on this CU
            const uint2* ent = reinterpret_cast<const uint2*>(g.exc_ent);
            const __attribute__((address_space(4))) uint32_t* off4 =
                (const __attribute__((address_space(4))) uint32_t*)g.exc_off;
            uint32_t beg[T], end[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int64_t tl = tbase + t < ntiles ? tbase + t : ntiles - 1;
                const uint32_t b0 = off4[tl * G + g0];
                const uint32_t e0 = off4[tl * G + g0 + gn];
                beg[t] = b0;
                end[t] = tbase + t < ntiles ? e0 : b0;
            }
            // 2. the first 64 entries of every tile, all loads in flight at once
            uint2 e[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                // lanes without an entry load nothing (every workgroup pointing
                // its idle lanes at one shared word made that word's cache
                // line a hot spot); this wave has no weight ring to pace
                const uint32_t i = beg[t] + (uint32_t)lane;
                e[t] = make_uint2(0u, 0u);
                if (i < end[t]) e[t] = ent[i];
            }
            // 3. per round of TB tiles: the x values of their entries, then
            // per tile the staged walk and the two sums of each output
#pragma unroll
            for (int t0 = 0; t0 < T; t0 += TB) {
                uint16_t xv[TB][MR];
                int cl_row[TB];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int t = t0 + tb < T ? t0 + tb : T - 1;
                    const bool has = beg[t] + (uint32_t)lane < end[t];
                    const uint32_t kk = e[t].x & 0xFFFFFFu;
                    const int grp = (int)(kk >> 7);
                    cl_row[tb] = has && grp >= g0 && grp < g0 + gn ? (int)(e[t].x >> 24) : -1;
                    const uint16_t* px = g.x + kk;
#pragma unroll
                    for (int m = 0; m < MR; ++m) xv[tb][m] = 0;
                    if (cl_row[tb] >= 0) {
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            if (m < g.M) xv[tb][m] = *px;
                            px += m + 1 < g.M ? g.ldx : 0;   // stays on the last row of x
                        }
                    }
                }
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int t = t0 + tb;
                    if (t >= T) break;
                    float* orig = reinterpret_cast<float*>(area + 256);
                    float* clamp = reinterpret_cast<float*>(area + 512);
                    uint16_t* xs = reinterpret_cast<uint16_t*>(area + 768);
                    const int c = cl_row[tb];
                    orig[lane] = c >= 0 ? bf16_to_f32(e[t].y & 0xFFFFu) : 0.f;
                    clamp[lane] = c >= 0 ? bf16_to_f32(F::clamp_word(e[t].y)) : 0.f;
#pragma unroll
                    for (int m = 0; m < MR; ++m)
                        xs[m * 64 + lane] = (uint16_t)(c >= 0 && m < g.M ? xv[tb][m] : 0u);
                    float cm[MR], cp[MR];
#pragma unroll
                    for (int m = 0; m < MR; ++m) cm[m] = cp[m] = 0.f;
                    auto acc = [&](float o, float cl, auto xs_of) {
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            const float xm = xs_of(m);
                            cm[m] = fmaf(xm, cl, cm[m]);
                            cp[m] = fmaf(xm, o, cp[m]);
                        }
                    };
                    exc_walk(lane, col, area, c, acc);
                    // more than 64 entries in this tile's slice: the rest in
                    // batches with their own loads
                    if (end[t] - beg[t] > 64u)
                        exc_corrections<F, MR>(g, tbase + t, g0, gn, lane, col, area, 0, acc,
                                               (int64_t)beg[t] + 64, (int64_t)end[t]);
                    if (q == 0) {
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            exc_corr[((t * 16 + col) * MR + m) * 2] = cm[m];
                            exc_corr[((t * 16 + col) * MR + m) * 2 + 1] = cp[m];
                        }
                    }
                }
            }
            __syncthreads();   // with the owners' K-wave reduction (or its stand-in)
            if (gridDim.y > 2) {
                __syncthreads();   // the two barriers of split_finish
                __syncthreads();
            }
            return;
        }
    }

    constexpr int kXRows = XD ? (MFMA ? kMT : MR) : 1;  // x registers per slot
    constexpr int kXBlocks = MFMA ? 4 : 1;
    struct Slot {
        Raw w[R];
        uint4 x[kXRows][kXBlocks];
    };
    Slot ring[D];
    // Meta bytes (GEMV): the fetch of ring slot d with d % MB == 0 loads them
    // for the MB slots d .. d + MB - 1 at once -- quarter q of the wave takes
    // the group of slot d + q % MB -- and compute() passes each slot its byte
    // with one cross-lane move, so a wave issues one meta load per MB groups
    // instead of one per group (QKV M = 1: 10.8 -> 10.4 us; O 9.2 -> 8.7 us).
    // d is a constant after unrolling.  The MFMA kernels load the byte with
    // each group (MB = 1): there the cross-lane moves compete with the LDS
    // reads of x and made the x-staged path 2-6% slower.
    constexpr int MB = MFMA ? 1 : (D < 4 ? D : 4);
    uint32_t meta_cur[R];   // the meta block of the slots being computed
    auto fetch = [&](int j, Slot& dst, int d) {
        const int j0 = j;
        j = j < Jlast ? j : Jlast;
        int grp = g0 + kw + j * KW;
        grp = grp < glast ? grp : glast;   // only when this wave has no group at all
#pragma unroll
        for (int r = 0; r < R; ++r) F::load(wbase[r], grp, lane, dst.w[r]);
        if constexpr (F::kHasMeta) {
            if (d % MB == 0) {
                int jm = j0 + q % MB;
                jm = jm < Jlast ? jm : Jlast;
                int gm = g0 + kw + jm * KW;
                gm = gm < glast ? gm : glast;
#pragma unroll
                for (int r = 0; r < R; ++r) dst.w[r].beta = F::load_meta(wbase[r], gm, lane);
            }
        }
        if constexpr (XD && MFMA) {
#pragma unroll
            for (int i = 0; i < kXRows; ++i) {
                const int m = 16 * i + col;
                const int mc = m < g.M ? m : g.M - 1;   // rows past M: valid address, unused
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    dst.x[i][b] = *reinterpret_cast<const uint4*>(
                        g.x + (int64_t)mc * g.ldx + 128 * grp + 32 * b + 8 * q);
            }
        } else if constexpr (XD) {
            // GEMV: the group's 128 x values of a row are 16 pieces of 8;
            // quad position p = col & 3 of quarter q loads piece 4 p + q, the
            // piece block p needs in quarter q (broadcast in compute()).
#pragma unroll
            for (int m = 0; m < kXRows; ++m)
                dst.x[m][0] = *reinterpret_cast<const uint4*>(
                    g.x + (int64_t)m * g.ldx + 128 * grp + 8 * (4 * (col & 3) + q));
        }
    };

    float gacc[MFMA ? 1 : R][MFMA ? 1 : MR];
    f32x4_t macc[MFMA ? R : 1][MFMA ? kMT : 1];
    if constexpr (MFMA) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < kMT; ++i) macc[r][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MR; ++m) gacc[r][m] = 0.f;
    }

    auto compute = [&](const Slot& slot, int j, int d) {
        Raw rr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            rr[r] = slot.w[r];
            if constexpr (F::kHasMeta) {
                if (d % MB == 0) meta_cur[r] = slot.w[r].beta;   // before the slot is refilled
                rr[r].beta = MB == 1 ? meta_cur[r] : (uint32_t)__shfl((int)meta_cur[r], col + 16 * (d % MB));
            }
        }
        const uint4* xb = lds + (CHUNKED ? (c & 1) * kBuf : 0);
        const int grp = g0 + kw + j * KW;
        // unit of (block b) = (128 grp + 32 b + 8 q) / 8, relative to the
        // slice and the chunk
        const int u0 = 16 * (grp - g0) - c * (KC / 8) + q;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (MFMA) {
                bf16x8_t a[kMT];
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt) {
                    if constexpr (XD)
                        a[mt] = __builtin_bit_cast(bf16x8_t, slot.x[mt][b]);
                    else
                        a[mt] = __builtin_bit_cast(bf16x8_t,
                                                   xb[XLayout::phys(16 * mt + col, u0 + 4 * b, units_per_row)]);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    uint32_t wv[4];
                    F::block(rr[r], b, wv);
                    const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3]));
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
                        macc[r][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], bw, macc[r][mt], 0, 0, 0);
                }
            } else {
                uint4 xv[MR];
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if constexpr (XD)
                        xv[m] = quad_bcast(slot.x[m][0], b);
                    else
                        xv[m] = xb[XLayout::phys(m, u0 + 4 * b, units_per_row)];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    uint32_t wv[4];
                    F::block(rr[r], b, wv);
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        float a = gacc[r][m];
                        a = dot2(wv[0], xv[m].x, a);
                        a = dot2(wv[1], xv[m].y, a);
                        a = dot2(wv[2], xv[m].z, a);
                        a = dot2(wv[3], xv[m].w, a);
                        gacc[r][m] = a;
                    }
                }
            }
        }
    };

    // Run after the refill of the group's ring slot has been issued (the
    // corrections need neither the slot nor memory), so they do not delay it.
    auto correct = [&](int j) {
        // In-loop corrections of this group, in list order: for the lanes of
        // the entry's row, acc = (acc - x * clamp) + x * original on the four
        // rows of each 16-row tile they hold (a one-hot x row still returns
        // the original word exactly).
        if constexpr (kInLoop) {
            {
                const int grp = g0 + kw + j * KW;
                const uint16_t* xb16 = reinterpret_cast<const uint16_t*>(lds + (CHUNKED ? (c & 1) * kBuf : 0));
                const int64_t k0 = kbase + (CHUNKED ? (int64_t)c * KC : 0);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    uint64_t mask = __ballot(exc_grp[r] == grp);
                    while (mask != 0) {
                        const int t = __ffsll((unsigned long long)mask) - 1;
                        mask &= mask - 1;
                        const uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)exc_pre[r].x, t);
                        const uint32_t val = (uint32_t)__builtin_amdgcn_readlane((int)exc_pre[r].y, t);
                        if (col == (int)(pos >> 24)) {
                            const int kr = (int)((int64_t)(pos & 0xFFFFFFu) - k0);
                            const float o = bf16_to_f32(val & 0xFFFFu);
                            const float cl = bf16_to_f32(F::clamp_word(val));
#pragma unroll
                            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                                for (int e4 = 0; e4 < 4; ++e4) {
                                    const int m = 16 * mt + 4 * q + e4;
                                    const float xv = bf16_to_f32(
                                        xb16[XLayout::phys(m, kr >> 3, units_per_row) * 8 + (kr & 7)]);
                                    macc[r][mt][e4] = fmaf(xv, o, fmaf(-xv, cl, macc[r][mt][e4]));
                                }
                        }
                    }
                }
            }
        }
    };

    // Prologue: x first, then the ring, so the barrier waits for x only.
    // Chunked: chunks 0 and 1 are both loaded before the ring is primed, so
    // that on entering the loop -- as after every chunk step -- the loads
    // of the next x chunk are followed by one window of ring loads, and the
    // compiler's wait for them at the first chunk step counts exactly (with
    // chunk 1 loaded after the ring it waited for everything, either here
    // or at every chunk step).
    XChunk<MR, KC, NW * 64> xr;
    XAll<NW * 64> xa;
    if constexpr (CHUNKED) {
        XChunk<MR, KC, NW * 64> x0;
        x0.load(g, kbase);
        xr.load(g, kbase + (int64_t)(nchunks > 1 ? 1 : 0) * KC);
#pragma unroll
        for (int d = 0; d < D; ++d) fetch(d, ring[d], d);
        exc_prefetch();
        x0.template store<FixedLayout<XLayout, KC / 8>>(lds);
    } else {
        if constexpr (!XD) xa.load(g, MR, kbase, units_per_row);
#pragma unroll
        for (int d = 0; d < D; ++d) fetch(d, ring[d], d);
        exc_prefetch();
        if constexpr (!XD) xa.template store<XLayout>(lds);
    }
    if constexpr (!XD) __syncthreads();

    auto store_next = [&]() {
        xr.template store<FixedLayout<XLayout, KC / 8>>(lds + ((c + 1) & 1) * kBuf);
    };
    exc_inloop_ready();
    W12_RING_LOOP(D, CHUNKED, J, L, nchunks, xr, store_next, fetch, compute)

    if constexpr (MFMA) {
        if constexpr (KW > 1) {
            if constexpr (!XD) __syncthreads();  // every wave is done reading x
            f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);
            constexpr int kPer = R * kMT;
            if (kw > 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
                        red[(((kw - 1) * kRowWaves + nw) * 64 + lane) * kPer + r * kMT + mt] = macc[r][mt];
            }
            __syncthreads();
            if (kw == 0) {
                for (int p = 1; p < KW; ++p)
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int mt = 0; mt < kMT; ++mt)
                            macc[r][mt] += red[(((p - 1) * kRowWaves + nw) * 64 + lane) * kPer + r * kMT + mt];
            }
        }
        // D layout of the 16x16 MFMA: lane (col, q) holds rows 4q..4q+3 of
        // column col, i.e. y[m = 16 mt + 4q + e][n = 16 tile + col].  With a
        // split K the values go to this slice's partial sums instead.
        if constexpr (kExcWave) {
            if constexpr (KW == 1) __syncthreads();   // the correction wave's results are in
            if (kw == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = 16 * mt + 4 * q + e;
                            const float* cc = exc_corr + (((nw * R + r) * 16 + col) * MR + m) * 2;
                            macc[r][mt][e] = (macc[r][mt][e] - cc[0]) + cc[1];
                        }
            }
        } else if constexpr (F::kHasExceptions) {
            if (kw == 0 && g.exc_off != nullptr) {
                // above 32 rows x is staged 16 rows at a time (the list is
                // walked once per 16 rows): each output still takes its
                // entries in list order.  After in-loop corrections only the
                // entries past each slice's first 64 are left.
                constexpr int kXR = exc_rows(MFMA, MR);
                uint8_t* area = reinterpret_cast<uint8_t*>(lds) + walk_b + nw * ExcStage<kXR>::kBytes;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (tile0 + r >= ntiles) continue;
                    if (kInLoop && exc_e[r] - exc_b[r] <= 64u) continue;
                    const bool rest = kInLoop;
#pragma unroll
                    for (int mb = 0; mb < 16 * kMT; mb += kXR) {
                        if (mb >= g.M) break;
                        exc_corrections<F, kXR>(g, tile0 + r, g0, gn, lane, col, area, mb,
                                                [&](float orig, float clamp, auto xs) {
#pragma unroll
                            for (int t = 0; t < kXR / 16; ++t)
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int mt = mb / 16 + t;
                                    const float xv = xs(16 * t + 4 * q + e);
                                    macc[r][mt][e] = fmaf(xv, orig, fmaf(-xv, clamp, macc[r][mt][e]));
                                }
                        }, rest ? exc_b[r] + 64 : exc_b[r], exc_e[r], !rest, exc_pre[r]);
                    }
                }
            }
        }
        if (kw == 0) {
            if (MR <= 32 && gridDim.y == 2) {
                // all exchanges of the lane in flight together, then finish
                uint64_t old[R][kMT][4];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int64_t n = (tile0 + r) * 16 + col;
                            const int m = 16 * mt + 4 * q + e;
                            old[r][mt][e] = n < g.N && m < g.M ? pair_publish(g, m, n, macc[r][mt][e]) : 0;
                        }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int64_t n = (tile0 + r) * 16 + col;
                            const int m = 16 * mt + 4 * q + e;
                            if (n < g.N && m < g.M) pair_complete(g, m, n, macc[r][mt][e], old[r][mt][e]);
                        }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t n = (tile0 + r) * 16 + col;
                    if (n >= g.N) continue;
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = 16 * mt + 4 * q + e;
                            if (m < g.M) out_value(g, m, n, macc[r][mt][e]);
                        }
                }
            }
        }
        // 64 and 128 rows: each lane of the last workgroup finishes the
        // outputs it stored
        if constexpr (MR >= 64) {
            if (gridDim.y > 1 && split_arrive(g) && kw == 0) {
                constexpr int kNO = R * kMT * 4;
                auto pos = [&](int i) {
                    const int64_t n = (tile0 + i / (kMT * 4)) * 16 + col;
                    const int m = 16 * (i / 4 % kMT) + 4 * q + i % 4;
                    return OutPos{m, n < g.N && m < g.M, n};
                };
                float v[kNO];
#pragma unroll
                for (int i = 0; i < kNO; ++i) v[i] = macc[i / (kMT * 4)][i / 4 % kMT][i % 4];
                split_sum(g, v, pos);
#pragma unroll
                for (int i = 0; i < kNO; ++i) {
                    const OutPos o = pos(i);
                    if (o.ok) store_y(g, o.m, o.n, v[i]);
                }
            }
        }
    } else {
        // Add the 4 quarter sums of each row (fixed butterfly order).
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float v = gacc[r][m];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                gacc[r][m] = v;
            }
        if constexpr (KW > 1) {
            if constexpr (!XD) __syncthreads();  // every wave is done reading x
            float* red = reinterpret_cast<float*>(lds);
            if (kw > 0 && q == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MR; ++m)
                        red[(((kw - 1) * kRowWaves + nw) * 16 + col) * (R * MR) + r * MR + m] = gacc[r][m];
            }
            __syncthreads();
            if (kw == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        float v = gacc[r][m];
                        for (int p = 1; p < KW; ++p)
                            v += red[(((p - 1) * kRowWaves + nw) * 16 + col) * (R * MR) + r * MR + m];
                        gacc[r][m] = v;
                    }
            }
        }
        if constexpr (kExcWave) {
            if constexpr (KW == 1) __syncthreads();   // the correction wave's results are in
            if (kw == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const float* cc = exc_corr + (((nw * R + r) * 16 + col) * MR + m) * 2;
                        gacc[r][m] = (gacc[r][m] - cc[0]) + cc[1];
                    }
            }
        } else if constexpr (F::kHasExceptions) {
            if (kw == 0 && g.exc_off != nullptr) {
                uint8_t* area = reinterpret_cast<uint8_t*>(lds) + walk_b + nw * ExcStage<MR>::kBytes;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (tile0 + r >= ntiles) continue;
                    exc_corrections<F, MR>(g, tile0 + r, g0, gn, lane, col, area, 0,
                                        [&](float orig, float clamp, auto xs) {
#pragma unroll
                        for (int m = 0; m < MR; ++m) {
                            const float xv = xs(m);
                            gacc[r][m] = fmaf(xv, orig, fmaf(-xv, clamp, gacc[r][m]));
                        }
                    }, exc_b[r], exc_e[r], true, exc_pre[r]);
                }
            }
        }
        // Lane (col, q) stores the outputs m with m % 4 == q.
        if (kw == 0) {
            if (gridDim.y == 2) {
                uint64_t old[R][MR];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int64_t n = (tile0 + r) * 16 + col;
                        old[r][m] = (m & 3) == q && n < g.N && m < g.M ? pair_publish(g, m, n, gacc[r][m]) : 0;
                    }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const int64_t n = (tile0 + r) * 16 + col;
                        if ((m & 3) == q && n < g.N && m < g.M) pair_complete(g, m, n, gacc[r][m], old[r][m]);
                    }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int64_t n = (tile0 + r) * 16 + col;
#pragma unroll
                    for (int m = 0; m < MR; ++m)
                        if ((m & 3) == q && n < g.N && m < g.M) out_value(g, m, n, gacc[r][m]);
                }
            }
        }
    }
    if constexpr (!(MFMA && MR >= 64))
        if (gridDim.y > 2) split_finish<kRowWaves * R, NW * 64>(g);
}

// ---- launch helpers ----------------------------------------------------------------------

template <class F, bool MFMA, int MR, int R, int KW, int D, bool CHUNKED, bool XD, int NW>
hipError_t launch_one(const GemmArgs& a, hipStream_t s) {
    constexpr int kTilesPerWG = (NW / KW) * R;
    const int64_t ntiles = (a.N + 15) / 16;
    const dim3 grid((unsigned)((ntiles + kTilesPerWG - 1) / kTilesPerWG), (unsigned)a.S);
    size_t lds = lds_bytes<MFMA, MR, R, KW, D, CHUNKED, XD, NW>(a.gs);
    constexpr bool kExcWave = F::kExcWave && XD;
    if (kExcWave)
        lds += excwave_lds_bytes<MR, R, KW, NW>();
    else if (F::kHasExceptions && a.exc_off != nullptr) {
        size_t extra;
        (void)walk_base<MFMA, MR, R, KW, D, CHUNKED, XD, NW>(a.gs, &extra);
        lds += extra;
    }
    hipLaunchKernelGGL((gemm_kernel<F, MFMA, MR, R, KW, D, CHUNKED, XD, NW>), grid,
                       dim3(NW * 64 + (kExcWave ? 64 : 0)), lds, s, a);
    return hipGetLastError();
}

// Direct x is built when the ring fits about 192 VGPRs (larger rings spill):
// per slot 16 registers per weight tile, plus 4 per x row (GEMV, up to
// M = 4) or 16 per 16-row A tile (MFMA).
__host__ __device__ constexpr bool xd_ok(bool mfma, int mr, int r, int d) {
    return mfma ? d * 16 * (r + mr / 16) <= 192 : (mr <= 4 && d * (16 * r + 4 * mr) <= 192);
}

template <class F, bool MFMA, int MR, int R, int KW, int D, int NW = 4>
hipError_t launch_ch(const GemmArgs& a, const Tiling& t, hipStream_t s) {
    if (t.xdirect) {
        if constexpr (NW == 4 && xd_ok(MFMA, MR, R, D))
            return launch_one<F, MFMA, MR, R, KW, D, false, true, NW>(a, s);
        return hipErrorInvalidValue;
    }
    if (!t.chunked) return launch_one<F, MFMA, MR, R, KW, D, false, false, NW>(a, s);
    if constexpr (chunk_ok(MR, kc_of(MFMA, MR, KW, D), NW))
        return launch_one<F, MFMA, MR, R, KW, D, true, false, NW>(a, s);
    return hipErrorInvalidValue;
}

template <class F, bool MFMA, int MR, int R, int D>
hipError_t launch_kw(const GemmArgs& a, const Tiling& t, hipStream_t s) {
    switch (t.kw) {
        case 1: return launch_ch<F, MFMA, MR, R, 1, D>(a, t, s);
        case 2: return launch_ch<F, MFMA, MR, R, 2, D>(a, t, s);
        case 4: return launch_ch<F, MFMA, MR, R, 4, D>(a, t, s);
        default: return hipErrorInvalidValue;
    }
}

// Eight-wave workgroups (512 threads): the MFMA kernels with x staged in LDS,
// one tile per wave (two at 64 and 128 rows with one K-wave), ring depth 2
// -- eight waves share each x chunk, which halves the x traffic of the
// two-K-wave tiling on long-K weights.
template <class F, int MR>
hipError_t dispatch8(const GemmArgs& a, const Tiling& t, hipStream_t s) {
    if (t.depth != 2 || t.xdirect) return hipErrorInvalidValue;
    if (t.r == 2) {
        // two tiles per wave read each A fragment once for both: 64 and 128
        // rows, one K-wave
        if constexpr (MR >= 64)
            if (t.kw == 1) return launch_ch<F, true, MR, 2, 1, 2, 8>(a, t, s);
        return hipErrorInvalidValue;
    }
    if (t.r != 1) return hipErrorInvalidValue;
    switch (t.kw) {
        case 1: return launch_ch<F, true, MR, 1, 1, 2, 8>(a, t, s);
        case 2: return launch_ch<F, true, MR, 1, 2, 2, 8>(a, t, s);
        case 4: return launch_ch<F, true, MR, 1, 4, 2, 8>(a, t, s);
        case 8: return launch_ch<F, true, MR, 1, 8, 2, 8>(a, t, s);
        default: return hipErrorInvalidValue;
    }
}

// Sixteen-wave workgroups (1024 threads): the same MFMA kernels with x
// staged in LDS, one tile per wave, ring depth 2, 16 and 32 rows -- twice the
// waves (and weight bytes in flight) of an eight-wave workgroup on one x
// copy, for grids with too few row blocks to fill the CUs twice.
template <class F, int MR>
hipError_t dispatch16(const GemmArgs& a, const Tiling& t, hipStream_t s) {
    if (t.depth != 2 || t.xdirect || t.r != 1) return hipErrorInvalidValue;
    switch (t.kw) {
        case 2: return launch_ch<F, true, MR, 1, 2, 2, 16>(a, t, s);
        case 4: return launch_ch<F, true, MR, 1, 4, 2, 16>(a, t, s);
        case 8: return launch_ch<F, true, MR, 1, 8, 2, 16>(a, t, s);
        default: return hipErrorInvalidValue;
    }
}

// (r, depth) pairs that are instantiated: see pair_built() in w12_gemm.hip.
template <class F, bool MFMA, int MR>
hipError_t dispatch(const GemmArgs& a, const Tiling& t, hipStream_t s) {
    if (t.r == 1 && t.depth == 2) return launch_kw<F, MFMA, MR, 1, 2>(a, t, s);
    if (t.r == 1 && t.depth == 4) return launch_kw<F, MFMA, MR, 1, 4>(a, t, s);
    if (t.r == 1 && t.depth == 8) return launch_kw<F, MFMA, MR, 1, 8>(a, t, s);
    if (t.r == 2 && t.depth == 2) return launch_kw<F, MFMA, MR, 2, 2>(a, t, s);
    if (t.r == 2 && t.depth == 4) {
        // with the exception-list code the two-tile ring of depth 4 does not
        // fit the registers: depth 2 (the ring depth only moves loads;
        // products and sums are the same)
        if constexpr (F::kHasExceptions)
            return launch_kw<F, MFMA, MR, 2, 2>(a, t, s);
        else
            return launch_kw<F, MFMA, MR, 2, 4>(a, t, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace kern
}  // namespace w12
