// w12_internal.hpp -- launch helpers shared by the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

// Bit allocations of the planes: W12-v1 (3-bit offset of E[7:1] from an
// even base, low byte verbatim) and W12-b (4-bit offset of E from a base of
// any value).
enum Format { kFmtV1 = 0, kFmtB = 1 };
// Weight fetch of a GEMM launch: the BF16 control or a W12 container.
enum Fetch { kFetchBF16 = 0, kFetchW12 = 1, kFetchW12B = 2 };

// Everything a GEMM launch needs.  Exactly one of {p0,p1,p2,meta} (W12
// container) or w (plain BF16) is used, by the weight-fetch policy.
struct GemmArgs {
    const uint16_t* x;
    int64_t ldx;
    int M;
    const uint8_t* p0;
    const uint8_t* p1;
    const uint8_t* p2;
    const uint8_t* meta;
    // Optional exception list of the container (both NULL when it has none):
    // block (tile T, group g) owns entries exc_off[T * G + g] ..
    // exc_off[T * G + g + 1] - 1 (G = K / 128), two words each.
    const uint32_t* exc_off;
    const uint32_t* exc_ent;
    const uint16_t* w;
    int64_t N;
    int64_t K;
    void* y;
    int64_t ldy;
    int y_f32;
    // K split across workgroups (grid y): slice s holds groups
    // [s * gs, min(G, (s + 1) * gs)).  With S = 2 (up to 32 x rows) the two
    // workgroups of a row block meet in 64-bit slots ws64[m][Np] (one atomic
    // exchange per output; the second adds slice 0 + slice 1).  With S > 2
    // every workgroup writes its fp32 partial sums to ws[s][m][Np] and the
    // last of the S workgroups of a row block (counted in cnt[block]) adds
    // them in slice order and writes y.  Every launch leaves the counters at
    // zero and no slot tagged.
    int S;
    int gs;
    float* ws;
    uint32_t* cnt;
};

// Tiling of one GEMM launch.
//   mfma    = 0: GEMV (v_dot2c_f32_bf16); 1: MFMA 16x16x32 bf16.
//   r       = 16-row weight tiles per wave (1 or 2).
//   mt      = GEMV: M (1..8); MFMA: x rows padded to 16, 32, 64 or 128 (64
//             and 128 with nw = 8 only).
//   kw      = waves of a workgroup that split K between them (1, 2, 4; 8
//             with nw = 8).
//   depth   = 32-weight slices each lane keeps in flight (2, 4 or 8).
//   xdirect = 1: x is read by each lane with its weights instead of being
//             staged in LDS (GEMV up to M = 4, MFMA; within a register
//             budget, see kern::xd_ok).
//   splitk  = workgroups that split K between them (1 = none); completed to
//             the number of non-empty slices of gs groups each.
//   chunked = 0 if the x columns of a K slice are staged in LDS at once, 1 if
//             they are streamed through LDS in double-buffered chunks (set
//             from the shape).
//   nw      = waves per workgroup: 4 (256 threads), 8 (512 threads; MFMA
//             with x in LDS, r = 1, depth = 2 only) or 16 (1024 threads;
//             the same, 16 and 32 rows, kw 2-8).
struct Tiling {
    int mfma;
    int mt;
    int r;
    int kw;
    int depth;
    int xdirect;
    int splitk;
    int gs;
    int chunked;
    int nw;
};

constexpr int kMaxSplitK = 64;
// A split-K workspace starts with a fixed counter area, so that the counters
// of any launch lie outside the partial sums of any other launch and stay
// zero between launches of different shapes; split K therefore needs at most
// kMaxSplitRowBlocks workgroups along N.
constexpr int64_t kCounterBytes = 65536;
constexpr int64_t kMaxSplitRowBlocks = kCounterBytes / 4;

// Pick the tiling used by w12_gemm / bf16_gemm for this shape; split-K
// tilings (which need a workspace) only if allow_splitk.
Tiling choose_tiling(int M, int64_t N, int64_t K, bool allow_splitk);
// Complete a caller-given tiling (mt, splitk, gs, chunked) for this shape;
// false if the combination is not built (or splits K over more than
// kMaxSplitRowBlocks row blocks).
bool complete_tiling(Tiling& t, int M, int64_t N, int64_t K);
const char* tiling_name(const Tiling& t, int fetch);
// Workgroups along N (grid x) of a launch with this tiling.
int64_t row_blocks(const Tiling& t, int64_t N);
// Workspace a completed tiling needs: 0 without split-K, else the counter
// area (kCounterBytes) followed by S * M * Np fp32 partials.
size_t workspace_bytes(const Tiling& t, int M, int64_t N);
// Point the split-K fields of `a` at `ws` (which holds workspace_bytes).
void bind_split(GemmArgs& a, const Tiling& t, void* ws);

hipError_t launch_gemm(const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s);
// Per-M (GEMV) and per-MT (MFMA) launchers, one object file each.
hipError_t launch_gemv_m(int M, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s);
hipError_t launch_mfma_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s);
hipError_t launch_mfma8_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s);
hipError_t launch_mfma16_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s);
hipError_t launch_mfma8_big_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch,
                               hipStream_t s);
hipError_t launch_pack(int fmt, const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1,
                       void* p2, uint8_t* meta, uint32_t* bad, hipStream_t s);
hipError_t launch_unpack(int fmt, const void* p0, const void* p1, const void* p2,
                         const uint8_t* meta, int64_t N, int64_t K, uint16_t* w,
                         hipStream_t s);
// Exception list: count per block into ws (nblocks words), scan, write the
// tile offsets, the total and at most `capacity` entries.
hipError_t launch_exceptions(int fmt, const uint16_t* w, int64_t N, int64_t K, uint32_t* ws,
                             uint32_t* offsets, uint32_t* entries, int64_t capacity,
                             uint32_t* total, hipStream_t s);
// Write the exceptions' original words over an unpacked [N, K] weight.
hipError_t launch_apply_exceptions(const uint32_t* offsets, const uint32_t* entries, int64_t N,
                                   int64_t K, uint16_t* w, hipStream_t s);
hipError_t launch_bf16_tile(const uint16_t* w, int64_t N, int64_t K, uint16_t* out, hipStream_t s);

}  // namespace w12
