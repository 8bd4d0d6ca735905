// w12_gemm.hip -- tiling choice, variant names and launch dispatch for the
// decode GEMM kernels (templates in w12_gemm_kernels.hpp, instantiated per
// x height by w12_gemm_inst.hip).
#include <mutex>
#include <string>
#include <unordered_set>

#include "w12_gemm_kernels.hpp"
#include "w12_internal.hpp"

namespace w12 {

hipError_t launch_gemv_m1(const GemmArgs&, const Tiling&, int, hipStream_t);
hipError_t launch_gemv_m2(const GemmArgs&, const Tiling&, int, hipStream_t);
hipError_t launch_gemv_m3(const GemmArgs&, const Tiling&, int, hipStream_t);
hipError_t launch_gemv_m4(const GemmArgs&, const Tiling&, int, hipStream_t);
hipError_t launch_gemv_m5(const GemmArgs&, const Tiling&, int, hipStream_t);
hipError_t launch_gemv_m6(const GemmArgs&, const Tiling&, int, hipStream_t);
hipError_t launch_gemv_m7(const GemmArgs&, const Tiling&, int, hipStream_t);
hipError_t launch_gemv_m8(const GemmArgs&, const Tiling&, int, hipStream_t);

hipError_t launch_gemv_m(int M, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (M) {
        case 1: return launch_gemv_m1(a, t, fetch, s);
        case 2: return launch_gemv_m2(a, t, fetch, s);
        case 3: return launch_gemv_m3(a, t, fetch, s);
        case 4: return launch_gemv_m4(a, t, fetch, s);
        case 5: return launch_gemv_m5(a, t, fetch, s);
        case 6: return launch_gemv_m6(a, t, fetch, s);
        case 7: return launch_gemv_m7(a, t, fetch, s);
        case 8: return launch_gemv_m8(a, t, fetch, s);
        default: return hipErrorInvalidValue;
    }
}

namespace {

// (r, depth) pairs that are instantiated (both variants).
bool pair_built(int r, int d) {
    return (r == 1 && (d == 2 || d == 4 || d == 8)) || (r == 2 && (d == 2 || d == 4));
}

}  // namespace

int64_t row_blocks(const Tiling& t, int64_t N) {
    const int64_t tiles_per_wg = (int64_t)(t.nw / t.kw) * t.r;
    return ((N + 15) / 16 + tiles_per_wg - 1) / tiles_per_wg;
}

bool complete_tiling(Tiling& t, int M, int64_t N, int64_t K) {
    if (t.nw == 0) t.nw = 4;
    if (t.nw != 4 && t.nw != 8 && t.nw != 16) return false;
    if (t.kw != 1 && t.kw != 2 && t.kw != 4 && t.kw != 8) return false;
    if (t.kw > t.nw) return false;
    // eight-wave workgroups: MFMA with x in LDS, depth 2, one tile per wave
    // (two with one K-wave above 32 rows)
    if (t.nw == 8 && (!t.mfma || t.xdirect || t.depth != 2)) return false;
    if (t.nw == 8 && t.r != 1 && !(t.r == 2 && t.kw == 1 && M > 32)) return false;
    // sixteen-wave workgroups: the same, one tile per wave, up to 32 rows,
    // two to eight K-waves
    if (t.nw == 16 && (!t.mfma || t.xdirect || t.depth != 2 || t.r != 1 || M > 32 || t.kw < 2))
        return false;
    if (t.splitk < 1 || t.splitk > kMaxSplitK) return false;
    // Slices of gs groups; a request above the group count gives one group
    // per slice.
    const int64_t G = K / 128;
    const int64_t gs = (G + t.splitk - 1) / t.splitk;
    t.gs = (int)gs;
    t.splitk = (int)((G + gs - 1) / gs);
    if (t.splitk > 1 && row_blocks(t, N) > kMaxSplitRowBlocks) return false;
    const int64_t width = gs * 128;  // x columns one workgroup reads
    if (t.mfma) {
        if (M > 128) return false;
        t.mt = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
        // 64 and 128 rows: eight-wave workgroups with x in LDS only
        if (t.mt > 32 && t.nw != 8) return false;
        if (!pair_built(t.r, t.depth)) return false;
        if (t.xdirect) {
            if (!kern::xd_ok(true, t.mt, t.r, t.depth)) return false;
            t.chunked = 0;
            return true;
        }
        t.chunked = (int64_t)t.mt * width * 2 > kern::kSingleBytes;
        if (t.chunked && !kern::chunk_ok(t.mt, kern::mfma_kc(t.mt, t.kw, t.depth), t.nw)) return false;
    } else {
        if (M < 1 || M > 8) return false;
        t.mt = M;
        if (!pair_built(t.r, t.depth)) return false;
        if (t.xdirect) {
            if (!kern::xd_ok(false, M, t.r, t.depth)) return false;
            t.chunked = 0;
            return true;
        }
        t.chunked = (int64_t)M * width * 2 > kern::kSingleBytes;
        if (t.chunked && !kern::chunk_ok(M, kern::gemv_kc(M, t.kw, t.depth), t.nw)) return false;
    }
    return true;
}

size_t workspace_bytes(const Tiling& t, int M, int64_t N) {
    if (t.splitk <= 1) return 0;
    const int64_t np = (N + 15) / 16 * 16;
    return (size_t)(kCounterBytes + (int64_t)t.splitk * M * np * 4);
}

void bind_split(GemmArgs& a, const Tiling& t, void* ws) {
    a.S = t.splitk;
    a.gs = t.gs;
    a.cnt = nullptr;
    a.ws = nullptr;
    if (t.splitk > 1) {
        a.cnt = static_cast<uint32_t*>(ws);
        a.ws = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
    }
}

// Defaults measured on MI355X over the QKV (7168x5120), O (5120x5120),
// gate+up (34816x5120) and down (5120x17408) shapes and N = 1024-2048 at
// K = 5120, M = 1-32.
//
// M = 1 runs the wavefront-reduction GEMV with x read directly (no x
// barrier), four groups in flight per wave, and two K-waves per 16-row tile
// on weights of 256-1024 tiles, four otherwise (QKV 10.9 us against 11.3 us
// with x staged in LDS, O 9.3 against 10.2; gate+up 43.0 us with four
// K-waves against 46.3 with two; N = 896: 5.8 us against 7.4), and K is
// never split across workgroups: no split factor 2-16 was faster on any
// weight measured (down 24.4 us unsplit against 25.2 in three).
//
// M = 2-8: each extra x row costs the GEMV four more dot2 per 8 weights,
// while the MFMA's cost does not grow until 16 rows (QKV M = 4: 12.9 us
// against 14.6 us).  It reads its A fragments straight from memory, four
// K-waves (no x barrier); x staged in LDS was 2-7% slower on QKV and
// gate+up.  So is M = 9-12 on weights of 385-1024 tiles and at most 64
// groups per row (QKV M = 9: 12.1 us against 12.8), and M <= 32 on weights
// of at most 256 tiles (N = 512-4096, K = 5120: 13-48% faster than any
// other tiling), where K is split from M = 9 into up to 256 / tiles slices
// of >= 10 groups.  Two tiles per wave at 257-512 tiles (at most 256
// workgroups; O M = 4: 10.2 us against 10.9 with one), one otherwise, and
// two again above 512 tiles from M = 7 (gate+up M = 4: 43.3 us with one
// against 45.0; M = 8: 46.6 with two against 48.1).
//
// Otherwise from M = 9 x is staged in LDS and shared by eight waves of a
// 512-thread workgroup, with four K-waves (two tiles per workgroup) when K
// is not split and M <= 16, two K-waves (four tiles) otherwise -- O M = 16:
// 11.4 us against 12.7 us with x read directly; N = 1024-2048: 4-14%
// faster; down M = 16 split in three: 27.4 us against 30.1 us with
// 256-thread workgroups; gate+up M = 32: 58.2 against 60.6.  Above 16 rows
// a weight of fewer than 128 row blocks that K does not split keeps four
// K-waves, its 128 KB x double buffer included (down M = 24: 41.3 us
// against 46.5 with 256 threads).
//
// M = 33-128: x padded to 64 or 128 rows, in LDS, eight waves.  With a
// workspace, on weights of >= 256 tiles: one K-wave (eight tiles per
// workgroup, x staged once for all of them) and K split into as many slices
// of >= 10 groups as fill 256 workgroups -- QKV and O four slices, down six
// (QKV M = 64: 21.1 us against 22.9 with two K-waves in two slices; M = 128:
// 30.6 against 41.1 in two slices; down M = 128: 55.5 against 80.1 in three).
// Otherwise two K-waves (64 rows) or one (128 rows: a 128 KB double buffer
// holds 256 columns); a weight of >= 512 row blocks that K does not split
// takes one K-wave and two tiles per wave, which read each A fragment from
// LDS once for both (gate+up M = 64: 74.2 us against 80.5 with one tile;
// M = 128: 93.6 against 130.7; on smaller grids the halved workgroup count
// loses: QKV M = 128 87.7 against 48.3).
//
// Splitting K across workgroups (the _ws entry points, MFMA only): slices of
// at least 40 groups (5120 weights) keep each workgroup's prologue and
// epilogue small against its stream, up to ~2048 workgroups -- three slices
// on the down shape.  Above 16 rows the LDS path also takes the fewest
// slices that give it >= 1280 waves, with slices of at least 13 groups, but
// at most two: those meet in one atomic exchange per output (QKV M = 32: 16.9
// us against 19.5 unsplit; O: 15.3 against 15.8 in three; 4352 x 5120 at
// M = 32: 13.1 against 14.7 in three).
//
// Small shapes (measured per tensor-parallel shard, W12 and BF16 alike):
// at most 128 tiles with 20-64 groups take two K slices at every M (896 x
// 5120 at M = 2: 5.2 us against 6.3 unsplit); rows of <= 8 groups take two
// K-waves per tile up to 32 rows (5120 x 640 at M = 8: 4.1 against 4.8; at
// M = 32: 5.9 against 6.0), and so do rows of 10-20 groups on 257-512 tiles
// at 9-12 rows (5120 x 2176 at M = 9: 6.7 against 7.5 with x in LDS);
// x is staged in LDS from 4 rows on 257-384 tiles with >= 40 groups (5120
// x 5120 at M = 4: 10.1 against 10.4; 5120 x 17408 at M = 4: 24.9 against
// 25.3), from 7 rows above 1024 tiles (34816 x 5120 at M = 8: 45.9 against
// 47.4) and from 11 rows on 385-1024 tiles (7168 x 5120 at M = 12: 12.5
// against 12.9).
Tiling choose_tiling(int M, int64_t N, int64_t K, bool allow_splitk) {
    Tiling t{};
    t.r = 1;
    t.splitk = 1;
    t.nw = 4;
    const int64_t ntiles = (N + 15) / 16;
    const int64_t G = K / 128;
    // small weights (at most 128 tiles, e.g. one GPU's QKV share under 8-way
    // tensor parallelism, N = 896) with 20-64 groups per row: K split in two
    // at every M -- the two slices meet in one atomic exchange per output,
    // and the grid doubles
    const bool small_pair = ntiles <= 128 && G >= 20 && G <= 64;
    // x staged in LDS already below 9 rows: from 4 rows on 257-384 tiles with
    // >= 40 groups (O, down), from 7 rows above 1024 tiles (gate+up)
    const bool lds_small_m = (M >= 4 && ntiles > 256 && ntiles <= 384 && G >= 40) ||
                             (M >= 7 && ntiles > 1024);
    if (M == 1) {
        t.mfma = 0;
        t.kw = ntiles >= 256 && ntiles <= 1024 ? 2 : 4;
        // two groups in flight per wave above 1024 tiles: with 2 000+
        // workgroups several share each CU and keep it fed (gate+up 41.7
        // against 42.3 us with four)
        t.depth = small_pair || ntiles > 1024 ? 2 : 4;
        t.xdirect = 1;
    } else if ((M <= 8 && !lds_small_m) || (M <= 32 && G <= 8) ||
               (M <= 12 && G >= 10 && G <= 20 && ntiles > 256 && ntiles <= 512) ||
               (M <= 32 && (ntiles <= 256 || (M <= 10 && ntiles > 384 && ntiles <= 1024 && G <= 64)))) {
        t.mfma = 1;
        t.r = ntiles <= 256 || (ntiles > 512 && M <= 6) || G <= 20 ? 1 : 2;
        // rows of at most 8 groups (one GPU's O share under 8-way tensor
        // parallelism, K = 640), and of 10-20 groups on 257-512 tiles from
        // 9 rows (the down share, K = 2176): two K-waves per tile
        t.kw = G <= 8 || (M > 8 && G <= 20) ? 2 : 4;
        t.depth = 2;
        t.xdirect = 1;
    } else {
        t.mfma = 1;
        t.nw = 8;
        t.depth = 2;
        t.kw = 2;
    }
    const int64_t nb = row_blocks(t, N);
    if (allow_splitk && small_pair && t.xdirect && t.r == 1) {
        t.splitk = 2;
    } else if (allow_splitk && t.mfma && t.xdirect && t.r == 1 && M <= 8 && ntiles > 256 &&
               ntiles <= 512 && G >= 10 && G <= 20) {
        // short rows on a mid-size grid (one GPU's down share under 8-way
        // tensor parallelism, 5120 x 2176): two slices
        t.splitk = 2;
    } else if (allow_splitk && t.mfma) {
        int64_t s = G / 40;
        const int64_t fill = (2048 + nb - 1) / nb;
        s = s < fill ? s : fill;
        if (!t.xdirect && M > 16) {
            const int64_t waves = nb * t.nw;
            int64_t s2 = (1280 + waves - 1) / waves;
            s2 = s2 < G / 13 ? s2 : G / 13;
            // up to 32 rows two slices meet in one atomic exchange, more in
            // a counted reduction: at most two for this purpose
            if (M <= 32) s2 = s2 < 2 ? s2 : 2;
            s = s > s2 ? s : s2;
        }
        if (t.xdirect && t.r == 1 && M > 8) {
            int64_t s2 = 256 / ntiles;
            s2 = s2 < G / 10 ? s2 : G / 10;
            s = s > s2 ? s : s2;
        }
        s = s < kMaxSplitK ? s : kMaxSplitK;
        t.splitk = s > 1 ? (int)s : 1;
        // above 32 rows, on weights of >= 256 tiles: one K-wave (eight tiles
        // per workgroup, x staged once for all eight) and as many slices of
        // >= 10 groups as fill 256 workgroups
        if (M > 32 && ntiles >= 256) {
            const int64_t nb1 = (ntiles + 7) / 8;
            int64_t s1 = 256 / nb1;
            s1 = s1 < G / 10 ? s1 : G / 10;
            if (s1 >= 2) {
                t.kw = 1;
                t.splitk = (int)(s1 < kMaxSplitK ? s1 : kMaxSplitK);
            }
        }
    }
    // 9-32 rows on long rows (>= 100 groups) of 257-512 tiles with K split
    // (the down projection, 5120 x 17408, in three slices): sixteen waves
    // with four K-waves per workgroup -- the same four tiles and x copy,
    // twice the weight loads in flight (M = 9: 25.7 us against 26.5; M = 32:
    // 30.4 against 30.9)
    if (t.nw == 8 && t.splitk > 1 && M > 8 && M <= 32 && G >= 100 && ntiles > 256 &&
        ntiles <= 512) {
        t.nw = 16;
        t.kw = 4;
    }
    if (t.nw == 8 && t.splitk == 1 && (M <= 16 || nb < 128)) t.kw = 4;
    // above 32 rows a grid of >= 512 row blocks unsplit keeps eight tiles per
    // workgroup (one K-wave each): x is staged once for eight tiles, and two
    // tiles per wave share each A fragment
    if (t.nw == 8 && t.splitk == 1 && M > 32 && nb >= 512) {
        t.kw = 1;
        t.r = 2;
    }
    // Step down to a built combination (a chunked x buffer must fit LDS).
    while (!complete_tiling(t, M, N, K)) {
        if (t.depth > 2)
            t.depth /= 2;
        else if (t.kw > 1)
            t.kw /= 2;
        else
            break;
    }
    return t;
}

const char* tiling_name(const Tiling& t, int fetch) {
    static std::mutex mu;
    static std::unordered_set<std::string> names;  // node-based: c_str() stays valid
    std::string n = fetch == kFetchW12 ? "w12_" : fetch == kFetchW12B ? "w12b_" : "bf16_";
    n += t.mfma ? "mfma_mt" : "gemv_m";
    n += std::to_string(t.mt) + "_r" + std::to_string(t.r) + "_kw" + std::to_string(t.kw) + "_d" +
         std::to_string(t.depth) + (t.xdirect ? "_xdirect" : t.chunked ? "_chunked" : "_single");
    if (t.nw == 8) n += "_w8";
    if (t.nw == 16) n += "_w16";
    if (t.splitk > 1) n += "_s" + std::to_string(t.splitk);
    std::lock_guard<std::mutex> lock(mu);
    return names.insert(std::move(n)).first->c_str();
}

hipError_t launch_gemm(const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    if (t.mfma && t.mt > 32) return launch_mfma8_big_mt(t.mt, a, t, fetch, s);
    if (t.mfma)
        return t.nw == 16  ? launch_mfma16_mt(t.mt, a, t, fetch, s)
               : t.nw == 8 ? launch_mfma8_mt(t.mt, a, t, fetch, s)
                           : launch_mfma_mt(t.mt, a, t, fetch, s);
    return launch_gemv_m(t.mt, a, t, fetch, s);
}

}  // namespace w12
