// w12_gemm.hip -- tiling choice, variant names and launch dispatch for the
// decode GEMM kernels (templates in w12_gemm_kernels.hpp, instantiated per
// x height by w12_gemm_inst.hip).
#include <mutex>
#include <string>
#include <unordered_set>

#include "w12_gemm_kernels.hpp"
#include "w12_internal.hpp"

namespace w12 {

hipError_t launch_gemv_m1(const GemmArgs&, const Tiling&, bool, hipStream_t);
hipError_t launch_gemv_m2(const GemmArgs&, const Tiling&, bool, hipStream_t);
hipError_t launch_gemv_m3(const GemmArgs&, const Tiling&, bool, hipStream_t);
hipError_t launch_gemv_m4(const GemmArgs&, const Tiling&, bool, hipStream_t);
hipError_t launch_gemv_m5(const GemmArgs&, const Tiling&, bool, hipStream_t);
hipError_t launch_gemv_m6(const GemmArgs&, const Tiling&, bool, hipStream_t);
hipError_t launch_gemv_m7(const GemmArgs&, const Tiling&, bool, hipStream_t);
hipError_t launch_gemv_m8(const GemmArgs&, const Tiling&, bool, hipStream_t);

hipError_t launch_gemv_m(int M, const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s) {
    switch (M) {
        case 1: return launch_gemv_m1(a, t, is_w12, s);
        case 2: return launch_gemv_m2(a, t, is_w12, s);
        case 3: return launch_gemv_m3(a, t, is_w12, s);
        case 4: return launch_gemv_m4(a, t, is_w12, s);
        case 5: return launch_gemv_m5(a, t, is_w12, s);
        case 6: return launch_gemv_m6(a, t, is_w12, s);
        case 7: return launch_gemv_m7(a, t, is_w12, s);
        case 8: return launch_gemv_m8(a, t, is_w12, s);
        default: return hipErrorInvalidValue;
    }
}

namespace {

// (r, depth) pairs that are instantiated (both variants).
bool pair_built(int r, int d) {
    return (r == 1 && (d == 2 || d == 4 || d == 8)) || (r == 2 && (d == 2 || d == 4));
}

int64_t waves_of(const Tiling& t, int64_t N) { return row_blocks(t, N) * 4; }

}  // namespace

int64_t row_blocks(const Tiling& t, int64_t N) {
    const int64_t tiles_per_wg = (int64_t)(4 / t.kw) * t.r;
    return ((N + 15) / 16 + tiles_per_wg - 1) / tiles_per_wg;
}

bool complete_tiling(Tiling& t, int M, int64_t N, int64_t K) {
    if (t.kw != 1 && t.kw != 2 && t.kw != 4) return false;
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
        if (M > 32) return false;
        t.mt = M <= 16 ? 16 : 32;
        if (!pair_built(t.r, t.depth)) return false;
        if (t.xdirect) {
            if (!kern::xd_ok(true, t.mt, t.r, t.depth)) return false;
            t.chunked = 0;
            return true;
        }
        t.chunked = (int64_t)t.mt * width * 2 > kern::kSingleBytes;
        if (t.chunked && !kern::chunk_ok(t.mt, kern::mfma_kc(t.mt, t.kw, t.depth))) return false;
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
        if (t.chunked && !kern::chunk_ok(M, kern::gemv_kc(M, t.kw, t.depth))) return false;
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
// gate+up (34816x5120) and down (5120x17408) shapes at M = 1-32.  M = 1 runs
// the wavefront-reduction GEMV with x read directly (no x barrier), four
// groups in flight per wave, and two K-waves per 16-row tile on weights of
// 256-1024 tiles, four otherwise (QKV 10.9 us against 11.3 us with x staged
// in LDS, O 9.3 against 10.2; gate+up 43.0 us with four K-waves against 46.3
// with two; N = 896: 5.8 us against 7.4), and K is never split across
// workgroups: no split factor 2-16 was faster on any weight measured (N =
// 640-34816, K = 2176-17408; down 24.4 us unsplit against 25.2 in three).  From M = 2 each extra x row costs the GEMV four more dot2 per 8
// weights, and the MFMA, whose cost does not grow until 16 rows, measured
// faster on all shapes (QKV M = 4: 12.9 us against 14.6 us): up to M = 8 it
// reads its A fragments straight from memory with two tiles per wave and
// four K-waves (no x barrier).  So does M = 9-32 on weights of at most 1024
// tiles and 64 groups per row (QKV M = 16: 13.4 us against 15.4 us with x
// in LDS; M = 32: 18.7 against 19.2; O M = 16: 12.7 against 13.7).  On
// larger weights x goes through LDS from M = 9, shared by the waves of a
// workgroup, with two K-waves or, above 16 rows, one when the grid has
// >= 1024 row blocks anyway (gate+up M = 32: 64 us against 69.5 us).
//
// Splitting K across workgroups (the _ws entry points, MFMA only): slices of at
// least 40 groups (5120 weights) keep each workgroup's prologue and
// epilogue small against its stream, up to ~2048 workgroups -- three
// slices on the down shape (M = 16-32: 31-38 us instead of 40-51 us).  The
// LDS path from M = 9 also splits until it has ~480 workgroups, with slices
// of at least 13 groups: its x chunks make few large workgroups slow (O,
// 160 row blocks, three slices: M = 12-24 5-7% faster; QKV, 224 row
// blocks, two slices at M = 24-32; three were 30% slower).
Tiling choose_tiling(int M, int64_t N, int64_t K, bool allow_splitk) {
    Tiling t{};
    t.r = 1;
    t.splitk = 1;
    const int64_t ntiles = (N + 15) / 16;
    if (M == 1) {
        t.mfma = 0;
        t.kw = ntiles >= 256 && ntiles <= 1024 ? 2 : 4;
        t.depth = 4;
        t.xdirect = 1;
    } else if (M <= 8 || (ntiles <= 1024 && K / 128 <= 64)) {
        t.mfma = 1;
        t.r = 2;
        t.kw = 4;
        t.depth = 2;
        t.xdirect = 1;
    } else {
        t.mfma = 1;
        t.kw = 2;
        t.depth = 2;
        if (M > 16 && row_blocks(t, N) >= 1024) t.kw = 1;
    }
    if (allow_splitk && t.mfma) {
        const int64_t G = K / 128;
        const int64_t nb = row_blocks(t, N);
        int64_t s = G / 40;
        const int64_t fill = (2048 + nb - 1) / nb;
        s = s < fill ? s : fill;
        if (t.mfma && !t.xdirect) {
            int64_t s2 = 480 / nb;
            s2 = s2 < G / 13 ? s2 : G / 13;
            s = s > s2 ? s : s2;
        }
        s = s < kMaxSplitK ? s : kMaxSplitK;
        t.splitk = s > 1 ? (int)s : 1;
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

const char* tiling_name(const Tiling& t, bool is_w12) {
    static std::mutex mu;
    static std::unordered_set<std::string> names;  // node-based: c_str() stays valid
    std::string n = is_w12 ? "w12_" : "bf16_";
    n += t.mfma ? "mfma_mt" : "gemv_m";
    n += std::to_string(t.mt) + "_r" + std::to_string(t.r) + "_kw" + std::to_string(t.kw) + "_d" +
         std::to_string(t.depth) + (t.xdirect ? "_xdirect" : t.chunked ? "_chunked" : "_single");
    if (t.splitk > 1) n += "_s" + std::to_string(t.splitk);
    std::lock_guard<std::mutex> lock(mu);
    return names.insert(std::move(n)).first->c_str();
}

hipError_t launch_gemm(const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s) {
    if (t.mfma) return launch_mfma_mt(t.mt, a, t, is_w12, s);
    return launch_gemv_m(t.mt, a, t, is_w12, s);
}

}  // namespace w12
