// w12_gemm.hip -- tiling choice, variant names and launch dispatch for the
// decode GEMM kernels (templates in w12_gemm_kernels.hpp, instantiated per
// x height by w12_gemm_inst.hip).
#include <mutex>
#include <string>
#include <unordered_map>

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

int64_t waves_of(const Tiling& t, int64_t N) {
    const int64_t tiles_per_wg = (int64_t)(4 / t.kw) * t.r;
    return ((N + 15) / 16 + tiles_per_wg - 1) / tiles_per_wg * 4;
}

}  // namespace

bool complete_tiling(Tiling& t, int M, int64_t K) {
    if (t.kw != 1 && t.kw != 2 && t.kw != 4) return false;
    if (t.mfma) {
        if (M > 32) return false;
        t.mt = M <= 16 ? 16 : 32;
        if (!pair_built(t.r, t.depth)) return false;
        t.chunked = (int64_t)t.mt * K * 2 > kern::kSingleBytes;
        if (t.chunked && !kern::chunk_ok(t.mt, kern::mfma_kc(t.mt, t.kw, t.depth))) return false;
        if (t.xdirect) return false;
    } else {
        if (M < 1 || M > 8) return false;
        t.mt = M;
        if (!pair_built(t.r, t.depth)) return false;
        if (t.xdirect) {
            if (!kern::xd_ok(false, M, t.r, t.depth)) return false;
            t.chunked = 0;
            return true;
        }
        t.chunked = (int64_t)M * K * 2 > kern::kSingleBytes;
        if (t.chunked && !kern::chunk_ok(M, kern::gemv_kc(M, t.kw, t.depth))) return false;
    }
    return true;
}

// Defaults measured on MI355X over the QKV (7168x5120), gate+up (34816x5120)
// and down (5120x17408) shapes: the GEMV wins up to M = 4 with all four
// waves of a workgroup splitting K; from M = 5 on the MFMA wins (the VALU
// work of eight dot2 rows outweighs the padded MFMA tile).  Splitting K
// helps until there are ~4000 waves; a chunked 32-row x limits KW through
// the LDS budget.
Tiling choose_tiling(int M, int64_t N, int64_t K) {
    Tiling t{};
    t.r = 1;
    t.depth = 2;
    if (M <= 4) {
        t.mfma = 0;
        t.kw = 4;
    } else {
        t.mfma = 1;
        t.kw = 1;
        const int64_t ntiles = (N + 15) / 16;
        if (M <= 16) {
            while (t.kw < 4 && waves_of(t, N) < 4000) t.kw *= 2;
        } else {
            t.kw = ntiles >= 2048 ? 1 : 2;
        }
    }
    // Step down to a built combination (a chunked x buffer must fit LDS).
    while (!complete_tiling(t, M, K)) {
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
    static std::unordered_map<int, std::string> names;
    const int key = (is_w12 << 25) | (t.xdirect << 24) | (t.mfma << 23) | (t.chunked << 22) |
                    (t.mt << 12) | (t.r << 8) | (t.kw << 4) | t.depth;
    std::lock_guard<std::mutex> lock(mu);
    auto it = names.find(key);
    if (it != names.end()) return it->second.c_str();
    std::string n = is_w12 ? "w12_" : "bf16_";
    n += t.mfma ? "mfma_mt" : "gemv_m";
    n += std::to_string(t.mt) + "_r" + std::to_string(t.r) + "_kw" + std::to_string(t.kw) + "_d" +
         std::to_string(t.depth) + (t.xdirect ? "_xdirect" : t.chunked ? "_chunked" : "_single");
    return names.emplace(key, std::move(n)).first->second.c_str();
}

hipError_t launch_gemm(const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s) {
    if (t.mfma) return launch_mfma_mt(t.mt, a, t, is_w12, s);
    return launch_gemv_m(t.mt, a, t, is_w12, s);
}

}  // namespace w12
