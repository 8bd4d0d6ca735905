// w12_api.hip -- the C ABI declared in include/w12.h: host-side argument
// checks, tiling choice, and launches on the caller's stream.  Nothing here
// allocates or synchronises.  Split-K launches keep their counters in the
// caller's workspace -- except w12_gemm_noalloc, which uses the library's
// own fixed device array `scratch` (defined below with its set-up), for
// callers that cannot allocate.
#include <stdint.h>

#include <mutex>

#include "../../include/w12.h"
#include "w12_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest element count a launch accepts: keeps every grid below 2^31 blocks
// and every byte offset far inside int64.  K below 2^24 keeps the in-tile
// offsets the kernels form in 32 bits (group * 1024 + lane * 16, 128 * group).
constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int64_t kMaxK = (int64_t)1 << 24;

int check_weight_shape(int64_t N, int64_t K) {
    if (N < 1 || K < W12_GROUP || K % W12_GROUP != 0 || K >= kMaxK) return W12_ERR_SHAPE;
    if (N + W12_TILE_ROWS > kMaxElems / K) return W12_ERR_SHAPE;
    return W12_OK;
}

int check_gemm_common(const uint16_t* x, int64_t M, int64_t ldx, int64_t N, int64_t K, void* y,
                      int64_t ldy, int y_type) {
    if (x == nullptr || y == nullptr) return W12_ERR_NULL;
    if (int rc = check_weight_shape(N, K)) return rc;
    if (M < 1) return W12_ERR_SHAPE;
    if (M > W12_MAX_M) return W12_ERR_UNSUPPORTED;
    if (ldx < K || ldy < N) return W12_ERR_SHAPE;
    if (y_type != W12_OUT_BF16 && y_type != W12_OUT_F32) return W12_ERR_DTYPE;
    if (!aligned16(x) || ldx % 8 != 0) return W12_ERR_ALIGN;
    const uintptr_t ya = reinterpret_cast<uintptr_t>(y);
    if (y_type == W12_OUT_F32 ? (ya & 3u) : (ya & 1u)) return W12_ERR_ALIGN;
    return W12_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? W12_OK : W12_ERR_HIP; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Exception lists index k in 24 bits and elements in 32 bits.
constexpr int64_t kExcMaxK = (int64_t)1 << 24;
constexpr int64_t kExcMaxElems = (int64_t)1 << 32;

bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Both list pointers or neither; 8-byte aligned (the GEMMs read entries and
// offset pairs as 8-byte words); a shape the list can index.
int check_exceptions(const uint32_t* off, const uint32_t* ent, int64_t N, int64_t K) {
    if ((off == nullptr) != (ent == nullptr)) return W12_ERR_NULL;
    if (off == nullptr) return W12_OK;
    if (!aligned8(off) || !aligned8(ent)) return W12_ERR_ALIGN;
    if (K >= kExcMaxK || (N + W12_TILE_ROWS) * K >= kExcMaxElems) return W12_ERR_SHAPE;
    return W12_OK;
}

w12::GemmArgs make_args(const uint16_t* x, int64_t M, int64_t ldx, int64_t N, int64_t K, void* y,
                        int64_t ldy, int y_type) {
    w12::GemmArgs a{};
    a.x = x;
    a.ldx = ldx;
    a.M = (int)M;
    a.N = N;
    a.K = K;
    a.y = y;
    a.ldy = ldy;
    a.y_f32 = y_type == W12_OUT_F32;
    return a;
}

}  // namespace

extern "C" {

int w12_abi_version(void) { return W12_ABI_VERSION; }

const char* w12_status_string(int status) {
    switch (status) {
        case W12_OK: return "ok";
        case W12_ERR_NULL: return "a required pointer is NULL";
        case W12_ERR_SHAPE: return "bad shape (need N >= 1, K a positive multiple of 128, M >= 1, ldx >= K, ldy >= N)";
        case W12_ERR_ALIGN: return "misaligned pointer or leading dimension (16-byte tensors, ldx % 8 == 0)";
        case W12_ERR_DTYPE: return "unknown output type";
        case W12_ERR_UNSUPPORTED: return "unsupported size or tiling (M > 128, or a tiling that is not built for this shape)";
        case W12_ERR_HIP: return "HIP launch failed";
        case W12_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned for this split-K tiling";
        case W12_ERR_SCRATCH: return "the split-K partial sums of this shape exceed the library's fixed 16 MiB scratch (w12_gemm_noalloc); use w12_gemm_ws with a workspace";
        default: return "unknown status";
    }
}

int64_t w12_padded_rows(int64_t N) { return N < 1 ? 0 : (N + W12_TILE_ROWS - 1) / W12_TILE_ROWS * W12_TILE_ROWS; }

size_t w12_plane_bytes(int64_t N, int64_t K) {
    if (check_weight_shape(N, K) != W12_OK) return 0;
    return (size_t)(w12_padded_rows(N) * K / 2);
}

size_t w12_meta_bytes(int64_t N, int64_t K) {
    if (check_weight_shape(N, K) != W12_OK) return 0;
    return (size_t)(w12_padded_rows(N) * (K / W12_GROUP));
}

size_t w12_bf16_tiled_bytes(int64_t N, int64_t K) {
    if (check_weight_shape(N, K) != W12_OK) return 0;
    return (size_t)(w12_padded_rows(N) * K * 2);
}

int w12_bf16_tile(const uint16_t* w, int64_t N, int64_t K, uint16_t* w_tiled, void* stream) {
    if (!w || !w_tiled) return W12_ERR_NULL;
    if (int rc = check_weight_shape(N, K)) return rc;
    if (!aligned16(w) || !aligned16(w_tiled)) return W12_ERR_ALIGN;
    return status_of(w12::launch_bf16_tile(w, N, K, w_tiled, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

static int pack_fmt(int fmt, const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1, void* p2,
                    uint8_t* meta, uint32_t* bad_groups, void* stream) {
    if (!w || !p0 || !p1 || !p2 || !meta) return W12_ERR_NULL;
    if (int rc = check_weight_shape(N, K)) return rc;
    if (!aligned16(w) || !aligned16(p0) || !aligned16(p1) || !aligned16(p2)) return W12_ERR_ALIGN;
    if (bad_groups && (reinterpret_cast<uintptr_t>(bad_groups) & 3u)) return W12_ERR_ALIGN;
    return status_of(w12::launch_pack(fmt, w, N, K, p0, p1, p2, meta, bad_groups,
                                      static_cast<hipStream_t>(stream)));
}

extern "C" {

int w12_pack(const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1, void* p2, uint8_t* meta,
             uint32_t* bad_groups, void* stream) {
    return pack_fmt(w12::kFmtV1, w, N, K, p0, p1, p2, meta, bad_groups, stream);
}

int w12b_pack(const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1, void* p2, uint8_t* meta,
              uint32_t* bad_groups, void* stream) {
    return pack_fmt(w12::kFmtB, w, N, K, p0, p1, p2, meta, bad_groups, stream);
}

size_t w12_exceptions_workspace_bytes(int64_t N, int64_t K) {
    if (check_weight_shape(N, K) != W12_OK) return 0;
    return (size_t)((N + W12_TILE_ROWS - 1) / W12_TILE_ROWS * (K / W12_GROUP) * 4);
}

}  // extern "C"

static int exceptions_fmt(int fmt, const uint16_t* w, int64_t N, int64_t K, void* workspace,
                          size_t workspace_bytes, uint32_t* exc_offsets, uint32_t* exc_entries,
                          int64_t capacity, uint32_t* total, void* stream) {
    if (!w || !exc_offsets || !total) return W12_ERR_NULL;
    if (int rc = check_weight_shape(N, K)) return rc;
    if (K >= kExcMaxK || (N + W12_TILE_ROWS) * K >= kExcMaxElems) return W12_ERR_SHAPE;
    if (capacity < 0 || (capacity > 0 && exc_entries == nullptr)) return W12_ERR_NULL;
    if (!aligned16(w) || !aligned8(exc_offsets) || !aligned4(total) ||
        (exc_entries && !aligned8(exc_entries)))
        return W12_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < w12_exceptions_workspace_bytes(N, K) ||
        !aligned4(workspace))
        return W12_ERR_WORKSPACE;
    return status_of(w12::launch_exceptions(fmt, w, N, K, static_cast<uint32_t*>(workspace),
                                            exc_offsets, exc_entries, capacity, total,
                                            static_cast<hipStream_t>(stream)));
}

static int unpack_fmt(int fmt, const void* p0, const void* p1, const void* p2, const uint8_t* meta,
                      const uint32_t* exc_offsets, const uint32_t* exc_entries, int64_t N,
                      int64_t K, uint16_t* w_out, void* stream) {
    if (!p0 || !p1 || !p2 || !meta || !w_out) return W12_ERR_NULL;
    if (int rc = check_weight_shape(N, K)) return rc;
    if (!aligned16(p0) || !aligned16(p1) || !aligned16(p2) || !aligned16(w_out)) return W12_ERR_ALIGN;
    if (int rc = check_exceptions(exc_offsets, exc_entries, N, K)) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (int rc = status_of(w12::launch_unpack(fmt, p0, p1, p2, meta, N, K, w_out, s))) return rc;
    if (exc_offsets == nullptr) return W12_OK;
    return status_of(w12::launch_apply_exceptions(exc_offsets, exc_entries, N, K, w_out, s));
}

extern "C" {

int w12_exceptions(const uint16_t* w, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                   uint32_t* exc_offsets, uint32_t* exc_entries, int64_t capacity, uint32_t* total,
                   void* stream) {
    return exceptions_fmt(w12::kFmtV1, w, N, K, workspace, workspace_bytes, exc_offsets, exc_entries,
                          capacity, total, stream);
}

int w12b_exceptions(const uint16_t* w, int64_t N, int64_t K, void* workspace,
                    size_t workspace_bytes, uint32_t* exc_offsets, uint32_t* exc_entries,
                    int64_t capacity, uint32_t* total, void* stream) {
    return exceptions_fmt(w12::kFmtB, w, N, K, workspace, workspace_bytes, exc_offsets, exc_entries,
                          capacity, total, stream);
}

int w12_unpack(const void* p0, const void* p1, const void* p2, const uint8_t* meta,
               const uint32_t* exc_offsets, const uint32_t* exc_entries, int64_t N, int64_t K,
               uint16_t* w_out, void* stream) {
    return unpack_fmt(w12::kFmtV1, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, w_out, stream);
}

int w12b_unpack(const void* p0, const void* p1, const void* p2, const uint8_t* meta,
                const uint32_t* exc_offsets, const uint32_t* exc_entries, int64_t N, int64_t K,
                uint16_t* w_out, void* stream) {
    return unpack_fmt(w12::kFmtB, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, w_out, stream);
}

static int resolve_tiling(const w12_tiling_t* tiling, bool allow_splitk, int64_t M, int64_t N,
                          int64_t K, w12::Tiling* out) {
    if (tiling == nullptr) {
        *out = w12::choose_tiling((int)M, N, K, allow_splitk);
        return W12_OK;
    }
    w12::Tiling t{};
    t.mfma = tiling->kind != 0;
    if (tiling->kind != 0 && tiling->kind != 1) return W12_ERR_UNSUPPORTED;
    t.r = tiling->r;
    t.kw = tiling->kw;
    t.depth = tiling->depth;
    if (tiling->x_direct != 0 && tiling->x_direct != 1) return W12_ERR_UNSUPPORTED;
    t.xdirect = tiling->x_direct;
    t.splitk = tiling->splitk == 0 ? 1 : tiling->splitk;
    t.nw = tiling->waves == 0 ? 4 : tiling->waves;
    if (!w12::complete_tiling(t, (int)M, N, K)) return W12_ERR_UNSUPPORTED;
    *out = t;
    return W12_OK;
}

static int check_workspace(const w12::Tiling& t, int64_t M, int64_t N, void* ws, size_t bytes) {
    const size_t need = w12::workspace_bytes(t, (int)M, N);
    if (need == 0) return W12_OK;
    if (ws == nullptr || bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return W12_ERR_WORKSPACE;
    return W12_OK;
}

// The default tiling of a W12-v1 GEMM whose container carries an exception
// list.  The x-direct MFMA tilings run one tile per wave: their workgroup's
// correction wave then has one tile's entries to prepare instead of two, and
// finishes within the main loop (the summation order of every output is
// unchanged).  From 6 rows the LDS-staged kernel, which applies the
// corrections inside its main loop, is faster than the x-direct one with its
// correction wave (raw QKV M = 8 13.1 against 14.2 us, gate+up M = 6 47.9
// against 49.1), and so it is at any row count when K is split three ways or
// more, with two K-waves (raw down M = 2, three slices: 26.0 against 31.4);
// it is taken with the same split when it needs no more workspace, so a
// workspace sized by w12_gemm_workspace_bytes still fits.
static void list_tiling(w12::Tiling& t, int64_t M, int64_t N, int64_t K) {
    if (!t.mfma || !t.xdirect) return;
    w12::Tiling t2{};
    t2.mfma = 1;
    t2.r = 1;
    t2.kw = t.splitk >= 3 ? 2 : 4;
    t2.depth = 2;
    t2.xdirect = 0;
    t2.splitk = t.splitk;
    t2.nw = 8;
    w12::Tiling t1 = t;
    t1.r = 1;
    if ((M >= 6 || t.splitk >= 3) && w12::complete_tiling(t2, (int)M, N, K) &&
        w12::workspace_bytes(t2, (int)M, N) <= w12::workspace_bytes(t, (int)M, N))
        t = t2;
    else if (t.r == 2 && w12::complete_tiling(t1, (int)M, N, K))
        t = t1;
}

static int gemm_w12(int fetch, const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
                    const void* p2, const uint8_t* meta, const uint32_t* exc_off,
                    const uint32_t* exc_ent, int64_t N, int64_t K, void* y,
                    int64_t ldy, int y_type, const w12_tiling_t* tiling, bool allow_splitk,
                    void* ws, size_t ws_bytes, void* stream) {
    if (!p0 || !p1 || !p2 || !meta) return W12_ERR_NULL;
    if (int rc = check_gemm_common(x, M, ldx, N, K, y, ldy, y_type)) return rc;
    if (!aligned16(p0) || !aligned16(p1) || !aligned16(p2)) return W12_ERR_ALIGN;
    if (int rc = check_exceptions(exc_off, exc_ent, N, K)) return rc;
    w12::Tiling t;
    if (int rc = resolve_tiling(tiling, allow_splitk, M, N, K, &t)) return rc;
    if (tiling == nullptr && exc_off != nullptr && fetch == w12::kFetchW12) list_tiling(t, M, N, K);
    if (int rc = check_workspace(t, M, N, ws, ws_bytes)) return rc;
    w12::GemmArgs a = make_args(x, M, ldx, N, K, y, ldy, y_type);
    a.p0 = static_cast<const uint8_t*>(p0);
    a.p1 = static_cast<const uint8_t*>(p1);
    a.p2 = static_cast<const uint8_t*>(p2);
    a.meta = meta;
    a.exc_off = exc_off;
    a.exc_ent = exc_ent;
    w12::bind_split(a, t, ws);
    return status_of(w12::launch_gemm(a, t, fetch, static_cast<hipStream_t>(stream)));
}

static int gemm_bf16(const uint16_t* x, int64_t M, int64_t ldx, const uint16_t* w, int64_t N,
                     int64_t K, void* y, int64_t ldy, int y_type, const w12_tiling_t* tiling,
                     bool allow_splitk, void* ws, size_t ws_bytes, void* stream) {
    if (!w) return W12_ERR_NULL;
    if (int rc = check_gemm_common(x, M, ldx, N, K, y, ldy, y_type)) return rc;
    if (!aligned16(w)) return W12_ERR_ALIGN;
    w12::Tiling t;
    if (int rc = resolve_tiling(tiling, allow_splitk, M, N, K, &t)) return rc;
    if (int rc = check_workspace(t, M, N, ws, ws_bytes)) return rc;
    w12::GemmArgs a = make_args(x, M, ldx, N, K, y, ldy, y_type);
    a.w = w;
    w12::bind_split(a, t, ws);
    return status_of(w12::launch_gemm(a, t, w12::kFetchBF16, static_cast<hipStream_t>(stream)));
}

int w12_gemm_ex(const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
                const void* p2, const uint8_t* meta, const uint32_t* exc_offsets,
                const uint32_t* exc_entries, int64_t N, int64_t K, void* y, int64_t ldy,
                int y_type, const w12_tiling_t* tiling, void* workspace, size_t workspace_bytes,
                void* stream) {
    return gemm_w12(w12::kFetchW12, x, M, ldx, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, y,
                    ldy, y_type, tiling, workspace != nullptr, workspace, workspace_bytes, stream);
}

int w12b_gemm_ex(const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
                 const void* p2, const uint8_t* meta, const uint32_t* exc_offsets,
                 const uint32_t* exc_entries, int64_t N, int64_t K, void* y, int64_t ldy,
                 int y_type, const w12_tiling_t* tiling, void* workspace, size_t workspace_bytes,
                 void* stream) {
    return gemm_w12(w12::kFetchW12B, x, M, ldx, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, y,
                    ldy, y_type, tiling, workspace != nullptr, workspace, workspace_bytes, stream);
}

int bf16_gemm_ex(const uint16_t* x, int64_t M, int64_t ldx, const uint16_t* w, int64_t N,
                 int64_t K, void* y, int64_t ldy, int y_type, const w12_tiling_t* tiling,
                 void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_bf16(x, M, ldx, w, N, K, y, ldy, y_type, tiling, workspace != nullptr, workspace,
                     workspace_bytes, stream);
}

int w12_gemm(const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
             const void* p2, const uint8_t* meta, const uint32_t* exc_offsets,
             const uint32_t* exc_entries, int64_t N, int64_t K, void* y, int64_t ldy, int y_type,
             void* stream) {
    return gemm_w12(w12::kFetchW12, x, M, ldx, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, y,
                    ldy, y_type, nullptr, false, nullptr, 0, stream);
}

int w12b_gemm(const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
              const void* p2, const uint8_t* meta, const uint32_t* exc_offsets,
              const uint32_t* exc_entries, int64_t N, int64_t K, void* y, int64_t ldy, int y_type,
              void* stream) {
    return gemm_w12(w12::kFetchW12B, x, M, ldx, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, y,
                    ldy, y_type, nullptr, false, nullptr, 0, stream);
}

int bf16_gemm(const uint16_t* x, int64_t M, int64_t ldx, const uint16_t* w, int64_t N, int64_t K,
              void* y, int64_t ldy, int y_type, void* stream) {
    return gemm_bf16(x, M, ldx, w, N, K, y, ldy, y_type, nullptr, false, nullptr, 0, stream);
}

int w12_gemm_ws(const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
                const void* p2, const uint8_t* meta, const uint32_t* exc_offsets,
                const uint32_t* exc_entries, int64_t N, int64_t K, void* y, int64_t ldy,
                int y_type, void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_w12(w12::kFetchW12, x, M, ldx, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, y,
                    ldy, y_type, nullptr, true, workspace, workspace_bytes, stream);
}

int w12b_gemm_ws(const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
                 const void* p2, const uint8_t* meta, const uint32_t* exc_offsets,
                 const uint32_t* exc_entries, int64_t N, int64_t K, void* y, int64_t ldy,
                 int y_type, void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_w12(w12::kFetchW12B, x, M, ldx, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, y,
                    ldy, y_type, nullptr, true, workspace, workspace_bytes, stream);
}

int bf16_gemm_ws(const uint16_t* x, int64_t M, int64_t ldx, const uint16_t* w, int64_t N,
                 int64_t K, void* y, int64_t ldy, int y_type, void* workspace,
                 size_t workspace_bytes, void* stream) {
    return gemm_bf16(x, M, ldx, w, N, K, y, ldy, y_type, nullptr, true, workspace, workspace_bytes,
                     stream);
}

int w12_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const w12_tiling_t* tiling,
                             size_t* bytes) {
    if (bytes == nullptr) return W12_ERR_NULL;
    *bytes = 0;
    if (int rc = check_weight_shape(N, K)) return rc;
    if (M < 1) return W12_ERR_SHAPE;
    if (M > W12_MAX_M) return W12_ERR_UNSUPPORTED;
    w12::Tiling t;
    if (int rc = resolve_tiling(tiling, true, M, N, K, &t)) return rc;
    *bytes = w12::workspace_bytes(t, (int)M, N);
    return W12_OK;
}

int w12_default_tiling(int64_t M, int64_t N, int64_t K, int allow_splitk, w12_tiling_t* out) {
    if (out == nullptr) return W12_ERR_NULL;
    if (int rc = check_weight_shape(N, K)) return rc;
    if (M < 1) return W12_ERR_SHAPE;
    if (M > W12_MAX_M) return W12_ERR_UNSUPPORTED;
    const w12::Tiling t = w12::choose_tiling((int)M, N, K, allow_splitk != 0);
    out->kind = t.mfma;
    out->r = t.r;
    out->kw = t.kw;
    out->depth = t.depth;
    out->x_direct = t.xdirect;
    out->splitk = t.splitk;
    out->waves = t.nw;
    return W12_OK;
}

const char* w12_tiling_variant(int64_t M, int64_t N, int64_t K, const w12_tiling_t* tiling,
                               int is_w12) {
    if (tiling == nullptr || is_w12 < 0 || is_w12 > 2) return nullptr;
    if (check_weight_shape(N, K) != W12_OK || M < 1 || M > W12_MAX_M) return nullptr;
    w12::Tiling t;
    if (resolve_tiling(tiling, true, M, N, K, &t) != W12_OK) return nullptr;
    const int fetch = is_w12 == 2 ? w12::kFetchW12B : is_w12 != 0 ? w12::kFetchW12 : w12::kFetchBF16;
    return w12::tiling_name(t, fetch);
}

const char* w12_gemm_variant(int64_t M, int64_t N, int64_t K, int is_w12, int allow_splitk) {
    if (check_weight_shape(N, K) != W12_OK || M < 1 || M > W12_MAX_M) return nullptr;
    if (is_w12 < 0 || is_w12 > 3) return nullptr;
    const int fetch = is_w12 == 2 ? w12::kFetchW12B : is_w12 != 0 ? w12::kFetchW12 : w12::kFetchBF16;
    w12::Tiling t = w12::choose_tiling((int)M, N, K, allow_splitk != 0);
    if (is_w12 == 3) list_tiling(t, M, N, K);
    return w12::tiling_name(t, fetch);
}

}  // extern "C"

// ---- w12_gemm_noalloc: split-K scratch in a fixed device array ---------------
// The counters (kCounterBytes, one per row block) followed by room for
// kScratchPartialBytes of fp32 partial sums.  Each GPU the library runs on
// holds its own copy for the life of the process.  In host code `scratch`
// names a host-side stand-in, never the device copy: kernels and copies
// take the address hipGetSymbolAddress returns for the current device.
namespace {
constexpr size_t kScratchPartialBytes = (size_t)16 << 20;
constexpr size_t kScratchBytes = (size_t)w12::kCounterBytes + kScratchPartialBytes;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void zero_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Device address of `scratch` on the current device.  The first call on a
// device looks it up and clears the whole array on `s` (a fill kernel, so
// the call may also be captured in a graph); every split-K launch leaves
// the counters at zero and no two-slice slot tagged.
int scratch_on_device(hipStream_t s, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W12_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return W12_ERR_HIP;
        constexpr int kWords = (int)(kScratchBytes / 4);
        hipLaunchKernelGGL(zero_words, dim3((kWords + 255) / 256), dim3(256), 0, s,
                           static_cast<uint32_t*>(ptr), kWords);
        if (hipGetLastError() != hipSuccess) return W12_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return W12_OK;
}

}  // namespace

extern "C" {

int w12_gemm_noalloc(const uint16_t* x, int64_t M, int64_t ldx, const void* p0, const void* p1,
                     const void* p2, const uint8_t* meta, const uint32_t* exc_offsets,
                     const uint32_t* exc_entries, int64_t N, int64_t K, void* y, int64_t ldy,
                     int y_type, void* stream) {
    // the argument checks of w12_gemm_ws, then the scratch limit, all before
    // any HIP call
    if (!p0 || !p1 || !p2 || !meta) return W12_ERR_NULL;
    if (int rc = check_gemm_common(x, M, ldx, N, K, y, ldy, y_type)) return rc;
    if (!aligned16(p0) || !aligned16(p1) || !aligned16(p2)) return W12_ERR_ALIGN;
    if (int rc = check_exceptions(exc_offsets, exc_entries, N, K)) return rc;
    const w12::Tiling t = w12::choose_tiling((int)M, N, K, true);
    if (w12::workspace_bytes(t, (int)M, N) > kScratchBytes) return W12_ERR_SCRATCH;
    void* ws = nullptr;
    if (int rc = scratch_on_device(static_cast<hipStream_t>(stream), &ws)) return rc;
    return gemm_w12(w12::kFetchW12, x, M, ldx, p0, p1, p2, meta, exc_offsets, exc_entries, N, K, y,
                    ldy, y_type, nullptr, true, ws, kScratchBytes, stream);
}

}  // extern "C"
