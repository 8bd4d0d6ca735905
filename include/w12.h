/*
 * w12.h -- C ABI of libw12.so: the W12 lossless 12-bit BF16 weight format and
 * small-M decode GEMMs for AMD MI355X (gfx950).
 *
 * The operation.  W12 stores each BF16 weight in 12 bits spread over three
 * 4-bit planes and rebuilds the exact BF16 bits in registers inside the GEMM
 * (AI Radar paper summary of SpecPilot, English edition, "Reasons", item on
 * the discovered mechanisms; HotRepo digest "StargazerX0/SpecPilot",
 * project introduction, second paragraph: decoded bit-exactly inside the
 * GEMM, batch 1-32).  The pages give no bit allocation; this library uses
 * format W12-v1:
 *
 *   group    = 128 consecutive weights along K of one row (K % 128 == 0);
 *   beta     = smallest beta >= 0 with 2*beta+15 >= the group's largest
 *              biased exponent E (0 <= beta <= 120);
 *   stored   = exponents {0, 1} and [2*beta+2, 2*beta+15] (4096 values);
 *   nibbles  = P0 = v[3:0], P1 = v[7:4], P2 = sign<<3 | h with h = 0 for
 *              E <= 1, else h = (E >> 1) - beta (1..7);
 *   layout   = rows are padded to Np = N rounded up to 16 (W12_TILE_ROWS);
 *              each plane is Np*K/2 bytes of 1 KB blocks, one per (16-row
 *              tile T = n/16, group g = k/128), ordered by (T, g); in a
 *              block, the 16-byte piece L = 16*q + c (q = 0..3, c = n%16)
 *              holds row n and, in its dword b (0..3), the 8 weights
 *              k = 128*g + 32*b + 8*q + e (e = 0..7): byte e%4 of the dword,
 *              low nibble for e < 4, high nibble for e >= 4;
 *   meta     = Np*K/128 bytes, 16 per (T, g), byte c = beta | 0x80 if the
 *              group of row 16*T + c is unencodable.
 * This order makes every load of a GEMM wave read 1 KB of contiguous memory
 * (one block of one plane), for both the GEMV and the MFMA kernels.
 *
 * A group holding an exponent in [2, 2*beta+1] cannot be stored exactly: the
 * packer flags it (meta bit 7), counts it, and stores that element as the
 * window floor +-2^(2*beta+2-127).  Unpack and GEMM ignore the flag and use
 * the stored (clamped) value -- unless the container carries an exception
 * list (w12_exceptions), which keeps it lossless for every input:
 *   exc_offsets = (Np/16)*(K/128) + 1 uint32 words, one per (tile, group)
 *                 block in block order and then the total: block
 *                 t = T*(K/128) + g (tile T = n/16, group g = k/128) owns
 *                 entries exc_offsets[t] .. exc_offsets[t+1]-1
 *                 (exc_offsets[0] = 0), so a GEMM finds the entries of the
 *                 block it is streaming without a search;
 *   exc_entries = two uint32 words per element below its window:
 *                 (c << 24 | k) with c = n % 16, and (beta << 16 | the
 *                 original BF16 word) with beta the group's base;
 *                 inside a block in storage order (piece L, dword b,
 *                 element e).
 * Unpack writes the original words back; the GEMMs add x[m][k] * (original -
 * clamp) for each entry to their sums (W12-v1 with x read directly: an extra
 * wave of each workgroup prepares those sums while the others stream the
 * weights; otherwise after the main loop).  Every call that takes a
 * container accepts exc_offsets = exc_entries = NULL for "no list"; a list
 * must come from w12_exceptions for the same weight (it is not validated on
 * the device), both arrays 8-byte aligned, and needs K < 2^24.
 *
 * Conventions for every call below:
 *   - all tensor pointers are DEVICE memory owned by the caller; the library
 *     allocates, frees and keeps nothing, and never synchronises;
 *   - BF16 tensors are passed as their 16-bit patterns;
 *   - `stream` is a hipStream_t (NULL = the default stream); work is enqueued
 *     on it and the call returns without waiting;
 *   - arguments are checked on the host before any launch; on error nothing
 *     is enqueued and a negative w12_status_t is returned;
 *   - launch failures return W12_ERR_HIP;
 *   - calls on different streams are independent (the library is stateless
 *     and thread-safe); outputs must not alias inputs;
 *   - the *_ws / *_ex GEMM calls may split K over workgroups; they then use a
 *     caller-owned device workspace (w12_gemm_workspace_bytes) that must be
 *     zero-filled before its first use and is left in that state by every
 *     call.  Calls that may run at the same time need separate workspaces.
 */
#ifndef W12_H
#define W12_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W12_ABI_VERSION 8
#define W12_GROUP 128
#define W12_TILE_ROWS 16
#define W12_MAX_M 128

typedef enum {
    W12_OK = 0,
    W12_ERR_NULL = -1,        /* a required pointer is NULL                  */
    W12_ERR_SHAPE = -2,       /* N < 1, K < 128, K % 128 != 0, K >= 2^24,
                                 N*K >= 2^40, M < 1, ld < K/N               */
    W12_ERR_ALIGN = -3,       /* pointer or leading dimension misaligned     */
    W12_ERR_DTYPE = -4,       /* unknown output type                         */
    W12_ERR_UNSUPPORTED = -6, /* M > 128, or a tiling not built             */
    W12_ERR_HIP = -7,         /* the HIP launch reported an error            */
    W12_ERR_WORKSPACE = -8,   /* split-K workspace NULL, short or misaligned */
    W12_ERR_SCRATCH = -9      /* w12_gemm_noalloc: partial sums over 16 MiB   */
} w12_status_t;

typedef enum {
    W12_OUT_BF16 = 0,         /* y stored as BF16 bits, round to nearest even */
    W12_OUT_F32 = 1           /* y stored as fp32                             */
} w12_out_t;

/* ABI version of the loaded library (W12_ABI_VERSION at build time). */
int w12_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *w12_status_string(int status);

/* Rows of the container: N rounded up to a multiple of 16 (0 if N < 1). */
int64_t w12_padded_rows(int64_t N);

/* Bytes of ONE nibble plane for an [N, K] weight: Np*K/2, so the three
 * planes hold exactly 0.75x the BF16 bytes when N % 16 == 0 -- 12 of every
 * 16 bits, in three 4-bit planes (AI Radar paper summary of SpecPilot,
 * English edition, "Reasons", mechanisms item).  0 on bad shape. */
size_t w12_plane_bytes(int64_t N, int64_t K);

/* Bytes of the metadata array: Np*K/128 (0 on bad shape). */
size_t w12_meta_bytes(int64_t N, int64_t K);

/* Bytes of a BF16 weight in the control layout: Np*K*2 (0 on bad shape). */
size_t w12_bf16_tiled_bytes(int64_t N, int64_t K);

/*
 * w12_pack -- BF16 [N, K] (row-major, contiguous) -> three planes + meta.
 * The format's encoder: it splits every BF16 weight into three 4-bit planes
 * (AI Radar paper summary of SpecPilot, English edition, "Reasons",
 * mechanisms item: W12 keeps 12 of the 16 bits of each weight, as three
 * nibble planes; HotRepo digest "StargazerX0/SpecPilot", project
 * introduction, second paragraph).  One 128-weight
 * group at a time, integer only; a group it cannot store exactly is flagged,
 * never silently rounded.
 *   w          : device, N*K BF16 words, 16-byte aligned.
 *   p0, p1, p2 : device outputs, w12_plane_bytes(N, K) bytes each, 16-byte
 *                aligned; padding rows are written as zeros.
 *   meta       : device output, w12_meta_bytes(N, K) bytes.
 *   bad_groups : device uint32 counter or NULL; the number of unencodable
 *                groups is ADDED to it (the caller zeroes it beforehand).
 * Errors: W12_ERR_NULL, W12_ERR_SHAPE, W12_ERR_ALIGN, W12_ERR_HIP.
 */
int w12_pack(const uint16_t *w, int64_t N, int64_t K,
             void *p0, void *p1, void *p2, uint8_t *meta,
             uint32_t *bad_groups, void *stream);

/*
 * w12_exceptions -- the exception list of a BF16 [N, K] weight: the escape
 * path that keeps the container lossless for every input, since the pages
 * call W12 lossless (AI Radar paper summary of SpecPilot, English edition,
 * "Reasons", mechanisms item) without saying how values outside a group's
 * 12-bit range are kept.  Format above.  Three launches: per-block counts
 * into `workspace`, one scan, and the entries.
 *   w           : device, the same N*K BF16 words given to w12_pack, 16-byte
 *                 aligned.
 *   workspace   : device, w12_exceptions_workspace_bytes(N, K) bytes, 4-byte
 *                 aligned (no initial contents needed).
 *   exc_offsets : device output, (Np/16)*(K/128) + 1 uint32 words, 8-byte
 *                 aligned.
 *   exc_entries : device output with room for `capacity` entries (2 words
 *                 each), 8-byte aligned, or NULL with capacity 0 to count
 *                 only.
 *   total       : device uint32 output: the number of entries.  Entries past
 *                 `capacity` are not written; a caller that finds
 *                 total > capacity calls again with more room.
 * Needs K < 2^24 and N*K < 2^32.
 * Errors: W12_ERR_NULL, W12_ERR_SHAPE, W12_ERR_ALIGN, W12_ERR_WORKSPACE,
 *         W12_ERR_HIP.
 */
size_t w12_exceptions_workspace_bytes(int64_t N, int64_t K);
int w12_exceptions(const uint16_t *w, int64_t N, int64_t K,
                   void *workspace, size_t workspace_bytes,
                   uint32_t *exc_offsets, uint32_t *exc_entries, int64_t capacity,
                   uint32_t *total, void *stream);

/*
 * w12_unpack -- planes + meta (+ exception list) -> BF16 [N, K]: the
 * lossless inverse of w12_pack (AI Radar paper summary of SpecPilot, English
 * edition, "Reasons", mechanisms item: W12 is lossless and rebuilt bit by
 * bit), exact on every unflagged group, and on every group when the
 * exception list is given; same in-register decode as the GEMMs.
 *   p0, p1, p2 : device, w12_plane_bytes(N, K) bytes each, 16-byte aligned.
 *   meta       : device, w12_meta_bytes(N, K) bytes.
 *   exc_offsets, exc_entries : the container's exception list, or both NULL.
 *   w_out      : device output, N*K BF16 words, 16-byte aligned.
 * Errors: W12_ERR_NULL, W12_ERR_SHAPE, W12_ERR_ALIGN, W12_ERR_HIP.
 */
int w12_unpack(const void *p0, const void *p1, const void *p2,
               const uint8_t *meta, const uint32_t *exc_offsets,
               const uint32_t *exc_entries, int64_t N, int64_t K,
               uint16_t *w_out, void *stream);

/*
 * w12_gemm -- y[m, n] = sum_k x[m, k] * W[n, k] with W read from a W12
 * container and rebuilt bit by bit in registers inside the GEMM (AI Radar
 * paper summary of SpecPilot, English edition, "Reasons", mechanisms item;
 * HotRepo digest "StargazerX0/SpecPilot", project introduction, second
 * paragraph: decoded bit-exactly inside the GEMM at batch 1-32), fp32
 * accumulation.
 *   x      : device BF16 [M, K], row stride ldx elements (ldx >= K,
 *            ldx % 8 == 0), 16-byte aligned.  1 <= M <= 128.
 *   p0..meta: the container of an [N, K] weight as written by w12_pack.
 *   exc_offsets, exc_entries: its exception list (w12_exceptions) or both
 *            NULL; with a list the result is the GEMM of the original
 *            weights (within the fp32 tolerance; each correction takes the
 *            clamp back out and adds the original, so a one-hot x row
 *            returns an original word exactly; applied by an extra wave
 *            when x is read directly, inside the main loop when x is
 *            staged in LDS, up to 32 rows, else after the main loop).
 *   y      : device output [M, N], row stride ldy elements (ldy >= N),
 *            BF16 bits (2-byte aligned) or fp32 (4-byte aligned) per y_type.
 * By default M = 1 runs a wavefront-reduction GEMV (v_dot2c_f32_bf16) and
 * 2 <= M <= 128 runs bf16 MFMA with x padded to 16, 32, 64 or 128 rows
 * (measured crossover; above 32 rows with x in LDS, 512-thread
 * workgroups); w12_gemm_ex selects either explicitly (GEMV up to M = 8).
 * Each workgroup covers all of K for its rows, so no workspace is needed;
 * w12_gemm_ws adds the split-K tilings.
 * Errors: W12_ERR_NULL, W12_ERR_SHAPE, W12_ERR_ALIGN, W12_ERR_DTYPE,
 *         W12_ERR_UNSUPPORTED (M > 128), W12_ERR_HIP.
 */
int w12_gemm(const uint16_t *x, int64_t M, int64_t ldx,
             const void *p0, const void *p1, const void *p2,
             const uint8_t *meta, const uint32_t *exc_offsets,
             const uint32_t *exc_entries, int64_t N, int64_t K,
             void *y, int64_t ldy, int y_type, void *stream);

/*
 * w12_bf16_tile -- row-major BF16 [N, K] -> the layout of the BF16 control,
 * the plain BF16 decoding W12 is measured against (HotRepo digest
 * "StargazerX0/SpecPilot", project introduction, second paragraph): the
 * same (tile, group) blocks and lane order as the W12 planes,
 * with whole BF16 words: block (T, g) of 2048 words, 1 KB sub-block b, lane
 * L's 8 words k = 128*g + 32*b + 8*q + e in natural order; padding rows zero.
 *   w       : device, N*K words, 16-byte aligned.
 *   w_tiled : device output, w12_bf16_tiled_bytes(N, K) bytes, 16-byte aligned.
 * Errors: W12_ERR_NULL, W12_ERR_SHAPE, W12_ERR_ALIGN, W12_ERR_HIP.
 */
int w12_bf16_tile(const uint16_t *w, int64_t N, int64_t K, uint16_t *w_tiled,
                  void *stream);

/*
 * bf16_gemm -- the control: plain BF16 decoding, the baseline W12 is said to
 * speed up by 1.15-1.26x at batch 1-32 (HotRepo digest
 * "StargazerX0/SpecPilot", project introduction, second paragraph; AI Radar
 * paper summary of SpecPilot, English edition, "Reasons", mechanisms item).
 * The same kernels, tiling, memory access order and summation order as
 * w12_gemm, with W read as plain BF16 words.  For
 * w_tiled = w12_bf16_tile(unpack(pack(W))) the two calls return bitwise
 * identical y.
 *   w_tiled : device, the [N, K] weight in the control layout (see
 *             w12_bf16_tile), 16-byte aligned.
 *   other arguments and errors as w12_gemm.
 */
int bf16_gemm(const uint16_t *x, int64_t M, int64_t ldx,
              const uint16_t *w_tiled, int64_t N, int64_t K,
              void *y, int64_t ldy, int y_type, void *stream);

/*
 * Explicit tiling, for callers that tune the kernels on their own shapes.
 *   kind  : 0 = wavefront-reduction GEMV (M <= 8), 1 = bf16 MFMA (M <= 128;
 *           above 32 rows only with waves = 8).
 *   r     : 16-row weight tiles per wave (1, 2).
 *   kw    : waves of a workgroup that split K (1, 2, 4; 8 with waves = 8);
 *           the workgroup's other waves take further weight tiles.
 *   depth : 128-weight groups each wave keeps in flight
 *           (r = 1: 2, 4 or 8; r = 2: 2 or 4).
 *   x_direct : 1 = each lane loads the x values of a group together with
 *           its weights (no LDS staging, no x barrier); 0 = x is staged in
 *           LDS.  Built when the register ring stays within ~192 VGPRs:
 *           GEMV M <= 4 with depth * (16 * r + 4 * M) <= 192; MFMA with
 *           depth * 16 * (r + M/16 rounded up) <= 192.
 *   splitk : workgroups that split K between them (0 or 1 = none, up to
 *           64); the groups are dealt out in contiguous slices of
 *           ceil(G / splitk) groups (G = K / 128), so the launch uses
 *           ceil(G / that) slices.  Each slice's fp32 partial sums go to the
 *           workspace; the last workgroup of a row block to finish adds them
 *           in slice order and writes y.
 *   waves : waves per workgroup: 0 or 4 = 256 threads; 8 = 512 threads,
 *           built for kind 1 with x in LDS and depth = 2, with r = 1, or
 *           r = 2 and kw = 1 above 32 rows (more waves share each x tile
 *           staged in LDS); 16 = 1024 threads, the same with r = 1,
 *           2 <= kw <= 8 and at most 32 rows (twice the weight loads in
 *           flight per x copy).
 * When the x columns of a slice do not fit LDS at once they are streamed in
 * chunks; some kw x depth combinations then need more than 64 KB of LDS
 * (128 KB with waves = 8) and are rejected.  The summation order depends
 * on the tiling and never on scheduling; w12 and bf16 kernels with the
 * same tiling sum in the same order.
 */
typedef struct {
    int32_t kind;
    int32_t r;
    int32_t kw;
    int32_t depth;
    int32_t x_direct;
    int32_t splitk;
    int32_t waves;
} w12_tiling_t;

/* The tiling the GEMMs use for this shape: that of w12_gemm / bf16_gemm
 * (allow_splitk = 0) or of w12_gemm_ws / bf16_gemm_ws (allow_splitk = 1).
 * Returns W12_OK, or W12_ERR_NULL / W12_ERR_SHAPE / W12_ERR_UNSUPPORTED. */
int w12_default_tiling(int64_t M, int64_t N, int64_t K, int allow_splitk,
                       w12_tiling_t *out);

/*
 * Workspace bytes a GEMM of this shape needs with `tiling` (NULL = the
 * w12_gemm_ws default); 0 when the tiling does not split K.  The workspace
 * holds a 64 KB counter area (one 32-bit counter per row block, at most
 * 16384 row blocks, so a split-K tiling with more is W12_ERR_UNSUPPORTED)
 * and then splitk * M * Np fp32 partial sums (Np = N rounded up to 16).
 * The counter area sits at the start for every shape, so one workspace can
 * serve GEMMs of different shapes in turn.
 * Returns W12_OK, or W12_ERR_NULL / W12_ERR_SHAPE / W12_ERR_UNSUPPORTED.
 */
int w12_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K,
                             const w12_tiling_t *tiling, size_t *bytes);

/*
 * w12_gemm / bf16_gemm with the default tiling including split K, which
 * fills the GPU on shapes with few row blocks (small N, long K).  Same
 * operation and passages as w12_gemm and bf16_gemm.
 *   workspace       : device, at least w12_gemm_workspace_bytes(M, N, K,
 *                     NULL) bytes, 256-byte aligned, zero-filled before its
 *                     first use (every call leaves it ready for the next:
 *                     counters zero, two-slice slots empty);
 *                     may be NULL when that size is 0.
 * Additional error: W12_ERR_WORKSPACE.
 */
int w12_gemm_ws(const uint16_t *x, int64_t M, int64_t ldx,
                const void *p0, const void *p1, const void *p2,
                const uint8_t *meta, const uint32_t *exc_offsets,
                const uint32_t *exc_entries, int64_t N, int64_t K,
                void *y, int64_t ldy, int y_type,
                void *workspace, size_t workspace_bytes, void *stream);
int bf16_gemm_ws(const uint16_t *x, int64_t M, int64_t ldx,
                 const uint16_t *w_tiled, int64_t N, int64_t K,
                 void *y, int64_t ldy, int y_type,
                 void *workspace, size_t workspace_bytes, void *stream);

/* The GEMMs with an explicit tiling (same operation and passages as w12_gemm
 * and bf16_gemm).  tiling = NULL selects the default of
 * w12_gemm_ws if a workspace is given, else that of w12_gemm.  A tiling with
 * splitk > 1 needs the workspace w12_gemm_workspace_bytes reports for it.
 * Additional errors: W12_ERR_UNSUPPORTED for a tiling that is not built or
 * does not fit M (GEMV needs M <= 8); W12_ERR_WORKSPACE. */
int w12_gemm_ex(const uint16_t *x, int64_t M, int64_t ldx,
                const void *p0, const void *p1, const void *p2,
                const uint8_t *meta, const uint32_t *exc_offsets,
                const uint32_t *exc_entries, int64_t N, int64_t K,
                void *y, int64_t ldy, int y_type, const w12_tiling_t *tiling,
                void *workspace, size_t workspace_bytes, void *stream);
int bf16_gemm_ex(const uint16_t *x, int64_t M, int64_t ldx,
                 const uint16_t *w_tiled, int64_t N, int64_t K,
                 void *y, int64_t ldy, int y_type, const w12_tiling_t *tiling,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Name of the kernel variant the GEMMs launch for this shape (static string,
 * for reports and profiles), or NULL if the shape is rejected.  `is_w12`
 * selects the weight fetch (0 = BF16 control, 1 = W12-v1, 2 = W12-b, 3 =
 * W12-v1 with an exception list, whose default can differ), `allow_splitk`
 * the w12_gemm_ws default.
 */
const char *w12_gemm_variant(int64_t M, int64_t N, int64_t K, int is_w12,
                             int allow_splitk);

/*
 * Name of the kernel variant an explicit tiling launches for this shape
 * (the same names as w12_gemm_variant; static string), or NULL if the
 * tiling or shape is rejected.  `is_w12` as above (0, 1 or 2).  For reports
 * and profiles of a chosen tiling.
 */
const char *w12_tiling_variant(int64_t M, int64_t N, int64_t K,
                               const w12_tiling_t *tiling, int is_w12);

/*
 * w12_gemm_noalloc -- w12_gemm_ws for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, default tiling (K split over
 * workgroups where that is faster) and result, bit for bit, as w12_gemm_ws,
 * with the split-K counters and partial sums kept in a fixed array inside
 * the library instead of a caller workspace.  The call allocates and frees
 * nothing, neither does any library routine it calls.
 *   arguments : as w12_gemm (the caller still owns x, the container and y).
 *   limit     : the shape's split-K partial sums, splitk * M * Np * 4 bytes
 *               of the w12_gemm_ws default tiling (w12_gemm_workspace_bytes
 *               minus its 64 KB counter area), must fit 16 MiB -- every M up
 *               to 128 on weights up to 7168 x 5120 and 5120 x 17408 does;
 *               larger ones return W12_ERR_SCRATCH before any launch.
 *   scratch   : 16 MiB + 64 KB of device memory per GPU the call runs on,
 *               held from its first call on that GPU until the process ends
 *               (that first call also enqueues one small kernel that clears
 *               it; every call leaves it ready for the next).  Every call on one GPU shares that GPU's
 *               array, so calls that may overlap on one GPU -- on different
 *               streams, or from different threads -- race and must be
 *               ordered by the caller.
 * Errors: those of w12_gemm, W12_ERR_SCRATCH, W12_ERR_HIP.
 */
int w12_gemm_noalloc(const uint16_t *x, int64_t M, int64_t ldx,
                     const void *p0, const void *p1, const void *p2,
                     const uint8_t *meta, const uint32_t *exc_offsets,
                     const uint32_t *exc_entries, int64_t N, int64_t K,
                     void *y, int64_t ldy, int y_type, void *stream);

/*
 * W12-b: the arbitrary-base bit allocation (the alternative to W12-v1 that
 * gives each group one more stored exponent at about 1.6x the decode
 * instructions; same pages as W12-v1: 12 bits per weight in three 4-bit
 * planes, rebuilt bit-exactly in the GEMM).  Per group:
 *   b        = smallest b >= 0 with b + 15 >= the group's largest biased
 *              exponent E (0 <= b <= 240);
 *   stored   = exponents {0} and [b+1, b+15] (4096 values);
 *   nibbles  = P0 = m[3:0], P1 = sign<<3 | m[6:4], P2 = c with c = 0 for
 *              E = 0, else c = E - b (1..15);
 *   layout   = the W12-v1 tiles, blocks and split-nibble order;
 *   meta     = the byte b itself (no flag bit: b needs 8 bits); flagged
 *              groups are only counted (bad_groups);
 *   clamp    = an exponent in [1, b] is stored as +-2^(b+1-127);
 *   list     = the W12-v1 exception-list layout, word 1 = (b << 16 | the
 *              original BF16 word).
 * The calls below take and return W12-b containers with exactly the
 * arguments, sizes, conventions and errors of the W12-v1 call of the same
 * name without the "b"; a W12-b container must not be passed to a W12-v1
 * call or the other way round (the meta bytes are read differently).
 */
int w12b_pack(const uint16_t *w, int64_t N, int64_t K,
              void *p0, void *p1, void *p2, uint8_t *meta,
              uint32_t *bad_groups, void *stream);
int w12b_exceptions(const uint16_t *w, int64_t N, int64_t K,
                    void *workspace, size_t workspace_bytes,
                    uint32_t *exc_offsets, uint32_t *exc_entries,
                    int64_t capacity, uint32_t *total, void *stream);
int w12b_unpack(const void *p0, const void *p1, const void *p2,
                const uint8_t *meta, const uint32_t *exc_offsets,
                const uint32_t *exc_entries, int64_t N, int64_t K,
                uint16_t *w_out, void *stream);
int w12b_gemm(const uint16_t *x, int64_t M, int64_t ldx,
              const void *p0, const void *p1, const void *p2,
              const uint8_t *meta, const uint32_t *exc_offsets,
              const uint32_t *exc_entries, int64_t N, int64_t K,
              void *y, int64_t ldy, int y_type, void *stream);
int w12b_gemm_ws(const uint16_t *x, int64_t M, int64_t ldx,
                 const void *p0, const void *p1, const void *p2,
                 const uint8_t *meta, const uint32_t *exc_offsets,
                 const uint32_t *exc_entries, int64_t N, int64_t K,
                 void *y, int64_t ldy, int y_type,
                 void *workspace, size_t workspace_bytes, void *stream);
int w12b_gemm_ex(const uint16_t *x, int64_t M, int64_t ldx,
                 const void *p0, const void *p1, const void *p2,
                 const uint8_t *meta, const uint32_t *exc_offsets,
                 const uint32_t *exc_entries, int64_t N, int64_t K,
                 void *y, int64_t ldy, int y_type, const w12_tiling_t *tiling,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * w12_read_probe -- measurement aid, not part of the W12 operation: reads
 * `bytes` of device memory with 16-byte non-temporal loads (each wave a
 * contiguous run, eight loads in flight per lane) and writes nothing but a
 * word to sink[0] in the rare case that the xor of all words read equals
 * 0x9E3779B9.  A GEMM that streams its weights once is bounded by this
 * rate on a buffer of the same size; the benchmark reports both.  The pages
 * tune kernels against the memory-bandwidth limit (AI Radar paper summary
 * of SpecPilot, English edition, opening paragraph).
 *   buf   : device, 16-byte aligned, bytes % 16 == 0, bytes > 0.
 *   sink  : device, 4 bytes, 4-byte aligned.
 * Errors: W12_ERR_NULL, W12_ERR_ALIGN, W12_ERR_SHAPE (bytes == 0), W12_ERR_HIP.
 */
int w12_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W12_H */
