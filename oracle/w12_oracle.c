/*
 * w12_oracle.c -- plain, slow, scalar CPU oracle for the W12 lossless
 * 12-bit weight format and the decode GEMM built on it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library; everything below is written from the
 * format definition, one element at a time.
 *
 * What the pages fix (AI Radar summary of SpecPilot, English edition,
 * "Reasons", the item on discovered mechanisms; HotRepo digest of
 * StargazerX0/SpecPilot, "项目介绍" / project introduction, second
 * paragraph): W12 is a lossless 12-bit weight format that splits each BF16
 * weight into three 4-bit planes and rebuilds the BF16 value bit-exactly
 * inside the GEMM.  The pages leave the bit allocation open; the allocation
 * used here (format "W12-v1") is this project's own reading:
 *
 *   BF16 word v = s | E[7:0] | m[6:0]  (sign, biased exponent, mantissa).
 *   The low byte of v (E bit 0 and the 7 mantissa bits) is kept verbatim in
 *   two planes: P0 = v[3:0], P1 = v[7:4].
 *   P2 = (s << 3) | h, where h is a 3-bit code for E[7:1] relative to a
 *   per-group base beta:  h = 0 when E <= 1 (zeros, subnormals, smallest
 *   normal binade), otherwise h = (E >> 1) - beta in 1..7.
 *   A group is 128 consecutive weights along K in one row; beta is the
 *   smallest value >= 0 whose window [2*beta+2, 2*beta+15] reaches the
 *   group's largest exponent.  Exponents in {0, 1} and in the window are
 *   stored exactly; any other exponent makes the group unencodable: the
 *   group is flagged (bit 7 of its metadata byte) and the offending element
 *   is written as the window floor +-2^(2*beta+2-127) (sign kept).
 *
 * Layout (K % 128 == 0; rows padded to Np = N rounded up to a multiple of 16,
 * padding rows hold zero nibbles and a zero meta byte):
 *   each plane is Np*K/2 bytes made of 1024-byte blocks, one per (16-row
 *   tile T = n/16, 128-weight group g = k/128), blocks ordered by (T, g);
 *   inside a block, 64 pieces of 16 bytes; piece L = 16*q + c (q = 0..3,
 *   c = n%16) holds row n and, in its dword b (b = 0..3), the 8 weights
 *   k = 128*g + 32*b + 8*q + e (e = 0..7) in "split-nibble" order: byte e%4
 *   of the dword, low nibble for e < 4, high nibble for e >= 4;
 *   meta is Np*K/128 bytes: 16 bytes per (T, g), one per row c, each
 *   beta | (bad ? 0x80 : 0).
 * The same order with whole BF16 words is the layout of the BF16 control
 * (w12o_bf16_tile): block (T, g) of 2048 words, sub-block b of 512 words,
 * 8 words per piece L, words k = 128*g + 32*b + 8*q + e in natural order.
 *
 * A second allocation, format "W12-b" (fmt = 1 in the *_fmt functions), is
 * the arbitrary-base alternative: a 4-bit exponent offset c from a
 * per-group base b that may take any value, instead of W12-v1's 3-bit offset
 * of E[7:1] from an even base:
 *   P0 = m[3:0];  P1 = (s << 3) | m[6:4];  P2 = c, where c = 0 when E = 0
 *   (zeros and subnormals) and c = E - b in 1..15 otherwise.
 *   b is the smallest value >= 0 with b + 15 >= the group's largest
 *   exponent (0 <= b <= 240); exponents {0} and [b+1, b+15] are stored
 *   exactly (15 + 1 per group, any alignment), anything else is written as
 *   the window floor +-2^(b+1-127) (c = 1, mantissa 0, sign kept).
 *   The meta byte is b itself (no flag bit: b needs all 8 bits); flagged
 *   groups are counted, and their elements are listed in the exception
 *   list with word 1 = (b << 16) | original.
 * Same planes, tiles, split-nibble order and exception-list order as W12-v1.
 *
 * Build: gcc -O2 -std=c11 -shared -fPIC w12_oracle.c -o libw12_oracle.so -lpthread
 * (no -ffast-math: the GEMM must keep IEEE semantics).
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <pthread.h>

#define W12O_GROUP 128

/* ---- BF16 fields (the IEEE bfloat16 definition) ------------------------ */

static int bf16_sign(uint16_t v) { return (v >> 15) & 1; }
static int bf16_exponent(uint16_t v) { return (v >> 7) & 0xFF; }
static int bf16_low_byte(uint16_t v) { return v & 0xFF; }

/* bf16 -> double: a bf16 word is the top half of an fp32 word, and every
 * fp32 value is exactly representable as a double. */
static double bf16_to_double(uint16_t v)
{
    uint32_t u = (uint32_t)v << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- per-group base (reading of "three 4-bit planes": beta rule) ------- */

#define W12O_FMT_V1 0
#define W12O_FMT_B 1

/* Smallest beta >= 0 whose window [2*beta+2, 2*beta+15] reaches emax.
 * Written as a search, not a closed form, so it can be read off the rule. */
int w12o_beta_for_emax(int emax)
{
    int beta = 0;
    while (2 * beta + 15 < emax)
        beta++;
    return beta;
}

/* 1 if the BF16 word v is stored exactly by a group with base beta. */
int w12o_encodable(uint16_t v, int beta)
{
    int e = bf16_exponent(v);
    return e <= 1 || (e >= 2 * beta + 2 && e <= 2 * beta + 15);
}

/* ---- one element: BF16 word <-> 12-bit code ------------------------------
 * code bits 11..8 = P2 nibble, 7..4 = P1 nibble, 3..0 = P0 nibble.
 * *ok is set to 0 when v is outside the group's window; the code then holds
 * the clamp (window floor for small exponents, window top for large ones --
 * the latter never occurs inside a packed group because beta covers the
 * group's largest exponent). */
uint16_t w12o_encode(uint16_t v, int beta, int *ok)
{
    int s = bf16_sign(v);
    int e = bf16_exponent(v);
    int lo = bf16_low_byte(v);
    int h;
    int good = 1;

    if (e <= 1) {
        h = 0;                        /* E[7:1] == 0: low byte carries E0 */
    } else if (e >= 2 * beta + 2 && e <= 2 * beta + 15) {
        h = (e >> 1) - beta;          /* 1..7 */
    } else if (e < 2 * beta + 2) {
        good = 0;                     /* below the window: clamp up */
        h = 1;
        lo = 0;                       /* E = 2*beta+2, mantissa 0 */
    } else {
        good = 0;                     /* above the window: saturate */
        h = 7;
        lo = 0xFF;                    /* E = 2*beta+15, mantissa all ones */
    }
    if (ok)
        *ok = good;
    return (uint16_t)((((s << 3) | h) << 8) | lo);
}

uint16_t w12o_decode(uint16_t code, int beta)
{
    int p2 = (code >> 8) & 0xF;
    int s = (p2 >> 3) & 1;
    int h = p2 & 7;
    int lo = code & 0xFF;
    int e_hi = (h == 0) ? 0 : beta + h;   /* E[7:1] */
    return (uint16_t)((s << 15) | (e_hi << 8) | lo);
}

/* ---- W12-b: the arbitrary-base allocation ------------------------------ */

/* Smallest b >= 0 whose window [b+1, b+15] reaches emax (a search again). */
int w12o_b_base_for_emax(int emax)
{
    int b = 0;
    while (b + 15 < emax)
        b++;
    return b;
}

int w12o_b_encodable(uint16_t v, int b)
{
    int e = bf16_exponent(v);
    return e == 0 || (e >= b + 1 && e <= b + 15);
}

/* code bits 11..8 = P2 nibble (c), 7..4 = P1 nibble (s, m6..m4), 3..0 = P0
 * nibble (m3..m0). */
uint16_t w12o_b_encode(uint16_t v, int b, int *ok)
{
    int s = bf16_sign(v);
    int e = bf16_exponent(v);
    int m = v & 0x7F;
    int c;
    int good = 1;

    if (e == 0) {
        c = 0;                        /* zeros and subnormals */
    } else if (e >= b + 1 && e <= b + 15) {
        c = e - b;                    /* 1..15 */
    } else if (e < b + 1) {
        good = 0;                     /* below the window: clamp up */
        c = 1;
        m = 0;                        /* E = b+1, mantissa 0 */
    } else {
        good = 0;                     /* above the window: saturate */
        c = 15;
        m = 0x7F;
    }
    if (ok)
        *ok = good;
    return (uint16_t)((c << 8) | (s << 7) | m);
}

uint16_t w12o_b_decode(uint16_t code, int b)
{
    int c = (code >> 8) & 0xF;
    int s = (code >> 7) & 1;
    int m = code & 0x7F;
    int e = (c == 0) ? 0 : b + c;
    return (uint16_t)((s << 15) | (e << 7) | m);
}

/* ---- the two allocations behind one interface -------------------------- */

static int fmt_base_for_emax(int fmt, int emax)
{
    return fmt == W12O_FMT_B ? w12o_b_base_for_emax(emax) : w12o_beta_for_emax(emax);
}

static int fmt_encodable(int fmt, uint16_t v, int base)
{
    return fmt == W12O_FMT_B ? w12o_b_encodable(v, base) : w12o_encodable(v, base);
}

static uint16_t fmt_encode(int fmt, uint16_t v, int base, int *ok)
{
    return fmt == W12O_FMT_B ? w12o_b_encode(v, base, ok) : w12o_encode(v, base, ok);
}

static uint16_t fmt_decode(int fmt, uint16_t code, int base)
{
    return fmt == W12O_FMT_B ? w12o_b_decode(code, base) : w12o_decode(code, base);
}

/* meta byte <-> base: W12-v1 keeps a flag in bit 7, W12-b the base only */
static uint8_t fmt_meta(int fmt, int base, int bad)
{
    return fmt == W12O_FMT_B ? (uint8_t)base : (uint8_t)(base | (bad ? 0x80 : 0));
}

static int fmt_base_of_meta(int fmt, uint8_t meta)
{
    return fmt == W12O_FMT_B ? meta : (meta & 0x7F);
}

/* Element-wise loops over the two functions above (for exhaustive tests). */
void w12o_encode_many(const uint16_t *v, int64_t n, int beta,
                      uint16_t *code, uint8_t *ok)
{
    for (int64_t i = 0; i < n; i++) {
        int good;
        code[i] = w12o_encode(v[i], beta, &good);
        ok[i] = (uint8_t)good;
    }
}

void w12o_decode_many(const uint16_t *code, int64_t n, int beta, uint16_t *v)
{
    for (int64_t i = 0; i < n; i++)
        v[i] = w12o_decode(code[i], beta);
}

void w12o_b_encode_many(const uint16_t *v, int64_t n, int b, uint16_t *code, uint8_t *ok)
{
    for (int64_t i = 0; i < n; i++) {
        int good;
        code[i] = w12o_b_encode(v[i], b, &good);
        ok[i] = (uint8_t)good;
    }
}

void w12o_b_decode_many(const uint16_t *code, int64_t n, int b, uint16_t *v)
{
    for (int64_t i = 0; i < n; i++)
        v[i] = w12o_b_decode(code[i], b);
}

/* ---- plane addressing (16 x 128 tiles, split-nibble order) ------------- */

int64_t w12o_padded_rows(int64_t N)
{
    return (N + 15) / 16 * 16;
}

static int64_t nibble_byte(int64_t n, int64_t K, int64_t k)
{
    int64_t tile = n / 16, c = n % 16;
    int64_t group = k / W12O_GROUP, r = k % W12O_GROUP;
    int64_t b = r / 32, q = (r % 32) / 8, e = r % 8;
    int64_t block = tile * (K / W12O_GROUP) + group;
    return block * 1024 + (16 * q + c) * 16 + 4 * b + e % 4;
}

static int nibble_shift(int64_t k)
{
    return (k % 8) < 4 ? 0 : 4;
}

static int64_t meta_byte(int64_t n, int64_t K, int64_t k)
{
    return ((n / 16) * (K / W12O_GROUP) + k / W12O_GROUP) * 16 + n % 16;
}

static void put_nibble(uint8_t *plane, int64_t n, int64_t K, int64_t k, int nib)
{
    int64_t b = nibble_byte(n, K, k);
    int sh = nibble_shift(k);
    plane[b] = (uint8_t)((plane[b] & ~(0xF << sh)) | ((nib & 0xF) << sh));
}

static int get_nibble(const uint8_t *plane, int64_t n, int64_t K, int64_t k)
{
    return (plane[nibble_byte(n, K, k)] >> nibble_shift(k)) & 0xF;
}

/* ---- pack / unpack ------------------------------------------------------- */

/* Returns the number of unencodable (flagged) groups, or -1 on bad shape. */
/* The planes and meta must hold w12o_padded_rows(N) rows; padding rows are
 * written as zeros. */
int64_t w12o_pack_fmt(int fmt, const uint16_t *w, int64_t N, int64_t K,
                      uint8_t *p0, uint8_t *p1, uint8_t *p2, uint8_t *meta)
{
    if (N < 0 || K < 0 || K % W12O_GROUP != 0)
        return -1;
    int64_t groups = K / W12O_GROUP;
    int64_t bad_groups = 0;
    int64_t Np = w12o_padded_rows(N);
    memset(p0, 0, (size_t)(Np * K / 2));
    memset(p1, 0, (size_t)(Np * K / 2));
    memset(p2, 0, (size_t)(Np * K / 2));
    memset(meta, 0, (size_t)(Np * groups));
    for (int64_t n = 0; n < N; n++) {
        for (int64_t g = 0; g < groups; g++) {
            int emax = 0;
            for (int i = 0; i < W12O_GROUP; i++) {
                int e = bf16_exponent(w[n * K + g * W12O_GROUP + i]);
                if (e > emax)
                    emax = e;
            }
            int beta = fmt_base_for_emax(fmt, emax);
            int bad = 0;
            for (int i = 0; i < W12O_GROUP; i++) {
                int64_t k = g * W12O_GROUP + i;
                int ok;
                uint16_t code = fmt_encode(fmt, w[n * K + k], beta, &ok);
                if (!ok)
                    bad = 1;
                put_nibble(p0, n, K, k, code & 0xF);
                put_nibble(p1, n, K, k, (code >> 4) & 0xF);
                put_nibble(p2, n, K, k, (code >> 8) & 0xF);
            }
            meta[meta_byte(n, K, g * W12O_GROUP)] = fmt_meta(fmt, beta, bad);
            bad_groups += bad;
        }
    }
    return bad_groups;
}

int64_t w12o_pack(const uint16_t *w, int64_t N, int64_t K,
                  uint8_t *p0, uint8_t *p1, uint8_t *p2, uint8_t *meta)
{
    return w12o_pack_fmt(W12O_FMT_V1, w, N, K, p0, p1, p2, meta);
}

/* Returns 0, or -1 on bad shape. Flagged groups decode to their clamped
 * values (the flag bit is ignored by the decoder). */
int w12o_unpack_fmt(int fmt, const uint8_t *p0, const uint8_t *p1, const uint8_t *p2,
                    const uint8_t *meta, int64_t N, int64_t K, uint16_t *w)
{
    if (N < 0 || K < 0 || K % W12O_GROUP != 0)
        return -1;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int beta = fmt_base_of_meta(fmt, meta[meta_byte(n, K, k)]);
            uint16_t code = (uint16_t)((get_nibble(p2, n, K, k) << 8) |
                                       (get_nibble(p1, n, K, k) << 4) |
                                       get_nibble(p0, n, K, k));
            w[n * K + k] = fmt_decode(fmt, code, beta);
        }
    }
    return 0;
}

int w12o_unpack(const uint8_t *p0, const uint8_t *p1, const uint8_t *p2,
                const uint8_t *meta, int64_t N, int64_t K, uint16_t *w)
{
    return w12o_unpack_fmt(W12O_FMT_V1, p0, p1, p2, meta, N, K, w);
}

/* ---- exception list: the escape path for unencodable groups --------------
 * An element whose exponent falls below its group's window is stored in the
 * planes as the clamp (above) and, in addition, as one exception entry of two
 * 32-bit words:
 *   word 0 = (c << 24) | k   c = n % 16 (row inside its 16-row tile), k < 2^24
 *   word 1 = (beta << 16) | the element's original BF16 word, beta being
 *            the base of the element's group (so an entry alone gives both
 *            the original and the clamp the planes hold)
 * Entries are grouped by block (T, g) -- 16-row tile T = n / 16, group
 * g = k / 128 -- in the order of the blocks in the planes, (T, g) ascending:
 * block t = T*G + g (G = K/128) owns entries offsets[t] .. offsets[t+1]-1
 * (offsets has (Np/16)*G + 1 words, offsets[0] = 0).  Inside a block they
 * follow the order in which the tiled layout stores the weights: piece
 * L = 16*q + c, then dword b, then element e (k = 128*g + 32*b + 8*q + e).
 * With the list, unpack reproduces every element exactly, whatever the
 * input.
 *
 * w12o_exceptions recomputes each group's base from the weights (it does not
 * read a container).  offsets and entries may be NULL (then only the count is
 * returned).  Returns the number of entries, or -1 on bad shape (K must be a
 * multiple of 128 and below 2^24). */
int64_t w12o_exceptions_fmt(int fmt, const uint16_t *w, int64_t N, int64_t K,
                            uint32_t *offsets, uint32_t *entries)
{
    if (N < 0 || K < 0 || K % W12O_GROUP != 0 || K >= ((int64_t)1 << 24))
        return -1;
    int64_t groups = K / W12O_GROUP;
    int64_t ntiles = w12o_padded_rows(N) / 16;
    int64_t count = 0;
    for (int64_t T = 0; T < ntiles; T++) {
        for (int64_t g = 0; g < groups; g++) {
            if (offsets)
                offsets[T * groups + g] = (uint32_t)count;
            int beta[16];
            for (int c = 0; c < 16; c++) {
                int64_t n = 16 * T + c;
                int emax = 0;
                for (int i = 0; n < N && i < W12O_GROUP; i++) {
                    int e = bf16_exponent(w[n * K + g * W12O_GROUP + i]);
                    if (e > emax)
                        emax = e;
                }
                beta[c] = fmt_base_for_emax(fmt, emax);
            }
            for (int L = 0; L < 64; L++) {
                int q = L / 16, c = L % 16;
                int64_t n = 16 * T + c;
                if (n >= N)
                    continue;
                for (int bb = 0; bb < 4; bb++)
                    for (int e = 0; e < 8; e++) {
                        int64_t k = g * W12O_GROUP + 32 * bb + 8 * q + e;
                        uint16_t v = w[n * K + k];
                        if (fmt_encodable(fmt, v, beta[c]))
                            continue;
                        if (entries) {
                            entries[2 * count] = ((uint32_t)c << 24) | (uint32_t)k;
                            entries[2 * count + 1] = ((uint32_t)beta[c] << 16) | v;
                        }
                        count++;
                    }
            }
        }
    }
    if (offsets)
        offsets[ntiles * groups] = (uint32_t)count;
    return count;
}

int64_t w12o_exceptions(const uint16_t *w, int64_t N, int64_t K,
                        uint32_t *offsets, uint32_t *entries)
{
    return w12o_exceptions_fmt(W12O_FMT_V1, w, N, K, offsets, entries);
}

/* Write the exceptions' original words over an unpacked [N, K] weight. */
int w12o_apply_exceptions(uint16_t *w, int64_t N, int64_t K,
                          const uint32_t *offsets, const uint32_t *entries)
{
    if (N < 0 || K < 0 || K % W12O_GROUP != 0)
        return -1;
    int64_t groups = K / W12O_GROUP;
    int64_t blocks = w12o_padded_rows(N) / 16 * groups;
    for (int64_t t = 0; t < blocks; t++)
        for (uint32_t i = offsets[t]; i < offsets[t + 1]; i++) {
            int64_t c = entries[2 * i] >> 24;
            int64_t k = entries[2 * i] & 0xFFFFFF;
            int64_t n = 16 * (t / groups) + c;
            if (n >= N || k >= K || k / W12O_GROUP != t % groups)
                return -1;
            w[n * K + k] = (uint16_t)(entries[2 * i + 1] & 0xFFFF);
        }
    return 0;
}

/* ---- BF16 control layout ----------------------------------------------------
 * Row-major BF16 [N, K] -> the tiled word order of the control GEMM
 * (w12o_padded_rows(N) * K words; padding rows are zero). */
int w12o_bf16_tile(const uint16_t *w, int64_t N, int64_t K, uint16_t *out)
{
    if (N < 0 || K < 0 || K % W12O_GROUP != 0)
        return -1;
    int64_t Np = w12o_padded_rows(N);
    memset(out, 0, (size_t)(Np * K) * sizeof(uint16_t));
    for (int64_t n = 0; n < N; n++) {
        for (int64_t k = 0; k < K; k++) {
            int64_t tile = n / 16, c = n % 16;
            int64_t group = k / W12O_GROUP, r = k % W12O_GROUP;
            int64_t b = r / 32, q = (r % 32) / 8, e = r % 8;
            int64_t block = tile * (K / W12O_GROUP) + group;
            out[block * 2048 + b * 512 + (16 * q + c) * 8 + e] = w[n * K + k];
        }
    }
    return 0;
}

/* ---- fp64 GEMM: y[m][n] = sum_k x[m][k] * w[n][k] ------------------------
 * The plain definition of y = x . W^T.  Each product of two bf16 values is
 * exact in double; the sum runs over k in ascending order; IEEE rules carry
 * NaN and Inf through. */
int w12o_gemm_bf16_f64(const uint16_t *x, int64_t M, int64_t K,
                       const uint16_t *w, int64_t N, double *y)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += bf16_to_double(x[m * K + k]) * bf16_to_double(w[n * K + k]);
            y[m * N + n] = acc;
        }
    return 0;
}

/* ---- decode + fp64 GEMM straight from the packed container --------------
 * The same definition with W read back through w12o_decode one row at a
 * time.  Rows are split evenly over nthreads POSIX threads (this is the
 * CPU baseline that the benchmark times; the arithmetic per output is the
 * same ascending-k fp64 sum as above). */
struct gemm_w12_job {
    int fmt;
    const uint16_t *x;
    const uint8_t *p0, *p1, *p2, *meta;
    int64_t M, N, K, n_begin, n_end;
    double *y;
};

static void *gemm_w12_rows(void *arg)
{
    struct gemm_w12_job *j = (struct gemm_w12_job *)arg;
    for (int64_t n = j->n_begin; n < j->n_end; n++) {
        for (int64_t m = 0; m < j->M; m++) {
            double acc = 0.0;
            for (int64_t k = 0; k < j->K; k++) {
                int beta = fmt_base_of_meta(j->fmt, j->meta[meta_byte(n, j->K, k)]);
                uint16_t code = (uint16_t)((get_nibble(j->p2, n, j->K, k) << 8) |
                                           (get_nibble(j->p1, n, j->K, k) << 4) |
                                           get_nibble(j->p0, n, j->K, k));
                acc += bf16_to_double(j->x[m * j->K + k]) *
                       bf16_to_double(fmt_decode(j->fmt, code, beta));
            }
            j->y[m * j->N + n] = acc;
        }
    }
    return NULL;
}

#define W12O_MAX_THREADS 256

int w12o_gemm_w12_f64_fmt(int fmt, const uint16_t *x, int64_t M, int64_t K,
                          const uint8_t *p0, const uint8_t *p1, const uint8_t *p2,
                          const uint8_t *meta, int64_t N, double *y, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % W12O_GROUP != 0)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > W12O_MAX_THREADS)
        nthreads = W12O_MAX_THREADS;
    if ((int64_t)nthreads > N)
        nthreads = N > 0 ? (int)N : 1;

    struct gemm_w12_job jobs[W12O_MAX_THREADS];
    pthread_t tids[W12O_MAX_THREADS];
    int started[W12O_MAX_THREADS];
    for (int t = 0; t < nthreads; t++) {
        jobs[t].fmt = fmt;
        jobs[t].x = x;
        jobs[t].p0 = p0;
        jobs[t].p1 = p1;
        jobs[t].p2 = p2;
        jobs[t].meta = meta;
        jobs[t].M = M;
        jobs[t].N = N;
        jobs[t].K = K;
        jobs[t].n_begin = N * t / nthreads;
        jobs[t].n_end = N * (t + 1) / nthreads;
        jobs[t].y = y;
        started[t] = 0;
    }
    for (int t = 1; t < nthreads; t++)
        started[t] = pthread_create(&tids[t], NULL, gemm_w12_rows, &jobs[t]) == 0;
    gemm_w12_rows(&jobs[0]);
    for (int t = 1; t < nthreads; t++) {
        if (started[t])
            pthread_join(tids[t], NULL);
        else
            gemm_w12_rows(&jobs[t]);   /* thread creation failed: run inline */
    }
    return 0;
}

int w12o_gemm_w12_f64(const uint16_t *x, int64_t M, int64_t K,
                      const uint8_t *p0, const uint8_t *p1, const uint8_t *p2,
                      const uint8_t *meta, int64_t N, double *y, int nthreads)
{
    return w12o_gemm_w12_f64_fmt(W12O_FMT_V1, x, M, K, p0, p1, p2, meta, N, y, nthreads);
}
