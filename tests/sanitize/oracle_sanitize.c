/*
 * oracle_sanitize.c -- a C driver for the oracle, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/test_oracle_sanitized.py.  Every
 * buffer is a heap block of exactly the size the oracle's documentation
 * gives (padded rows included), so any read or write past it, any signed
 * overflow or any misaligned access stops the run.  Besides running clean,
 * the driver checks the results that do not need a reference: the round trip
 * through the planes plus the exception list restores every input word, the
 * list holds exactly the words the planes cannot, and the container GEMM
 * equals the plain fp64 GEMM of the unpacked weights bit for bit.
 * Test infrastructure only.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t w12o_padded_rows(int64_t N);
int64_t w12o_pack_fmt(int fmt, const uint16_t *w, int64_t N, int64_t K,
                      uint8_t *p0, uint8_t *p1, uint8_t *p2, uint8_t *meta);
int w12o_unpack_fmt(int fmt, const uint8_t *p0, const uint8_t *p1, const uint8_t *p2,
                    const uint8_t *meta, int64_t N, int64_t K, uint16_t *w);
int64_t w12o_exceptions_fmt(int fmt, const uint16_t *w, int64_t N, int64_t K,
                            uint32_t *offsets, uint32_t *entries);
int w12o_apply_exceptions(uint16_t *w, int64_t N, int64_t K,
                          const uint32_t *offsets, const uint32_t *entries);
int w12o_bf16_tile(const uint16_t *w, int64_t N, int64_t K, uint16_t *out);
int w12o_gemm_bf16_f64(const uint16_t *x, int64_t M, int64_t K,
                       const uint16_t *w, int64_t N, double *y);
int w12o_gemm_w12_f64_fmt(int fmt, const uint16_t *x, int64_t M, int64_t K,
                          const uint8_t *p0, const uint8_t *p1, const uint8_t *p2,
                          const uint8_t *meta, int64_t N, double *y, int nthreads);
uint16_t w12o_encode(uint16_t v, int beta, int *ok);
uint16_t w12o_decode(uint16_t code, int beta);
uint16_t w12o_b_encode(uint16_t v, int b, int *ok);
uint16_t w12o_b_decode(uint16_t code, int b);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);          \
            fprintf(stderr, __VA_ARGS__);                                 \
            fprintf(stderr, "\n");                                        \
            exit(1);                                                      \
        }                                                                 \
    } while (0)

/* Weights: small Gaussian-like words (sum of uniforms, exponent near 120)
 * mixed with arbitrary 16-bit words, so both clean and flagged groups occur. */
static uint16_t weight_word(int mode)
{
    uint32_t r = next_u32();
    if (mode == 1 || (r & 15) == 0)
        return (uint16_t)(next_u32() & 0xFFFF);
    int e = 110 + (int)(next_u32() % 14);
    return (uint16_t)(((r >> 16) & 1) << 15 | (uint32_t)e << 7 | (r & 0x7F));
}

static void one_shape(int fmt, int64_t N, int64_t K, int64_t M, int mode)
{
    const int64_t Np = w12o_padded_rows(N);
    const size_t plane = (size_t)(Np * K / 2), metab = (size_t)(Np * K / 128);
    uint16_t *w = xmalloc((size_t)(N * K) * 2);
    for (int64_t i = 0; i < N * K; i++)
        w[i] = weight_word(mode);
    uint8_t *p0 = xmalloc(plane), *p1 = xmalloc(plane), *p2 = xmalloc(plane);
    uint8_t *meta = xmalloc(metab);
    int64_t bad = w12o_pack_fmt(fmt, w, N, K, p0, p1, p2, meta);
    CHECK(bad >= 0, "pack rejected N=%ld K=%ld", (long)N, (long)K);

    uint16_t *back = xmalloc((size_t)(N * K) * 2);
    CHECK(w12o_unpack_fmt(fmt, p0, p1, p2, meta, N, K, back) == 0, "unpack");
    int64_t differ = 0;
    for (int64_t i = 0; i < N * K; i++)
        differ += back[i] != w[i];

    int64_t count = w12o_exceptions_fmt(fmt, w, N, K, NULL, NULL);
    CHECK(count == differ, "list counts %ld entries, the planes lose %ld words", (long)count,
          (long)differ);
    CHECK((count > 0) == (bad > 0), "flagged groups %ld but %ld entries", (long)bad, (long)count);
    const int64_t blocks = Np / 16 * (K / 128);
    uint32_t *off = xmalloc((size_t)(blocks + 1) * 4);
    uint32_t *ent = xmalloc((size_t)count * 8);
    CHECK(w12o_exceptions_fmt(fmt, w, N, K, off, ent) == count, "list count changed");
    CHECK(off[blocks] == (uint32_t)count, "last offset");
    CHECK(w12o_apply_exceptions(back, N, K, off, ent) == 0, "apply");
    CHECK(memcmp(back, w, (size_t)(N * K) * 2) == 0, "planes + list do not restore the input");

    uint16_t *tiled = xmalloc((size_t)(Np * K) * 2);
    CHECK(w12o_bf16_tile(w, N, K, tiled) == 0, "tile");

    /* container GEMM == plain GEMM of the unpacked (clamped) weights */
    uint16_t *clamped = xmalloc((size_t)(N * K) * 2);
    CHECK(w12o_unpack_fmt(fmt, p0, p1, p2, meta, N, K, clamped) == 0, "unpack");
    uint16_t *x = xmalloc((size_t)(M * K) * 2);
    for (int64_t i = 0; i < M * K; i++)
        x[i] = weight_word(0);
    double *y1 = xmalloc((size_t)(M * N) * 8), *y2 = xmalloc((size_t)(M * N) * 8);
    CHECK(w12o_gemm_bf16_f64(x, M, K, clamped, N, y1) == 0, "gemm");
    CHECK(w12o_gemm_w12_f64_fmt(fmt, x, M, K, p0, p1, p2, meta, N, y2, 3) == 0, "gemm w12");
    /* bit for bit, except that NaN payloads may differ: with two NaN operands
     * an addition returns either one, as the compiler orders them */
    for (int64_t i = 0; i < M * N; i++) {
        if (y1[i] != y1[i])
            CHECK(y2[i] != y2[i], "container GEMM lost a NaN at %ld", (long)i);
        else
            CHECK(memcmp(&y1[i], &y2[i], 8) == 0, "container GEMM != plain GEMM at %ld",
                  (long)i);
    }

    free(w); free(p0); free(p1); free(p2); free(meta); free(back); free(off); free(ent);
    free(tiled); free(clamped); free(x); free(y1); free(y2);
}

int main(void)
{
    /* element codec: every BF16 word for a few bases of each format */
    static const int betas[] = {0, 1, 59, 119, 120};
    for (unsigned bi = 0; bi < sizeof betas / sizeof betas[0]; bi++)
        for (uint32_t v = 0; v < 65536; v++) {
            int ok;
            uint16_t c = w12o_encode((uint16_t)v, betas[bi], &ok);
            CHECK(c < 4096, "code range");
            if (ok)
                CHECK(w12o_decode(c, betas[bi]) == v, "v1 round trip");
        }
    static const int bases[] = {0, 1, 120, 239, 240};
    for (unsigned bi = 0; bi < sizeof bases / sizeof bases[0]; bi++)
        for (uint32_t v = 0; v < 65536; v++) {
            int ok;
            uint16_t c = w12o_b_encode((uint16_t)v, bases[bi], &ok);
            CHECK(c < 4096, "code range b");
            if (ok)
                CHECK(w12o_b_decode(c, bases[bi]) == v, "b round trip");
        }

    static const int64_t shapes[][3] = {
        {1, 128, 1}, {15, 128, 2}, {16, 256, 1}, {17, 384, 3}, {33, 1152, 2}, {48, 640, 5},
    };
    for (int fmt = 0; fmt < 2; fmt++)
        for (unsigned s = 0; s < sizeof shapes / sizeof shapes[0]; s++)
            for (int mode = 0; mode < 2; mode++)
                one_shape(fmt, shapes[s][0], shapes[s][1], shapes[s][2], mode);
    printf("oracle sanitize ok\n");
    return 0;
}
