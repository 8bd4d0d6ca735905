// w12_gemm.hip -- small-M decode GEMM y = x . W^T for gfx950, with W fetched
// either from a W12 container (rebuilt to BF16 in registers) or as plain BF16.
//
// The pages: in single-request decoding every step reads all target weights
// while only a few tokens are accepted, and kernels are tuned against the
// memory-bandwidth limit (AI Radar summary of SpecPilot, English edition,
// opening paragraph); W12 is rebuilt bit-exactly inside the GEMM at batch
// 1-32 (HotRepo digest of StargazerX0/SpecPilot, project introduction).  So
// the kernel is a weight stream: 1.5 B per weight for W12, 2 B for BF16, with
// x small enough to sit in LDS.
//
// Shared structure (both variants, both weight fetches):
//   * a workgroup = 4 waves owns a block of rows and the whole K range; KW of
//     its waves split K between them (step s goes to K-wave s % KW) and add
//     their partial sums through LDS in a fixed order at the end;
//   * x is staged through LDS in chunks of KC columns, double-buffered: the
//     next chunk is loaded into registers while the current one is used, and
//     one barrier per chunk publishes it;
//   * the weight fetch for step s+KW is issued before step s is computed, so
//     one step of 128-bit loads per row is always in flight;
//   * GEMV (M <= 8): 16 lanes per row, each lane 32 consecutive weights per
//     step (three 16-byte plane loads), R rows per lane so the x values read
//     from LDS are reused R times; v_dot2c_f32_bf16 accumulates in fp32; the
//     16 partial sums of a row are added with a fixed xor-butterfly.
//   * MFMA (M <= 32): v_mfma_f32_16x16x32_bf16.  A wave step covers 16 rows x
//     128 K (one W12 group per row).  Lane (col, q) loads 32 weights of row
//     col at K offset 32q; its 8-weight block i is the B fragment of MFMA i,
//     so MFMA i contracts the K set {32q + 8i + e}.  The A fragment (x) is
//     read from LDS with the same permutation, so the four MFMAs of a step
//     cover the group exactly once.
// The W12 and BF16 fetches produce identical B operands in identical order,
// so for W = unpack(pack(W)) both kernels return bitwise equal y.
#include "w12_decode.hpp"
#include "w12_internal.hpp"

namespace w12 {
namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
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

// ---- weight fetch policies --------------------------------------------------
// load(): the 32 consecutive weights of row n starting at k0 (k0 % 32 == 0),
// as raw registers; block(): 8-weight block b (0..3) as 4 dwords of BF16
// pairs in natural k order.

struct FetchW12 {
    struct Raw {
        uint4 a, b, c;
        uint32_t beta;
    };
    __device__ __forceinline__ static void load(const GemmArgs& g, int64_t n, int64_t k0, Raw& r) {
        const int64_t off = (n * g.K + k0) >> 1;  // byte offset, 16-byte aligned
        r.a = *reinterpret_cast<const uint4*>(g.p0 + off);
        r.b = *reinterpret_cast<const uint4*>(g.p1 + off);
        r.c = *reinterpret_cast<const uint4*>(g.p2 + off);
        r.beta = g.meta[(n * g.K + k0) >> 7] & 0x7Fu;
    }
    __device__ __forceinline__ static void zero(Raw& r) {
        r.a = r.b = r.c = make_uint4(0, 0, 0, 0);
        r.beta = 0;
    }
    __device__ __forceinline__ static void block(const Raw& r, int b, uint32_t out[4]) {
        const Lut t = make_lut(r.beta);
        const uint32_t pa = b == 0 ? r.a.x : b == 1 ? r.a.y : b == 2 ? r.a.z : r.a.w;
        const uint32_t pb = b == 0 ? r.b.x : b == 1 ? r.b.y : b == 2 ? r.b.z : r.b.w;
        const uint32_t pc = b == 0 ? r.c.x : b == 1 ? r.c.y : b == 2 ? r.c.z : r.c.w;
        decode8(pa, pb, pc, t, out);
    }
};

struct FetchBF16 {
    struct Raw {
        uint4 q[4];
    };
    __device__ __forceinline__ static void load(const GemmArgs& g, int64_t n, int64_t k0, Raw& r) {
        const uint4* p = reinterpret_cast<const uint4*>(g.w + n * g.K + k0);
#pragma unroll
        for (int b = 0; b < 4; ++b) r.q[b] = p[b];
    }
    __device__ __forceinline__ static void zero(Raw& r) {
#pragma unroll
        for (int b = 0; b < 4; ++b) r.q[b] = make_uint4(0, 0, 0, 0);
    }
    __device__ __forceinline__ static void block(const Raw& r, int b, uint32_t out[4]) {
        out[0] = r.q[b].x;
        out[1] = r.q[b].y;
        out[2] = r.q[b].z;
        out[3] = r.q[b].w;
    }
};

// ---- x staging ----------------------------------------------------------------
// Copy x[0:MROWS][k0:k0+KC] into an LDS buffer in 16-byte units (8 BF16).
// Rows >= M and columns >= K are zero.  phys() maps (row, unit) to the LDS
// slot; the two layouts below spread the units a wave reads at once over
// distinct 16-byte bank groups.
template <int MROWS, int KC>
struct XStage {
    static constexpr int kUnitsPerRow = KC / 8;
    static constexpr int kPerThread = MROWS * kUnitsPerRow / kThreads;
    static_assert(MROWS * kUnitsPerRow % kThreads == 0, "x chunk must split evenly");
    uint4 v[kPerThread];

    __device__ __forceinline__ void load(const GemmArgs& g, int64_t k0) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int id = threadIdx.x + kThreads * j;
            const int m = id / kUnitsPerRow;
            const int64_t k = k0 + 8 * (id % kUnitsPerRow);
            if (m < g.M && k < g.K)
                v[j] = *reinterpret_cast<const uint4*>(g.x + (int64_t)m * g.ldx + k);
            else
                v[j] = make_uint4(0, 0, 0, 0);
        }
    }
    template <class Layout>
    __device__ __forceinline__ void store(uint4* buf) const {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int id = threadIdx.x + kThreads * j;
            buf[Layout::phys(id / kUnitsPerRow, id % kUnitsPerRow)] = v[j];
        }
    }
};

// GEMV reads, per instruction, unit 4t + b of its row for lanes t = 0..15;
// xor-ing the unit's low two bits with bits 3..4 makes lanes 0..7 land in
// 8 different 16-byte slots of a 128-byte bank row.
template <int KC>
struct GemvLayout {
    __device__ __forceinline__ static int phys(int m, int u) {
        return m * (KC / 8) + (u ^ ((u >> 3) & 3));
    }
};

// MFMA reads, per instruction, the same unit of rows m = 0..15; xor-ing the
// unit with m & 7 gives those rows 8 different slots.
template <int KC>
struct MfmaLayout {
    __device__ __forceinline__ static int phys(int m, int u) {
        return m * (KC / 8) + (u ^ (m & 7));
    }
};

// ---- GEMV: M <= 8 ---------------------------------------------------------------

constexpr int kGemvKC = 2048;  // x columns per LDS chunk

template <class F, int M, int R, int KW>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemmArgs g) {
    constexpr int KC = kGemvKC;
    constexpr int kStep = 512;             // K per wave step (16 lanes x 32)
    constexpr int kStepsPerChunk = KC / kStep;
    static_assert(kStepsPerChunk % KW == 0, "chunk must split over the K-waves");
    constexpr int kRowsPerWave = 4 * R;
    constexpr int kRowWaves = 4 / KW;
    constexpr int BN = kRowWaves * kRowsPerWave;
    using Layout = GemvLayout<KC>;
    extern __shared__ uint4 lds[];
    constexpr int kBuf = M * (KC / 8);  // uint4 per x buffer

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4;
    const int t = lane & 15;
    const int kw = wave % KW;
    const int nw = wave / KW;
    const int64_t row0 = (int64_t)blockIdx.x * BN + nw * kRowsPerWave + grp;  // row r: row0 + 4r

    const int64_t nsteps = (g.K + kStep - 1) / kStep;
    const int64_t nchunks = (g.K + KC - 1) / KC;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

    typename F::Raw cur[R], nxt[R];
    auto fetch = [&](int64_t s, typename F::Raw* dst) {
        const int64_t k0 = s * kStep + 32 * t;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = row0 + 4 * r;
            if (n < g.N && k0 < g.K)
                F::load(g, n, k0, dst[r]);
            else
                F::zero(dst[r]);
        }
    };

    int64_t s = kw;
    if (s < nsteps) fetch(s, cur);
    {
        XStage<M, KC> xs;
        xs.load(g, 0);
        xs.template store<Layout>(lds);
    }
    __syncthreads();

    for (int64_t c = 0; c < nchunks; ++c) {
        XStage<M, KC> xs;
        const bool more = c + 1 < nchunks;
        if (more) xs.load(g, (c + 1) * KC);
        const uint4* xb = lds + (c & 1) * kBuf;
        const int64_t s_end = (c + 1) * kStepsPerChunk < nsteps ? (c + 1) * kStepsPerChunk : nsteps;
        for (; s < s_end; s += KW) {
            if (s + KW < nsteps) fetch(s + KW, nxt);
            const int ls = (int)(s - c * kStepsPerChunk);
            if (s * kStep + 32 * t < g.K) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    uint4 xv[M];
#pragma unroll
                    for (int m = 0; m < M; ++m) xv[m] = xb[Layout::phys(m, ls * 64 + 4 * t + b)];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        uint32_t wv[4];
                        F::block(cur[r], b, wv);
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            float a = acc[r][m];
                            a = dot2(wv[0], xv[m].x, a);
                            a = dot2(wv[1], xv[m].y, a);
                            a = dot2(wv[2], xv[m].z, a);
                            a = dot2(wv[3], xv[m].w, a);
                            acc[r][m] = a;
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) cur[r] = nxt[r];
        }
        if (more) xs.template store<Layout>(lds + ((c + 1) & 1) * kBuf);
        __syncthreads();
    }

    // Sum the 16 lanes of each row group (fixed butterfly order).
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float v = acc[r][m];
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 1);
            acc[r][m] = v;
        }

    if constexpr (KW > 1) {
        // K-waves 1..KW-1 hand their row sums to K-wave 0 through LDS
        // (the x buffers are free after the last barrier).
        float* red = reinterpret_cast<float*>(lds);
        if (kw > 0 && t == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m)
                    red[(((kw - 1) * kRowWaves + nw) * 4 + grp) * (R * M) + r * M + m] = acc[r][m];
        }
        __syncthreads();
        if (kw != 0) return;
        if (t == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float v = acc[r][m];
                    for (int j = 1; j < KW; ++j)
                        v += red[(((j - 1) * kRowWaves + nw) * 4 + grp) * (R * M) + r * M + m];
                    acc[r][m] = v;
                }
        }
        // broadcast the finished sums from lane t == 0 of the group
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = __shfl(acc[r][m], grp * 16);
    }

    // Lane t of the group stores the (r, m) outputs with (r*M + m) % 16 == t.
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = row0 + 4 * r;
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (((r * M + m) & 15) == t && n < g.N && m < g.M) store_y(g, m, n, acc[r][m]);
    }
}

// ---- MFMA: 9 <= M <= 32 ------------------------------------------------------------

template <int MT>
struct MfmaKC {
    static constexpr int value = MT == 16 ? 1024 : 512;  // 64 KB of LDS double-buffered
};

template <class F, int MT, int R, int KW>
__global__ __launch_bounds__(kThreads) void mfma_kernel(GemmArgs g) {
    constexpr int KC = MfmaKC<MT>::value;
    constexpr int kStep = 128;
    constexpr int kStepsPerChunk = KC / kStep;
    static_assert(kStepsPerChunk % KW == 0, "chunk must split over the K-waves");
    constexpr int kMT = MT / 16;           // 16-row tiles of x
    constexpr int kRowWaves = 4 / KW;
    constexpr int BN = kRowWaves * 16 * R;
    using Layout = MfmaLayout<KC>;
    extern __shared__ uint4 lds[];
    constexpr int kBuf = MT * (KC / 8);  // uint4 per x buffer

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;   // B column (weight row in the tile) and A row
    const int q = lane >> 4;     // K quarter of the step
    const int kw = wave % KW;
    const int nw = wave / KW;
    const int64_t row0 = (int64_t)blockIdx.x * BN + nw * 16 * R + col;  // tile r: row0 + 16r

    const int64_t nsteps = g.K / kStep;
    const int64_t nchunks = (g.K + KC - 1) / KC;

    f32x4_t acc[R][kMT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < kMT; ++i) acc[r][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    typename F::Raw cur[R], nxt[R];
    auto fetch = [&](int64_t s, typename F::Raw* dst) {
        const int64_t k0 = s * kStep + 32 * q;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = row0 + 16 * r;
            if (n < g.N)
                F::load(g, n, k0, dst[r]);
            else
                F::zero(dst[r]);
        }
    };

    int64_t s = kw;
    if (s < nsteps) fetch(s, cur);
    {
        XStage<MT, KC> xs;
        xs.load(g, 0);
        xs.template store<Layout>(lds);
    }
    __syncthreads();

    for (int64_t c = 0; c < nchunks; ++c) {
        XStage<MT, KC> xs;
        const bool more = c + 1 < nchunks;
        if (more) xs.load(g, (c + 1) * KC);
        const uint4* xb = lds + (c & 1) * kBuf;
        const int64_t s_end = (c + 1) * kStepsPerChunk < nsteps ? (c + 1) * kStepsPerChunk : nsteps;
        for (; s < s_end; s += KW) {
            if (s + KW < nsteps) fetch(s + KW, nxt);
            const int ls = (int)(s - c * kStepsPerChunk);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x8_t a[kMT];
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
                    a[mt] = __builtin_bit_cast(bf16x8_t,
                                               xb[Layout::phys(16 * mt + col, ls * 16 + 4 * q + i)]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    uint32_t wv[4];
                    F::block(cur[r], i, wv);
                    const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, make_uint4(wv[0], wv[1], wv[2], wv[3]));
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt)
                        acc[r][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], bw, acc[r][mt], 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) cur[r] = nxt[r];
        }
        if (more) xs.template store<Layout>(lds + ((c + 1) & 1) * kBuf);
        __syncthreads();
    }

    if constexpr (KW > 1) {
        f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);
        constexpr int kPer = R * kMT;  // f32x4 per lane
        if (kw > 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
                    red[(((kw - 1) * kRowWaves + nw) * 64 + lane) * kPer + r * kMT + mt] = acc[r][mt];
        }
        __syncthreads();
        if (kw != 0) return;
        for (int j = 1; j < KW; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
                    acc[r][mt] += red[(((j - 1) * kRowWaves + nw) * 64 + lane) * kPer + r * kMT + mt];
    }

    // D layout of the 16x16 MFMA: lane (col, q) holds rows 4q..4q+3 of
    // column col, i.e. y[m = 16 mt + 4q + e][n = tile row col].
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = row0 + 16 * r;
        if (n >= g.N) continue;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 16 * mt + 4 * q + e;
                if (m < g.M) store_y(g, m, n, acc[r][mt][e]);
            }
    }
}

// ---- dispatch ---------------------------------------------------------------------

template <class F, int M, int R>
hipError_t launch_gemv_kw(const GemmArgs& a, int kw, hipStream_t s) {
    const size_t lds = 2 * (size_t)M * kGemvKC * 2;
    auto grid = [&](int KW) { return dim3((unsigned)((a.N + (4 / KW) * 4 * R - 1) / ((4 / KW) * 4 * R))); };
    switch (kw) {
        case 1: hipLaunchKernelGGL((gemv_kernel<F, M, R, 1>), grid(1), dim3(kThreads), lds, s, a); break;
        case 2: hipLaunchKernelGGL((gemv_kernel<F, M, R, 2>), grid(2), dim3(kThreads), lds, s, a); break;
        case 4: hipLaunchKernelGGL((gemv_kernel<F, M, R, 4>), grid(4), dim3(kThreads), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class F, int M>
hipError_t launch_gemv_r(const GemmArgs& a, int r, int kw, hipStream_t s) {
    switch (r) {
        case 1: return launch_gemv_kw<F, M, 1>(a, kw, s);
        case 2: return launch_gemv_kw<F, M, 2>(a, kw, s);
        case 4: return launch_gemv_kw<F, M, 4>(a, kw, s);
        default: return hipErrorInvalidValue;
    }
}

template <class F>
hipError_t launch_gemv(const GemmArgs& a, const Tiling& t, hipStream_t s) {
    switch (t.mt) {
        case 1: return launch_gemv_r<F, 1>(a, t.r, t.kw, s);
        case 2: return launch_gemv_r<F, 2>(a, t.r, t.kw, s);
        case 3: return launch_gemv_r<F, 3>(a, t.r, t.kw, s);
        case 4: return launch_gemv_r<F, 4>(a, t.r, t.kw, s);
        case 5: return launch_gemv_r<F, 5>(a, t.r, t.kw, s);
        case 6: return launch_gemv_r<F, 6>(a, t.r, t.kw, s);
        case 7: return launch_gemv_r<F, 7>(a, t.r, t.kw, s);
        case 8: return launch_gemv_r<F, 8>(a, t.r, t.kw, s);
        default: return hipErrorInvalidValue;
    }
}

template <class F, int MT, int R>
hipError_t launch_mfma_kw(const GemmArgs& a, int kw, hipStream_t s) {
    const size_t lds = 2 * (size_t)MT * MfmaKC<MT>::value * 2;
    auto grid = [&](int KW) { return dim3((unsigned)((a.N + (4 / KW) * 16 * R - 1) / ((4 / KW) * 16 * R))); };
    switch (kw) {
        case 1: hipLaunchKernelGGL((mfma_kernel<F, MT, R, 1>), grid(1), dim3(kThreads), lds, s, a); break;
        case 2: hipLaunchKernelGGL((mfma_kernel<F, MT, R, 2>), grid(2), dim3(kThreads), lds, s, a); break;
        case 4: hipLaunchKernelGGL((mfma_kernel<F, MT, R, 4>), grid(4), dim3(kThreads), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class F, int MT>
hipError_t launch_mfma_r(const GemmArgs& a, int r, int kw, hipStream_t s) {
    switch (r) {
        case 1: return launch_mfma_kw<F, MT, 1>(a, kw, s);
        case 2: return launch_mfma_kw<F, MT, 2>(a, kw, s);
        default: return hipErrorInvalidValue;
    }
}

template <class F>
hipError_t launch_mfma(const GemmArgs& a, const Tiling& t, hipStream_t s) {
    switch (t.mt) {
        case 16: return launch_mfma_r<F, 16>(a, t.r, t.kw, s);
        case 32: return launch_mfma_r<F, 32>(a, t.r, t.kw, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool tiling_valid(const Tiling& t, int M) {
    if (t.kw != 1 && t.kw != 2 && t.kw != 4) return false;
    if (t.mfma) {
        if (t.mt != 16 && t.mt != 32) return false;
        if (M > t.mt) return false;
        return t.r == 1 || t.r == 2;
    }
    if (t.mt != M || M < 1 || M > 8) return false;
    return t.r == 1 || t.r == 2 || t.r == 4;
}

Tiling choose_tiling(int M, int64_t N, int64_t K) {
    (void)K;
    Tiling t;
    if (M <= 8) {
        t.mfma = 0;
        t.mt = M;
        t.r = M <= 2 ? 1 : (M <= 4 ? 2 : 4);
        // Enough waves to keep ~8 per CU streaming: split K inside the
        // workgroup when the row count alone gives too few.
        t.kw = 1;
        while (t.kw < 4 && ((N + 4 * t.r - 1) / (4 * t.r)) * t.kw < 2048) t.kw *= 2;
    } else {
        t.mfma = 1;
        t.mt = M <= 16 ? 16 : 32;
        t.r = 1;
        t.kw = 1;
        while (t.kw < 4 && ((N + 16 * t.r - 1) / (16 * t.r)) * t.kw < 2048) t.kw *= 2;
    }
    return t;
}

const char* tiling_name(const Tiling& t, bool is_w12) {
    // A fixed table of names so the pointer stays valid.
    static const char* const gemv_names[2][8][3][3] = {
#define W12_N3(F, M, R) {F "_gemv_m" #M "_r" #R "_kw1", F "_gemv_m" #M "_r" #R "_kw2", F "_gemv_m" #M "_r" #R "_kw4"}
#define W12_NM(F, M) {W12_N3(F, M, 1), W12_N3(F, M, 2), W12_N3(F, M, 4)}
        {W12_NM("bf16", 1), W12_NM("bf16", 2), W12_NM("bf16", 3), W12_NM("bf16", 4),
         W12_NM("bf16", 5), W12_NM("bf16", 6), W12_NM("bf16", 7), W12_NM("bf16", 8)},
        {W12_NM("w12", 1), W12_NM("w12", 2), W12_NM("w12", 3), W12_NM("w12", 4),
         W12_NM("w12", 5), W12_NM("w12", 6), W12_NM("w12", 7), W12_NM("w12", 8)},
#undef W12_NM
#undef W12_N3
    };
    static const char* const mfma_names[2][2][2][3] = {
#define W12_N3(F, MT, R) {F "_mfma_mt" #MT "_r" #R "_kw1", F "_mfma_mt" #MT "_r" #R "_kw2", F "_mfma_mt" #MT "_r" #R "_kw4"}
        {{W12_N3("bf16", 16, 1), W12_N3("bf16", 16, 2)}, {W12_N3("bf16", 32, 1), W12_N3("bf16", 32, 2)}},
        {{W12_N3("w12", 16, 1), W12_N3("w12", 16, 2)}, {W12_N3("w12", 32, 1), W12_N3("w12", 32, 2)}},
#undef W12_N3
    };
    const int kwi = t.kw == 1 ? 0 : t.kw == 2 ? 1 : 2;
    if (t.mfma) return mfma_names[is_w12][t.mt == 32][t.r - 1][kwi];
    const int ri = t.r == 1 ? 0 : t.r == 2 ? 1 : 2;
    return gemv_names[is_w12][t.mt - 1][ri][kwi];
}

hipError_t launch_gemm(const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s) {
    if (t.mfma) return is_w12 ? launch_mfma<FetchW12>(a, t, s) : launch_mfma<FetchBF16>(a, t, s);
    return is_w12 ? launch_gemv<FetchW12>(a, t, s) : launch_gemv<FetchBF16>(a, t, s);
}

}  // namespace w12
