// w12_internal.hpp -- launch helpers shared by the kernel files and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

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
    const uint16_t* w;
    int64_t N;
    int64_t K;
    void* y;
    int64_t ldy;
    int y_f32;
};

// Tiling of one GEMM launch.
//   mfma    = 0: GEMV (v_dot2c_f32_bf16); 1: MFMA 16x16x32 bf16.
//   r       = 16-row weight tiles per wave (1 or 2).
//   mt      = GEMV: M (1..8); MFMA: x rows padded to 16 or 32.
//   kw      = waves of a workgroup that split K between them (1, 2 or 4).
//   depth   = 32-weight slices each lane keeps in flight (2, 4 or 8).
//   xdirect = 1: GEMV only, M <= 4: x is read by each lane with its weights
//             instead of being staged in LDS.
//   chunked = 0 if all of x is staged in LDS at once, 1 if it is streamed
//             through LDS in double-buffered chunks (set from the shape).
struct Tiling {
    int mfma;
    int mt;
    int r;
    int kw;
    int depth;
    int xdirect;
    int chunked;
};

// Pick the tiling used by w12_gemm / bf16_gemm for this shape.
Tiling choose_tiling(int M, int64_t N, int64_t K);
// Complete a caller-given tiling (mt, chunked) for this shape; false if the
// combination is not built.
bool complete_tiling(Tiling& t, int M, int64_t K);
const char* tiling_name(const Tiling& t, bool is_w12);

hipError_t launch_gemm(const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s);
// Per-M (GEMV) and per-MT (MFMA) launchers, one object file each.
hipError_t launch_gemv_m(int M, const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s);
hipError_t launch_mfma_mt(int MT, const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s);
hipError_t launch_pack(const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1,
                       void* p2, uint8_t* meta, uint32_t* bad, hipStream_t s);
hipError_t launch_unpack(const void* p0, const void* p1, const void* p2,
                         const uint8_t* meta, int64_t N, int64_t K, uint16_t* w,
                         hipStream_t s);
hipError_t launch_bf16_tile(const uint16_t* w, int64_t N, int64_t K, uint16_t* out, hipStream_t s);

}  // namespace w12
