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
//   mfma = 0: GEMV; every 16 lanes own a row, R rows per lane group.
//   mfma = 1: MFMA 16x16x32 bf16; a wave owns R tiles of 16 rows.
//   kw   = waves of a workgroup that split K between them (1, 2 or 4).
struct Tiling {
    int mfma;
    int mt;   // GEMV: M; MFMA: padded M (16 or 32)
    int r;
    int kw;
};

// Pick the tiling used by w12_gemm / bf16_gemm for this shape.
Tiling choose_tiling(int M, int64_t N, int64_t K);
bool tiling_valid(const Tiling& t, int M);
const char* tiling_name(const Tiling& t, bool is_w12);

hipError_t launch_gemm(const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s);
hipError_t launch_pack(const uint16_t* w, int64_t N, int64_t K, void* p0, void* p1,
                       void* p2, uint8_t* meta, uint32_t* bad, hipStream_t s);
hipError_t launch_unpack(const void* p0, const void* p1, const void* p2,
                         const uint8_t* meta, int64_t N, int64_t K, uint16_t* w,
                         hipStream_t s);

}  // namespace w12
