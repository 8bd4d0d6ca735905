// w12_decode.hpp -- in-register W12-v1 -> BF16 reassembly for gfx950.
//
// The pages describe W12 as BF16 split into three 4-bit planes and rebuilt
// bit by bit in GEMM registers (AI Radar summary of SpecPilot, English
// edition, "Reasons"; HotRepo digest of StargazerX0/SpecPilot, project
// introduction).  The layout decoded here is W12-v1 (declared in w12.h).
//
// One dword from each plane holds the same 8 consecutive weights k0..k7 in
// split-nibble order: byte j carries k = j in its low nibble and k = j+4 in
// its high nibble.  The decode works on all four bytes of a dword at once:
//
//   low BF16 byte  (E0 | m)       = P1 nibble << 4 | P0 nibble     (v_bfi_b32)
//   high BF16 byte (s | E[7:1])   = s << 7 | table[h]              (v_perm_b32)
//
// where table[0] = 0 and table[h] = beta + h for h = 1..7 is an 8-byte table
// held in two dwords (built once per 128-weight group).  v_perm_b32 picks,
// for each selector byte 0..7, byte (sel) of the 64-bit value {hi:lo}, so a
// 3-bit h is a table index directly.  Two more v_perm_b32 per output dword
// interleave low and high bytes into BF16 pairs in natural k order, which is
// the operand layout of both v_dot2c_f32_bf16 and the MFMA B fragment.
// About 16 VALU instructions per 8 weights; integer only, so every bit
// (signed zeros, subnormals, Inf, NaN payloads) passes through unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

// The 8-entry high-byte table for base beta (0 <= beta <= 120, so
// beta + 7 <= 127 and no entry carries into the sign bit).
struct Lut {
    uint32_t lo;  // bytes: 0, beta+1, beta+2, beta+3
    uint32_t hi;  // bytes: beta+4, beta+5, beta+6, beta+7
};

__device__ __forceinline__ Lut make_lut(uint32_t beta) {
    const uint32_t b4 = beta * 0x01010101u;
    Lut t;
    t.lo = (b4 + 0x03020100u) & 0xFFFFFF00u;
    t.hi = b4 + 0x07060504u;
    return t;
}

// v_perm_b32: result byte i = byte sel.i of the 64-bit value {a : b}
// (selector 0..3 -> b, 4..7 -> a).
__device__ __forceinline__ uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) {
    return __builtin_amdgcn_perm(a, b, sel);
}

// v_bfi_b32: (a & mask) | (b & ~mask)
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
    return (a & mask) | (b & ~mask);
}

// Decode 8 weights (one dword per plane) into 4 dwords of BF16 pairs:
// out[i] = bf16(k = 2i) | bf16(k = 2i + 1) << 16.
__device__ __forceinline__ void decode8(uint32_t p0, uint32_t p1, uint32_t p2,
                                        const Lut& t, uint32_t out[4]) {
    // low bytes of the BF16 words: k0..k3 and k4..k7
    const uint32_t lo_a = bfi(0xF0F0F0F0u, p1 << 4, p0);
    const uint32_t lo_b = bfi(0xF0F0F0F0u, p1, p0 >> 4);
    // exponent high bits through the table, then the sign bit
    const uint32_t x_a = perm(t.hi, t.lo, p2 & 0x07070707u);
    const uint32_t x_b = perm(t.hi, t.lo, (p2 >> 4) & 0x07070707u);
    const uint32_t hi_a = ((p2 << 4) & 0x80808080u) | x_a;
    const uint32_t hi_b = (p2 & 0x80808080u) | x_b;
    // interleave {hi, lo} byte pairs into BF16 pairs
    out[0] = perm(hi_a, lo_a, 0x05010400u);
    out[1] = perm(hi_a, lo_a, 0x07030602u);
    out[2] = perm(hi_b, lo_b, 0x05010400u);
    out[3] = perm(hi_b, lo_b, 0x07030602u);
}

}  // namespace w12
