// w12_decode.hpp -- in-register W12 -> BF16 reassembly for gfx950 (both
// bit allocations: W12-v1 and the arbitrary-base W12-b).
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

// ---- W12-b (arbitrary base) ------------------------------------------------
// P0 = m[3:0], P1 = s << 3 | m[6:4], P2 = c; E = c ? b + c : 0 with b the
// group's base (0..240, so b + c <= 255 and no byte carries).  Per dword of
// four weights:
//   sign|mantissa byte        = P1 nibble << 4 | P0 nibble          (v_bfi_b32)
//   E                         = (c + b) & keep, keep = 0xFF unless c == 0
//   high BF16 byte (s|E[7:1]) = bit 7 of the sign|mantissa byte, E >> 1
//   low BF16 byte  (E0|m)     = E << 7 into bit 7, the mantissa below
// keep comes from v_perm_b32, whose selector 12 gives 0x00 and selectors
// 13..255 give 0xFF: c + 12 is 12 exactly when c = 0.  About 26 VALU
// instructions per 8 weights (W12-v1: 16).

__device__ __forceinline__ uint32_t exps_b(uint32_t c, uint32_t b4) {
    const uint32_t keep = perm(0u, 0u, c + 0x0C0C0C0Cu);
    return (c + b4) & keep;
}

// b4 = b * 0x01010101 (the base in every byte).
__device__ __forceinline__ void decode8b(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t b4,
                                         uint32_t out[4]) {
    const uint32_t sm_a = bfi(0xF0F0F0F0u, p1 << 4, p0);   // k0..k3
    const uint32_t sm_b = bfi(0xF0F0F0F0u, p1, p0 >> 4);   // k4..k7
    const uint32_t e_a = exps_b(p2 & 0x0F0F0F0Fu, b4);
    const uint32_t e_b = exps_b((p2 >> 4) & 0x0F0F0F0Fu, b4);
    // E >> 1 and E << 7 spill bits into the neighbouring bytes; the bit
    // inserts keep only the bits of each byte that belong to it
    const uint32_t hi_a = bfi(0x80808080u, sm_a, e_a >> 1);
    const uint32_t hi_b = bfi(0x80808080u, sm_b, e_b >> 1);
    const uint32_t lo_a = bfi(0x80808080u, e_a << 7, sm_a);
    const uint32_t lo_b = bfi(0x80808080u, e_b << 7, sm_b);
    out[0] = perm(hi_a, lo_a, 0x05010400u);
    out[1] = perm(hi_a, lo_a, 0x07030602u);
    out[2] = perm(hi_b, lo_b, 0x05010400u);
    out[3] = perm(hi_b, lo_b, 0x07030602u);
}

}  // namespace w12
