// The int4 -> int8 code arithmetic of the grouped W4A8 decode, shared by the
// fused kernels ("[PR #97] HIP port of #90: grouped W4A8 over the INT8
// GEMM", What this adds: int4 codes with per-group scales become int8 codes
// against one scale per row):
//   w8 = clamp(rint(val(u) * mult), -127, 127),  mult = s[row, g] / s_row
// formed with the same fp32 operations as w4a8_decode_kernel, so every path
// that uses these helpers gives its int8 codes bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"

namespace ck4 {
namespace {

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// The int8 code of one int4 code: clamp(rint(q * mult), -127, 127), as a bit
// pattern whose low byte is the code. f = q + 8 (from the XOR-biased nibble)
// and m8 = -8 * mult, which is exact, so fma(f, mult, m8) is the single
// rounding of q * mult: the same fp32 value the decode kernel computes.
// The clamp before rounding equals the clamp after (the bounds are integers),
// and adding 1.5 * 2^23 rounds to the nearest integer, ties to even.
__device__ __forceinline__ uint32_t code8(float f, float mult, float m8) {
    float x = __builtin_fmaf(f, mult, m8);
    x = fminf(fmaxf(x, -127.0f), 127.0f);
    return __float_as_uint(x + 12582912.0f);
}

// Byte B of a word as fp32 in one instruction (the compiler otherwise
// extracts the byte first).
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
    float f;
    if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(x));
    else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(x));
    else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(x));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(x));
    return f;
}

// One packed word (8 codes, element 2j in the low nibble of byte j) -> the
// 8 codes as two words of int8, natural order.
__device__ __forceinline__ uint2 decode8(uint32_t w, float mult, float m8) {
    const uint32_t u = w ^ 0x88888888u;        // nibble = q + 8, unsigned
    const uint32_t lo = u & 0x0F0F0F0Fu;       // elements 0, 2, 4, 6
    const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu; // elements 1, 3, 5, 7
    uint32_t c[8];
    c[0] = code8(ubyte_f32<0>(lo), mult, m8);
    c[1] = code8(ubyte_f32<0>(hi), mult, m8);
    c[2] = code8(ubyte_f32<1>(lo), mult, m8);
    c[3] = code8(ubyte_f32<1>(hi), mult, m8);
    c[4] = code8(ubyte_f32<2>(lo), mult, m8);
    c[5] = code8(ubyte_f32<2>(hi), mult, m8);
    c[6] = code8(ubyte_f32<3>(lo), mult, m8);
    c[7] = code8(ubyte_f32<3>(hi), mult, m8);
    const uint32_t d0 = __builtin_amdgcn_perm(c[1], c[0], 0x0C0C0400u) | __builtin_amdgcn_perm(c[3], c[2], 0x04000C0Cu);
    const uint32_t d1 = __builtin_amdgcn_perm(c[5], c[4], 0x0C0C0400u) | __builtin_amdgcn_perm(c[7], c[6], 0x04000C0Cu);
    return make_uint2(d0, d1);
}

// Table decode for a lane whose 64 codes share one multiplier. The int8 code
// of nibble u (two's complement q = u or u - 16) is the same function of q for
// all of them, so the 16 codes are formed once with the same fp32 steps as
// code8 (RN(q * mult), clamp, round) and looked up per code with v_perm. By
// symmetry (RN, the clamp and ties-to-even rounding are odd functions) only
// q = 0..8 are evaluated; code(-q) is the negation, formed on the magic-add
// bit pattern as 2 * 0x4B400000 - bits. Table words: T0 = codes of q = 0..7
// (bytes 0..7 of {t.y, t.x}), T1 = codes of q = -8..-1 (bytes of {t.w, t.z}).
__device__ __forceinline__ uint4 code_table(float mult) {
    uint32_t r[9];
#pragma unroll
    for (int q = 0; q <= 8; ++q)
        r[q] = __float_as_uint(fminf(fmaxf((float)q * mult, -127.0f), 127.0f) + 12582912.0f);
    uint32_t n[9];
#pragma unroll
    for (int q = 1; q <= 8; ++q) n[q] = 2u * 0x4B400000u - r[q];
    auto pack4 = [](uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        return __builtin_amdgcn_perm(b, a, 0x0C0C0400u) | __builtin_amdgcn_perm(d, c, 0x04000C0Cu);
    };
    return make_uint4(pack4(r[0], r[1], r[2], r[3]), pack4(r[4], r[5], r[6], r[7]), pack4(n[8], n[7], n[6], n[5]),
                      pack4(n[4], n[3], n[2], n[1]));
}

// Four nibble bytes (0..15 each) -> their four codes: one v_perm per half of
// the table, and a byte mask from bit 3 (selector 0x0C gives 0x00, 0x0D 0xFF).
__device__ __forceinline__ uint32_t lookup4(uint32_t nib, uint4 tab) {
    const uint32_t sel = nib & 0x07070707u;
    const uint32_t a = __builtin_amdgcn_perm(tab.y, tab.x, sel);
    const uint32_t b = __builtin_amdgcn_perm(tab.w, tab.z, sel);
    const uint32_t mask = __builtin_amdgcn_perm(0u, 0u, ((nib >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
    return (b & mask) | (a & ~mask);
}

// One packed word (8 codes) -> two words of int8 codes in natural order, as decode8.
__device__ __forceinline__ uint2 decode8_table(uint32_t w, uint4 tab) {
    const uint32_t lo = lookup4(w & 0x0F0F0F0Fu, tab);         // elements 0, 2, 4, 6
    const uint32_t hi = lookup4((w >> 4) & 0x0F0F0F0Fu, tab);  // elements 1, 3, 5, 7
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

// decode8 with the first four codes (bytes 0-1) under one multiplier and the
// last four (bytes 2-3) under another: a word that spans two groups of 4.
__device__ __forceinline__ uint2 decode8_2(uint32_t w, float ma, float m8a, float mb, float m8b) {
    const uint32_t u = w ^ 0x88888888u;
    const uint32_t lo = u & 0x0F0F0F0Fu;
    const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;
    uint32_t c[8];
    c[0] = code8(ubyte_f32<0>(lo), ma, m8a);
    c[1] = code8(ubyte_f32<0>(hi), ma, m8a);
    c[2] = code8(ubyte_f32<1>(lo), ma, m8a);
    c[3] = code8(ubyte_f32<1>(hi), ma, m8a);
    c[4] = code8(ubyte_f32<2>(lo), mb, m8b);
    c[5] = code8(ubyte_f32<2>(hi), mb, m8b);
    c[6] = code8(ubyte_f32<3>(lo), mb, m8b);
    c[7] = code8(ubyte_f32<3>(hi), mb, m8b);
    const uint32_t d0 = __builtin_amdgcn_perm(c[1], c[0], 0x0C0C0400u) | __builtin_amdgcn_perm(c[3], c[2], 0x04000C0Cu);
    const uint32_t d1 = __builtin_amdgcn_perm(c[5], c[4], 0x0C0C0400u) | __builtin_amdgcn_perm(c[7], c[6], 0x04000C0Cu);
    return make_uint2(d0, d1);
}

// Codebook table for one multiplier: byte u = clamp(rint(RN(cb[u] * mult)),
// -127, 127), the same fp32 steps as the decode kernel, all 16 entries
// evaluated (a codebook has no symmetry to exploit). The entries come from
// the kernel arguments, i.e. scalar registers.
__device__ __forceinline__ uint4 code_table_cb(float mult, const Codebook &cb) {
    uint32_t r[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
        r[u] = __float_as_uint(fminf(fmaxf(cb.v[u] * mult, -127.0f), 127.0f) + 12582912.0f);
    auto pack4 = [](uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        return __builtin_amdgcn_perm(b, a, 0x0C0C0400u) | __builtin_amdgcn_perm(d, c, 0x04000C0Cu);
    };
    return make_uint4(pack4(r[0], r[1], r[2], r[3]), pack4(r[4], r[5], r[6], r[7]), pack4(r[8], r[9], r[10], r[11]),
                      pack4(r[12], r[13], r[14], r[15]));
}

// decode8_table with elements 0-3 (bytes 0-1) looked up in ta and elements
// 4-7 (bytes 2-3) in tb.
__device__ __forceinline__ uint2 decode8_table2(uint32_t w, uint4 ta, uint4 tb) {
    const uint32_t ln = w & 0x0F0F0F0Fu, hn = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t lo = __builtin_amdgcn_perm(lookup4(ln, tb), lookup4(ln, ta), 0x07060100u);
    const uint32_t hi = __builtin_amdgcn_perm(lookup4(hn, tb), lookup4(hn, ta), 0x07060100u);
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

}  // namespace
}  // namespace ck4
