// Row-scale quantisation steps shared by the activation quantiser and the
// fused decode-time layer, so that both produce the same codes bit for bit
// ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with fused CUDA
// kernels", Description: s = absmax / qmax, q = rint(r / s) with ties to
// even, int4 codes packed in pairs with the even element in the low nibble).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck4 {
namespace {

__device__ __forceinline__ float wave_max(float a) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    return a;
}

// Integer code of r / s as a bit pattern whose low byte is the code plus
// BIAS (two's complement). The packed-int4 path uses BIAS = 8, so the low
// byte is q + 8 in [1, 15] with nothing above bit 3; the int8 path uses 0.
// Adding 1.5 * 2^23 + BIAS (an even integer, ulp 1 at that magnitude) rounds
// q1 to the nearest integer, ties to even, exactly as adding 1.5 * 2^23 does.
template <int BIAS>
__device__ __forceinline__ uint32_t code_fast(float r, float s, float y) {
    const float q0 = r * y;
    const float e = __builtin_fmaf(-q0, s, r);
    const float q1 = __builtin_fmaf(e, y, q0);
    return __float_as_uint(q1 + (12582912.0f + (float)BIAS));  // 1.5 * 2^23 + BIAS
}

template <int BIAS>
__device__ __forceinline__ uint32_t code_exact(float r, float s, float qmax) {
    if (s == 0.0f) return (uint32_t)BIAS;
    float t = rintf(r / s);
    t = fminf(fmaxf(t, -qmax), qmax);
    return (uint32_t)((int)t + BIAS);
}

// 8 biased int4 codes (low byte q + 8) -> one word, element 2j in the low
// nibble of byte j: pairs are joined with one shift-or (bits above 7 are
// don't-care), the four low bytes gathered with byte permutes, and the bias
// removed with one XOR ((q + 8) ^ 8 == q & 15 for q in [-8, 7]).
__device__ __forceinline__ uint32_t pack8_biased(const uint32_t *c) {
    uint32_t b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = (c[2 * t + 1] << 4) | c[2 * t];
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);  // [b0.0, b1.0, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);  // [0, 0, b2.0, b3.0]
    return (lo | hi) ^ 0x88888888u;
}

// 4 int8 codes (low bytes) -> one word, byte j = code j.
__device__ __forceinline__ uint32_t pack4_bytes(const uint32_t *c) {
    const uint32_t lo = __builtin_amdgcn_perm(c[1], c[0], 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(c[3], c[2], 0x04000C0Cu);
    return lo | hi;
}

}  // namespace
}  // namespace ck4
