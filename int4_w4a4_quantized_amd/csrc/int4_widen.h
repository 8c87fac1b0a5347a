// Widening of packed int4 codes to the int8 matrix-core operands, shared by
// the W4A4 GEMM kernels ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot)
// with fused CUDA kernels", Description: the s4 x s4 product with int32
// accumulation). For a packed byte B (low nibble = code of element 2j, high =
// 2j + 1), B & 0xF0 read as int8 is exactly 16 hi and (B << 4) & 0xF0 is
// exactly 16 lo: a word of 8 codes widens to two words of 4 int8 each, the
// products carry a factor 256, and both operands split k the same way (even k
// in the low-nibble words, odd k in the high ones).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck4 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i as_v4i(uint4 u) {
    v4i r;
    r.x = (int)u.x;
    r.y = (int)u.y;
    r.z = (int)u.z;
    r.w = (int)u.w;
    return r;
}

__device__ __forceinline__ v4i widen_hi(uint4 p) {
    return as_v4i(make_uint4(p.x & 0xF0F0F0F0u, p.y & 0xF0F0F0F0u, p.z & 0xF0F0F0F0u, p.w & 0xF0F0F0F0u));
}

__device__ __forceinline__ v4i widen_lo(uint4 p) {
    return as_v4i(make_uint4((p.x << 4) & 0xF0F0F0F0u, (p.y << 4) & 0xF0F0F0F0u, (p.z << 4) & 0xF0F0F0F0u,
                             (p.w << 4) & 0xF0F0F0F0u));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

}  // namespace
}  // namespace ck4
