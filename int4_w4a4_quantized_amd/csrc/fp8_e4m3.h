// OCP FP8 E4M3 scale bytes ("[PR #97] HIP port of #90: grouped W4A8 over the
// INT8 GEMM", What this adds: group scales in fp32 or e4m3): sign, 4 exponent
// bits (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN; normals
// (1 + m/8) 2^(e-7) up to 448, subnormals (m/8) 2^-6.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck4 {

// Non-negative fp32 -> E4M3: nearest, ties to even, saturating at 448. Every
// step is exact in fp32 (power-of-two scaling, a subtraction within one
// binade, rint), so the byte is the correctly rounded one.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    if (!(x < 448.0f)) return 0x7Eu;
    if (x < 0x1p-6f) return (uint32_t)(int)rintf(x * 512.0f);  // subnormal; 8 is the least normal
    int ex;
    frexpf(x, &ex);
    int e = ex - 1;
    float mm = rintf((ldexpf(x, -e) - 1.0f) * 8.0f);
    if (mm == 8.0f) {
        mm = 0.0f;
        e += 1;
    }
    const int be = e + 7;
    if (be > 15 || (be == 15 && mm == 7.0f)) return 0x7Eu;
    return (uint32_t)((be << 3) | (int)mm);
}

// E4M3 -> fp32, exact.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    const int e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return __builtin_nanf("");
    const float v = e == 0 ? (float)m * 0x1p-9f : ldexpf((float)(8 + m), e - 10);
    return (b & 0x80u) ? -v : v;
}

// Group scale idx of fp32 or E4M3 storage, as fp32.
template <bool E4M3>
__device__ __forceinline__ float load_scale(const void *gs, int64_t idx) {
    if constexpr (E4M3) return e4m3_decode(static_cast<const uint8_t *>(gs)[idx]);
    else return static_cast<const float *>(gs)[idx];
}

}  // namespace ck4
