// The matrix-vector core of the W4A4 product for one or two activation
// rows, shared by gemv_w4a4_kernel and the one-call layer kernel
// ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with fused CUDA
// kernels", Description: the s4 x s4 product with int32 accumulation and the
// rank-one epilogue):
//   acc[m, n] = sum_k qx[m, k] qw[n, k]   (exact, int32)
//   y[m, n]   = bf16(((float)acc * sx[m]) * sw[n] (+ bias[n]))
// the same expression, in the same fp32 steps, as the GEMM kernels.
//
// A wavefront owns G consecutive weight rows. Lane l holds the 16-byte
// chunks l, l + 64, ... (CPL of them) of each of its rows and of each
// activation row, so a load instruction reads 1 KB of one row, coalesced. A
// chunk's 32 codes are widened x16 (int4_widen.h) and multiplied with
// v_dot4_i32_i8, four products per instruction; the products carry 256,
// removed by an exact shift after the sum. The 64 lane sums of a row meet
// through cross-lane shuffles (integer, exact in any order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "int4_widen.h"

namespace ck4 {
namespace {

constexpr int kGemvWaves = 4;           // wavefronts per workgroup
constexpr uint32_t kGemvOob = 0x40000000u;  // an offset past any operand here: the load returns zeros

// Buffer descriptor over weight rows [n0, n0 + rows) of a [N, row_bytes] matrix.
// n0 and rows are the same in every lane of the wavefront; the fields go
// through readfirstlane so that the compiler keeps the descriptor in scalar
// registers (a descriptor it cannot prove uniform costs a loop around every
// load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemv_rows_rsrc(const int8_t *base, int n0, int rows,
                                                                 int row_bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(rows > 0 ? base + (int64_t)n0 * row_bytes : base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const int nrec = __builtin_amdgcn_readfirstlane(rows > 0 ? rows * row_bytes : 0);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0, nrec,
                                             0x00020000);
}

// Issue the loads of the G rows' chunks: always G x CPL instructions, a chunk
// past the row or a row past the last one reading zeros through the bounds
// check, so that the number in flight is fixed.
template <int G, int CPL>
__device__ __forceinline__ void gemv_load_rows(__amdgpu_buffer_rsrc_t r, int lane, int nch, int rows, int row_bytes,
                                               v4i (&w)[G][CPL]) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            const uint32_t off = c < nch && g < rows ? (uint32_t)(g * row_bytes + c * 16) : kGemvOob;
            w[g][j] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        }
}

// acc[g][m] = this lane's part of 256 sum_k qw[g, k] qx[m, k].
template <int G, int MG, int CPL>
__device__ __forceinline__ void gemv_accumulate(const v4i (&w)[G][CPL], const v4i (&x)[MG][CPL],
                                                int (&acc)[G][MG]) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[g][m] = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        v4i xl[MG], xh[MG];
#pragma unroll
        for (int m = 0; m < MG; ++m) {
            const uint4 xp = make_uint4(x[m][j].x, x[m][j].y, x[m][j].z, x[m][j].w);
            xl[m] = widen_lo(xp);
            xh[m] = widen_hi(xp);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 wp = make_uint4(w[g][j].x, w[g][j].y, w[g][j].z, w[g][j].w);
            const v4i wl = widen_lo(wp), wh = widen_hi(wp);
#pragma unroll
            for (int m = 0; m < MG; ++m) {
                int a = acc[g][m];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a = __builtin_amdgcn_sdot4(wl[e], xl[m][e], a, false);
                    a = __builtin_amdgcn_sdot4(wh[e], xh[m][e], a, false);
                }
                acc[g][m] = a;
            }
        }
    }
}

// Sum the lanes and write y[m][n0 + g] from lane g MG + m, with sx[m] the
// activation row scales (m < M).
template <int G, int MG>
__device__ __forceinline__ void gemv_store(int (&acc)[G][MG], int lane, int M, int n0, int rows,
                                           const float (&sx)[MG], const float *__restrict__ sb,
                                           const float *__restrict__ bias, uint16_t *__restrict__ Y, int64_t ldy) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MG; ++m) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) acc[g][m] += __shfl_xor(acc[g][m], off, 64);
        }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MG; ++m) {
            if (lane != g * MG + m || m >= M || g >= rows) continue;
            const int n = n0 + g;
            float v = ((float)(acc[g][m] >> 8) * sx[m]) * sb[n];
            if (bias) v = v + bias[n];
            Y[(int64_t)m * ldy + n] = f32_to_bf16(v);
        }
}

}  // namespace
}  // namespace ck4
