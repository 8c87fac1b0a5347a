// Fused grouped W4A8 linear for one or two activation rows, as a matrix-vector
// product with coalesced weight loads, for gfx950.
//
// What it computes ("[PR #97] HIP port of #90: grouped W4A8 over the INT8
// GEMM", What this adds: int4 codes with per-group fp32 or e4m3 scales are
// decoded to int8 codes against one scale per row, then the rowwise int8 GEMM
// applies the activation and row scales):
//   s_row = (max_g s[n, g] * 7) / 127
//   w8    = clamp(rint(q * (s[n, g] / s_row)), -127, 127)
//   acc   = sum_k x8[m, k] w8[n, k]   (exact, int32)
//   y     = bf16((acc * sx[m]) * s_row)
// with the codes formed by the decode kernel's fp32 operations (w4a8_codes.h)
// and the int8 GEMM's epilogue, so y is bitwise decode + int8 GEMM.
//
// As in gemv_w4a4_kernel, a wavefront owns G weight rows (one here) and lane l the
// 16-byte chunks l, l + 64, ... (32 codes each) of every one of them, loaded
// coalesced into registers. With groups of 32 or more codes a chunk lies in
// one group, so the lane loads one group scale per chunk; since every group
// has a chunk, the wavefront's maximum of those loads is the row's maximum
// scale. Each chunk's 16 possible int8 codes are tabulated once for its
// multiplier and looked up per code (v_perm), then multiplied with the
// activation's int8 codes by v_dot4_i32_i8. The activation rows are copied
// into LDS once per workgroup; they are loaded first, the group scales
// second and the weight last, so each wait leaves the later loads in flight.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8_e4m3.h"
#include "gemv.h"
#include "gemv_core.h"
#include "w4a8_codes.h"

namespace ck4 {
namespace {

template <int MG, int G, int CPL, bool E4M3>
__global__ __launch_bounds__(64 * kGemvWaves) void w4a8_gemv_kernel(const int8_t *__restrict__ X,
                                                                   const float *__restrict__ sx,
                                                                   const int8_t *__restrict__ B,
                                                                   const void *__restrict__ gs, int M, int N, int K,
                                                                   int group, uint16_t *__restrict__ Y, int64_t ldy) {
    constexpr int T = 64 * kGemvWaves;
    constexpr int XPT = (MG * 2 * 64 * CPL + T - 1) / T;  // 16-byte activation chunks per thread
    constexpr int SB = E4M3 ? 1 : 4;                      // bytes per group scale
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // M x K int8
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_bytes = K / 2;
    const int nch = row_bytes / 16;  // 32-code chunks of a row
    const int ng = K / group;
    // a wavefront past N still takes part in the activation copy and its barrier
    const int n0 = (blockIdx.x * kGemvWaves + wave) * G;
    const int rows = max(0, min(G, N - n0));

    // the activation, M x K bytes
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(X), (short)0, M * K, 0x00020000);
    v4i xt[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * T;
        xt[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, c < M * 2 * nch ? (uint32_t)c * 16u : kGemvOob, 0, 0);
    }
    // the group scale of each of the lane's chunks (chunk c of 32 codes lies in group 32 c / group)
    const int8_t *gsb = static_cast<const int8_t *>(gs);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(rows > 0 ? gsb + (int64_t)n0 * ng * SB : gsb), (short)0, rows * ng * SB, 0x00020000);
    float sg[G][CPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            const uint32_t off = c < nch && g < rows ? (uint32_t)((g * ng + (32 * c) / group) * SB) : kGemvOob;
            if constexpr (E4M3) sg[g][j] = e4m3_decode(__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0));
            else sg[g][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        }
    v4i w[G][CPL];
    gemv_load_rows<G, CPL>(gemv_rows_rsrc(B, n0, rows, row_bytes), lane, nch, rows, row_bytes, w);

#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * T;
        if (c < M * 2 * nch) *reinterpret_cast<v4i *>(xs + c * 16) = xt[i];
    }
    // row scales: the maximum over the row's groups (chunks past the row read 0)
    float srow[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) a = fmaxf(a, sg[g][j]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
        srow[g] = (a * 7.0f) / 127.0f;
    }
    __syncthreads();  // the activation is in LDS

    int acc[G][MG];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[g][m] = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        v4i xl[MG][2];
#pragma unroll
        for (int m = 0; m < MG; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                xl[m][h] = m < M && c < nch ? *reinterpret_cast<const v4i *>(xs + m * K + c * 32 + h * 16)
                                            : v4i{0, 0, 0, 0};
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 tab = code_table(srow[g] == 0.0f ? 0.0f : sg[g][j] / srow[g]);
            int w8[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint2 d = decode8_table((uint32_t)w[g][j][e], tab);
                w8[2 * e] = (int)d.x;
                w8[2 * e + 1] = (int)d.y;
            }
#pragma unroll
            for (int m = 0; m < MG; ++m) {
                int a = acc[g][m];
#pragma unroll
                for (int e = 0; e < 8; ++e) a = __builtin_amdgcn_sdot4(w8[e], xl[m][e >> 2][e & 3], a, false);
                acc[g][m] = a;
            }
        }
    }

#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MG; ++m) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) acc[g][m] += __shfl_xor(acc[g][m], off, 64);
        }
    // lane g MG + m stores y[m][n0 + g]
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int m = 0; m < MG; ++m) {
            if (lane != g * MG + m || m >= M || g >= rows) continue;
            Y[(int64_t)m * ldy + n0 + g] = bf16_rne(((float)acc[g][m] * sx[m]) * srow[g]);
        }
}

template <int MG, int CPL>
hipError_t launch_cfg(const int8_t *x, const float *sx, const int8_t *w, const void *gs, bool e4m3, int64_t m,
                      int64_t n, int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream) {
    const dim3 grid((unsigned)((n + kGemvWaves - 1) / kGemvWaves)), block(64 * kGemvWaves);
    const size_t lds = (size_t)m * (size_t)k;
    if (e4m3)
        w4a8_gemv_kernel<MG, 1, CPL, true><<<grid, block, lds, stream>>>(x, sx, w, gs, (int)m, (int)n, (int)k, group,
                                                                         y, ldy);
    else
        w4a8_gemv_kernel<MG, 1, CPL, false><<<grid, block, lds, stream>>>(x, sx, w, gs, (int)m, (int)n, (int)k,
                                                                          group, y, ldy);
    return hipGetLastError();
}

template <int MG>
hipError_t launch_mg(const int8_t *x, const float *sx, const int8_t *w, const void *gs, bool e4m3, int64_t m,
                     int64_t n, int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream) {
    switch ((k / 32 + 63) / 64) {  // 16-byte weight chunks of a row per lane
    case 1: return launch_cfg<MG, 1>(x, sx, w, gs, e4m3, m, n, k, group, y, ldy, stream);
    case 2: return launch_cfg<MG, 2>(x, sx, w, gs, e4m3, m, n, k, group, y, ldy, stream);
    case 3: return launch_cfg<MG, 3>(x, sx, w, gs, e4m3, m, n, k, group, y, ldy, stream);
    default: return launch_cfg<MG, 4>(x, sx, w, gs, e4m3, m, n, k, group, y, ldy, stream);
    }
}

}  // namespace

// Where it beats the MFMA fused kernel (32 weight copies in turn, groups of
// 128, fp32 and E4M3 scales): one activation row up to N = 8192 (N = K =
// 5120: 7.2 against 9.6 us; N = K = 8192: 12.9 against 14.7 us), two rows
// up to N = 8192 and K = 5120; at N = 12288, K = 3072 the MFMA kernel's 9.4
// us is not beaten (the table decode costs as many VALU cycles as the wider
// launch hides there).
bool w4a8_gemv_fits(int64_t m, int64_t n, int64_t k, int group, bool codebook) {
    if (codebook || group < 32 || k < 256 || k % 128 != 0 || k > 8192 || n > 8192) return false;
    return m == 1 || (m == 2 && k <= 5120);
}

hipError_t launch_w4a8_gemv(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                            const void *group_scales, bool scale_e4m3, int64_t m, int64_t n, int64_t k, int group,
                            uint16_t *y, int64_t ldy, hipStream_t stream) {
    if (m <= 1)
        return launch_mg<1>(x_q8, x_scales, w_packed, group_scales, scale_e4m3, m, n, k, group, y, ldy, stream);
    return launch_mg<2>(x_q8, x_scales, w_packed, group_scales, scale_e4m3, m, n, k, group, y, ldy, stream);
}

}  // namespace ck4
