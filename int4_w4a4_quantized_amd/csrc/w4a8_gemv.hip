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
//
// w4a8_layer_kernel is the whole W4A8 layer from bf16 activations in one
// launch: every workgroup rotates the activation rows and quantises them to
// int8 (s = absmax / 127) into its LDS with the quantiser's own helpers
// (fwht.h, quant_codes.h), so codes and scales are bitwise the quantiser's,
// then runs the same per-row product.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8_e4m3.h"
#include "fwht.h"
#include "gemv.h"
#include "gemv_core.h"
#include "quant_codes.h"
#include "w4a8_codes.h"

namespace ck4 {
namespace {

// One weight row per wavefront: the group scales of the lane's chunks, then
// its chunks of the row (rows == 0: a wavefront past N, every load a no-op).
template <int CPL, bool E4M3>
__device__ __forceinline__ void w4a8_load_row(const int8_t *__restrict__ B, const void *__restrict__ gs, int n, int rows,
                                              int K, int group, int lane, float (&sg)[CPL], v4i (&w)[CPL]) {
    constexpr int SB = E4M3 ? 1 : 4;  // bytes per group scale
    const int row_bytes = K / 2;
    const int nch = row_bytes / 16;
    const int ng = K / group;
    const int8_t *gsb = static_cast<const int8_t *>(gs);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(rows > 0 ? gsb + (int64_t)n * ng * SB : gsb), (short)0, rows * ng * SB, 0x00020000);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;  // chunk c of 32 codes lies in group 32 c / group
        const uint32_t off = c < nch && rows > 0 ? (uint32_t)(((32 * c) / group) * SB) : kGemvOob;
        if constexpr (E4M3) sg[j] = e4m3_decode(__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0));
        else sg[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    }
    v4i wg[1][CPL];
    gemv_load_rows<1, CPL>(gemv_rows_rsrc(B, n, rows, row_bytes), lane, nch, rows, row_bytes, wg);
#pragma unroll
    for (int j = 0; j < CPL; ++j) w[j] = wg[0][j];
}

// The row scale: (max over the row's groups * 7) / 127; every group has a
// chunk, and chunks past the row read 0.
template <int CPL>
__device__ __forceinline__ float w4a8_row_scale(const float (&sg)[CPL]) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) a = fmaxf(a, sg[j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    return (a * 7.0f) / 127.0f;
}

// The row's int8 codes against the M activation rows in LDS (xs: M x K int8),
// summed over the wavefront, and y[m][n] = bf16((acc * sx[m]) * srow) from
// lane m.
template <int MG, int CPL>
__device__ __forceinline__ void w4a8_row_product(const float (&sg)[CPL], const v4i (&w)[CPL], float srow,
                                                 const uint8_t *xs, int M, int K, int lane, int n, int rows,
                                                 const float (&sx)[MG], uint16_t *__restrict__ Y, int64_t ldy) {
    const int nch = K / 32;
    int acc[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) acc[m] = 0;
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
        const uint4 tab = code_table(srow == 0.0f ? 0.0f : sg[j] / srow);
        int w8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint2 d = decode8_table((uint32_t)w[j][e], tab);
            w8[2 * e] = (int)d.x;
            w8[2 * e + 1] = (int)d.y;
        }
#pragma unroll
        for (int m = 0; m < MG; ++m) {
            int a = acc[m];
#pragma unroll
            for (int e = 0; e < 8; ++e) a = __builtin_amdgcn_sdot4(w8[e], xl[m][e >> 2][e & 3], a, false);
            acc[m] = a;
        }
    }
#pragma unroll
    for (int m = 0; m < MG; ++m) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc[m] += __shfl_xor(acc[m], off, 64);
    }
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        if (lane != m || m >= M || rows <= 0) continue;
        Y[(int64_t)m * ldy + n] = bf16_rne(((float)acc[m] * sx[m]) * srow);
    }
}

template <int MG, int CPL, bool E4M3>
__global__ __launch_bounds__(64 * kGemvWaves) void w4a8_gemv_kernel(const int8_t *__restrict__ X,
                                                                   const float *__restrict__ sx,
                                                                   const int8_t *__restrict__ B,
                                                                   const void *__restrict__ gs, int M, int N, int K,
                                                                   int group, uint16_t *__restrict__ Y, int64_t ldy) {
    constexpr int T = 64 * kGemvWaves;
    constexpr int XPT = (MG * 2 * 64 * CPL + T - 1) / T;  // 16-byte activation chunks per thread
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // M x K int8
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int xch = M * (K / 16);  // 16-byte activation chunks
    // a wavefront past N still takes part in the activation copy and its barrier
    const int n = blockIdx.x * kGemvWaves + wave;
    const int rows = n < N ? 1 : 0;

    // the activation (M x K bytes), then the row's scales and codes
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(X), (short)0, M * K, 0x00020000);
    v4i xt[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * T;
        xt[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, c < xch ? (uint32_t)c * 16u : kGemvOob, 0, 0);
    }
    float sg[CPL];
    v4i w[CPL];
    w4a8_load_row<CPL, E4M3>(B, gs, n, rows, K, group, lane, sg, w);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * T;
        if (c < xch) *reinterpret_cast<v4i *>(xs + c * 16) = xt[i];
    }
    const float srow = w4a8_row_scale<CPL>(sg);
    __syncthreads();  // the activation is in LDS
    float sxr[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) sxr[m] = m < M ? sx[m] : 0.0f;
    w4a8_row_product<MG, CPL>(sg, w, srow, xs, M, K, lane, n, rows, sxr, Y, ldy);
}

// The layer: NW wavefronts, one weight row each. Rotation mapping as in
// skinny_layer_kernel: thread t owns the 16-element chunks t + 64 NW j of
// each row, j < CPR; a 128-element block is 8 consecutive chunks in 8
// consecutive lanes of one wavefront.
template <int NW, int CPR, int MG, int CPL, bool E4M3>
__global__ __launch_bounds__(64 * NW) void w4a8_layer_kernel(const uint16_t *__restrict__ X, int64_t ldx, float c,
                                                             const int8_t *__restrict__ B,
                                                             const void *__restrict__ gs, int M, int N, int K,
                                                             int group, int8_t *__restrict__ XQ,
                                                             float *__restrict__ SX, uint16_t *__restrict__ Y,
                                                             int64_t ldy) {
    constexpr int T = 64 * NW;
    constexpr int LPB = 8;  // chunks per 128-element rotation block
    static_assert(MG * CPR <= 4, "rotation registers");
    __shared__ float amax_lds[MG * NW];
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // the int8 codes, M x K

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = blockIdx.x * NW + wave;
    const int rows = n < N ? 1 : 0;
    const int nchunks = K / kElems;

    // the bf16 activation first, then the row's scales and codes: loads
    // retire in order, so the wait for the activation leaves those in flight
    uint4 raw[MG][CPR][2];
#pragma unroll
    for (int r = 0; r < MG; ++r)
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
            const int ch = tid + j * T;
            if (r < M && ch < nchunks) {
                const uint4 *q = reinterpret_cast<const uint4 *>(X + (int64_t)r * ldx + (int64_t)ch * kElems);
                raw[r][j][0] = q[0];
                raw[r][j][1] = q[1];
            }
        }
    float sg[CPL];
    v4i w[CPL];
    w4a8_load_row<CPL, E4M3>(B, gs, n, rows, K, group, lane, sg, w);

    const float c_lane = (__popc(lane & (LPB - 1)) & 1) ? -c : c;  // sign left by the cross-lane stages
    float v[MG][CPR][kElems];
    float am[MG];
#pragma unroll
    for (int r = 0; r < MG; ++r) {
        am[r] = 0.0f;
        if (r < M) {
#pragma unroll
            for (int j = 0; j < CPR; ++j) {
                const int ch = tid + j * T;
                if (ch < nchunks) {
                    // bf16 -> fp32 as load_chunk does
                    const uint32_t wds[8] = {raw[r][j][0].x, raw[r][j][0].y, raw[r][j][0].z, raw[r][j][0].w,
                                             raw[r][j][1].x, raw[r][j][1].y, raw[r][j][1].z, raw[r][j][1].w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        v[r][j][2 * i] = __uint_as_float(wds[i] << 16);
                        v[r][j][2 * i + 1] = __uint_as_float(wds[i] & 0xFFFF0000u);
                    }
                    fwht_in_lane(v[r][j]);
                    fwht_cross_lane<LPB>(v[r][j], lane);
#pragma unroll
                    for (int i = 0; i < kElems; ++i) {
                        v[r][j][i] = v[r][j][i] * c_lane;
                        am[r] = fmaxf(am[r], fabsf(v[r][j][i]));
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < MG; ++r) {
        const float a = wave_max(am[r]);
        if (lane == 0) amax_lds[r * NW + wave] = a;
    }
    __syncthreads();
    float sxr[MG];
#pragma unroll
    for (int r = 0; r < MG; ++r) {
        sxr[r] = 0.0f;
        if (r >= M) continue;
        float a = amax_lds[r * NW];
#pragma unroll
        for (int q = 1; q < NW; ++q) a = fmaxf(a, amax_lds[r * NW + q]);
        const float s_row = a / 127.0f;
        const bool fast = s_row >= 0x1p-120f && s_row <= 0x1p120f;
        const float y_row = fast ? 1.0f / s_row : 0.0f;
        if (blockIdx.x == 0 && tid == 0) SX[r] = s_row;
        sxr[r] = s_row;
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
            const int ch = tid + j * T;
            if (ch >= nchunks) continue;
            uint32_t code[kElems];
            if (fast) {
#pragma unroll
                for (int i = 0; i < kElems; ++i) code[i] = code_fast<0>(v[r][j][i], s_row, y_row);
            } else {
#pragma unroll
                for (int i = 0; i < kElems; ++i) code[i] = code_exact<0>(v[r][j][i], s_row, 127.0f);
            }
            const uint4 pk = make_uint4(pack4_bytes(code), pack4_bytes(code + 4), pack4_bytes(code + 8),
                                        pack4_bytes(code + 12));
            *reinterpret_cast<uint4 *>(xs + r * K + ch * kElems) = pk;
            if (blockIdx.x == 0) *reinterpret_cast<uint4 *>(XQ + (int64_t)r * K + (int64_t)ch * kElems) = pk;
        }
    }
    const float srow = w4a8_row_scale<CPL>(sg);
    __syncthreads();  // the codes are in LDS
    w4a8_row_product<MG, CPL>(sg, w, srow, xs, M, K, lane, n, rows, sxr, Y, ldy);
}

template <int MG, int CPL>
hipError_t launch_cfg(const int8_t *x, const float *sx, const int8_t *w, const void *gs, bool e4m3, int64_t m,
                      int64_t n, int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream) {
    const dim3 grid((unsigned)((n + kGemvWaves - 1) / kGemvWaves)), block(64 * kGemvWaves);
    const size_t lds = (size_t)m * (size_t)k;
    if (e4m3)
        w4a8_gemv_kernel<MG, CPL, true><<<grid, block, lds, stream>>>(x, sx, w, gs, (int)m, (int)n, (int)k, group, y,
                                                                      ldy);
    else
        w4a8_gemv_kernel<MG, CPL, false><<<grid, block, lds, stream>>>(x, sx, w, gs, (int)m, (int)n, (int)k, group,
                                                                       y, ldy);
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

template <int NW, int CPR, int MG, int CPL>
hipError_t launch_layer_cfg(const uint16_t *x, int64_t ldx, const int8_t *w, const void *gs, bool e4m3, int64_t m,
                            int64_t n, int64_t k, int group, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                            hipStream_t stream) {
    const dim3 grid((unsigned)((n + NW - 1) / NW)), block(64 * NW);
    const size_t lds = (size_t)m * (size_t)k;
    const float c = (float)(1.0 / __builtin_sqrt(128.0));
    if (e4m3)
        w4a8_layer_kernel<NW, CPR, MG, CPL, true><<<grid, block, lds, stream>>>(x, ldx, c, w, gs, (int)m, (int)n,
                                                                                (int)k, group, xq, sx, y, ldy);
    else
        w4a8_layer_kernel<NW, CPR, MG, CPL, false><<<grid, block, lds, stream>>>(x, ldx, c, w, gs, (int)m, (int)n,
                                                                                 (int)k, group, xq, sx, y, ldy);
    return hipGetLastError();
}

template <int NW, int MG>
hipError_t launch_layer_mg(const uint16_t *x, int64_t ldx, const int8_t *w, const void *gs, bool e4m3, int64_t m,
                           int64_t n, int64_t k, int group, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                           hipStream_t stream) {
    // CPR: rotation chunks per thread (64 NW threads); CPL: 16-byte weight chunks per lane
    constexpr int C2 = (4096 + 64 * NW * 16 - 1) / (64 * NW * 16);
    switch ((k / 32 + 63) / 64) {
    case 1: return launch_layer_cfg<NW, (2048 + 64 * NW * 16 - 1) / (64 * NW * 16), MG, 1>(x, ldx, w, gs, e4m3, m, n, k, group, xq, sx, y, ldy, stream);
    case 2: return launch_layer_cfg<NW, C2, MG, 2>(x, ldx, w, gs, e4m3, m, n, k, group, xq, sx, y, ldy, stream);
    case 3: return launch_layer_cfg<NW, (6144 + 64 * NW * 16 - 1) / (64 * NW * 16), MG, 3>(x, ldx, w, gs, e4m3, m, n, k, group, xq, sx, y, ldy, stream);
    default: return launch_layer_cfg<NW, (8192 + 64 * NW * 16 - 1) / (64 * NW * 16), MG, 4>(x, ldx, w, gs, e4m3, m, n, k, group, xq, sx, y, ldy, stream);
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

// One-call layer against the quantiser + the W4A8 linear (32 weight copies in
// turn, groups of 128): with one activation row it is faster up to N = 8192
// (N = K = 5120: 10.2 against 11.2 us; N = 8192, K = 3072: 9.3 against
// 11.0; N = 4096, K = 2048: 4.7 against 7.1); at N = 12288, K = 3072 the
// product's table decode loses more than the launch saves (13.4 against
// 12.7). With two rows the quantisation repeated per workgroup costs what
// the quantiser's launch saves (N = K = 5120: 12.1 against 12.0).
// Workgroups of eight wavefronts measured faster than of sixteen on four of
// five shapes.
bool w4a8_layer_fits(int64_t m, int64_t n, int64_t k, int rot_block, int group, bool codebook, bool scale_e4m3) {
    (void)scale_e4m3;
    return !codebook && m == 1 && n <= 8192 && rot_block == 128 && group >= 32 && k >= 256 && k % 128 == 0 &&
           k <= 8192;
}

hipError_t launch_w4a8_layer(const uint16_t *x, int64_t ldx, const int8_t *w_packed, const void *group_scales,
                             bool scale_e4m3, int64_t m, int64_t n, int64_t k, int group, int8_t *x_q8,
                             float *x_scales, uint16_t *y, int64_t ldy, hipStream_t stream) {
    return launch_layer_mg<8, 1>(x, ldx, w_packed, group_scales, scale_e4m3, m, n, k, group, x_q8, x_scales, y, ldy,
                                 stream);
}

}  // namespace ck4
