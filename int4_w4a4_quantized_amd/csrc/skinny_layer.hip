// The whole W4A4 layer for m <= 2 activation rows in one launch: rotate +
// quantise + pack the activation, then the s4 x s4 GEMM with its rank-one
// epilogue, for gfx950.
//
// What it computes ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with
// fused CUDA kernels", Description: the activation kernel rotates, takes the
// row scale, quantises to int4 and packs; the GEMM multiplies the packed
// codes with int32 accumulation and applies the row and column scales once):
//   r = x * blockdiag(H_128, ...) * fp32(1/sqrt(128)),  s = absmax(r) / 7,
//   q = rint(r / s)  (ties to even),  acc = sum_k q[m, k] w[n, k]  (int32),
//   y = bf16(((float)acc * s[m]) * sw[n] (+ bias[n])).
//
// At decode sizes the quantiser is a launch of a few workgroups whose
// latency is a large part of the layer. Here every workgroup rotates and
// quantises the m rows itself (m x K bf16, a few KB, read from L2) into its
// LDS while its weight loads are in flight. The steps are those of
// rotate_quant_kernel, through the same helpers (fwht.h, quant_codes.h): the
// same butterflies in the same order, the same scale division, the same
// quotient and rounding, so the codes and scales are bitwise the
// two-launch path's. Workgroup 0 also writes them out (x_q, x_scales), so a
// caller can reuse them. The product is gemv_w4a4_kernel's (gemv_core.h):
// each wavefront owns G weight rows, lane l the 16-byte chunks l, l + 64, ...
// of each, loaded coalesced into registers, the activation chunks with the
// same k read from LDS. Integer accumulation is exact and the epilogue the
// same fp32 expression, so the output is bitwise the two-launch path's too.
//
// Rotation mapping: thread t of the workgroup (256 threads) owns the
// 16-element chunks t + 256 j of each row, j < CPR; a 128-element block is 8
// consecutive chunks in 8 consecutive lanes of one wavefront, as in the
// quantiser. Registers hold MQ rows x CPR chunks (MQ x CPR <= 4).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwht.h"
#include "gemv.h"
#include "gemv_core.h"
#include "quant_codes.h"

namespace ck4 {
namespace {

constexpr int kLayerRows = 2;  // activation rows the fused kernel takes

template <int NW, int MQ, int CPR, int MG, int G, int CPL>
__global__ __launch_bounds__(64 * NW) void skinny_layer_kernel(const uint16_t *__restrict__ X, int64_t ldx,
                                                                     float c, const int8_t *__restrict__ B,
                                                                     const float *__restrict__ sb,
                                                                     const float *__restrict__ bias, int M, int N,
                                                                     int K, int8_t *__restrict__ XQ,
                                                                     float *__restrict__ SX, uint16_t *__restrict__ Y,
                                                                     int64_t ldy) {
    constexpr int T = 64 * NW;
    constexpr int LPB = 8;  // chunks per 128-element rotation block
    static_assert(MQ * CPR <= 4 && MQ <= kLayerRows && MG <= MQ, "rotation registers");
    __shared__ float amax_lds[kLayerRows * NW];
    extern __shared__ __attribute__((aligned(16))) uint8_t xq[];  // the codes, M x K/2

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_bytes = K / 2;
    const int nch = row_bytes / 16;
    // a wavefront past N still takes part in the quantisation and its barriers
    const int n0 = (blockIdx.x * NW + wave) * G;
    const int rows = max(0, min(G, N - n0));

    // --- the activation first, then the weight rows: memory loads retire in
    // order, so the wait for the activation leaves the weight loads (a fixed
    // number of them) in flight while the rows are rotated and quantised.
    const int nchunks = K / kElems;
    uint4 raw[MQ][CPR][2];
#pragma unroll
    for (int r = 0; r < MQ; ++r)
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
            const int ch = tid + j * T;
            if (r < M && ch < nchunks) {
                const uint4 *q = reinterpret_cast<const uint4 *>(X + (int64_t)r * ldx + (int64_t)ch * kElems);
                raw[r][j][0] = q[0];
                raw[r][j][1] = q[1];
            }
        }
    v4i w[G][CPL];
    gemv_load_rows<G, CPL>(gemv_rows_rsrc(B, n0, rows, row_bytes), lane, nch, rows, row_bytes, w);

    const float c_lane = (__popc(lane & (LPB - 1)) & 1) ? -c : c;  // sign left by the cross-lane stages
    float v[MQ][CPR][kElems];
    float am[MQ];
#pragma unroll
    for (int r = 0; r < MQ; ++r) {
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
    for (int r = 0; r < MQ; ++r) {
        const float a = wave_max(am[r]);
        if (lane == 0) amax_lds[r * NW + wave] = a;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < MQ; ++r) {
        if (r >= M) continue;
        float a = amax_lds[r * NW];
#pragma unroll
        for (int q = 1; q < NW; ++q) a = fmaxf(a, amax_lds[r * NW + q]);
        const float s_row = a / 7.0f;
        const bool fast = s_row >= 0x1p-120f && s_row <= 0x1p120f;
        const float y_row = fast ? 1.0f / s_row : 0.0f;
        if (blockIdx.x == 0 && tid == 0) SX[r] = s_row;
        am[r] = s_row;  // from here on, the row scale
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
            const int ch = tid + j * T;
            if (ch >= nchunks) continue;
            uint32_t code[kElems];
            if (fast) {
#pragma unroll
                for (int i = 0; i < kElems; ++i) code[i] = code_fast<8>(v[r][j][i], s_row, y_row);
            } else {
#pragma unroll
                for (int i = 0; i < kElems; ++i) code[i] = code_exact<8>(v[r][j][i], s_row, 7.0f);
            }
            const uint2 pk = make_uint2(pack8_biased(code), pack8_biased(code + 8));
            *reinterpret_cast<uint2 *>(xq + r * row_bytes + ch * (kElems / 2)) = pk;
            if (blockIdx.x == 0)
                *reinterpret_cast<uint2 *>(XQ + (int64_t)r * row_bytes + (int64_t)ch * (kElems / 2)) = pk;
        }
    }
    __syncthreads();  // the codes are in LDS

    // --- the product: this lane's activation chunks from LDS (rows past M
    // and chunks past the row read as zeros)
    v4i x[MG][CPL];
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int ch = lane + 64 * j;
            x[m][j] = m < M && ch < nch ? *reinterpret_cast<const v4i *>(xq + m * row_bytes + ch * 16)
                                        : v4i{0, 0, 0, 0};
        }
    int acc[G][MG];
    gemv_accumulate<G, MG, CPL>(w, x, acc);
    float sx[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) sx[m] = am[m];
    gemv_store<G, MG>(acc, lane, M, n0, rows, sx, sb, bias, Y, ldy);
}

template <int NW, int MQ, int CPR, int MG, int G, int CPL>
hipError_t launch_layer_cfg(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const float *bias,
                            int64_t m, int64_t n, int64_t k, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                            hipStream_t stream) {
    static_assert((CPL + 1) / 2 <= CPR * NW / 4, "rotation chunks per thread");
    const size_t lds = (size_t)m * (size_t)(k / 2);
    const float c = (float)(1.0 / __builtin_sqrt(128.0));
    const dim3 grid((unsigned)((n + G * NW - 1) / (G * NW))), block(64 * NW);
    skinny_layer_kernel<NW, MQ, CPR, MG, G, CPL><<<grid, block, lds, stream>>>(x, ldx, c, w, ws, bias, (int)m, (int)n,
                                                                               (int)k, xq, sx, y, ldy);
    return hipGetLastError();
}

template <int NW, int CPR, int G, int CPL>
hipError_t launch_layer_mg(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const float *bias,
                           int64_t m, int64_t n, int64_t k, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                           hipStream_t stream) {
    if (m <= 1) return launch_layer_cfg<NW, 2, CPR, 1, G, CPL>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    return launch_layer_cfg<NW, 2, CPR, 2, G, CPL>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
}

template <int G>
hipError_t launch_layer_g(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const float *bias,
                          int64_t m, int64_t n, int64_t k, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                          hipStream_t stream) {
    // CPL = 16-byte code chunks per lane and row of the product; 16
    // wavefronts rotate up to 16384 elements a row at one chunk per thread
    switch ((k / 32 + 63) / 64) {
    case 1: return launch_layer_mg<16, 1, G, 1>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    case 2: return launch_layer_mg<16, 1, G, 2>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    case 3: return launch_layer_mg<16, 1, (G < 2 ? G : 2), 3>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    default: return launch_layer_mg<16, 1, (G < 2 ? G : 2), 4>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    }
}

}  // namespace

bool skinny_layer_fits(int64_t m, int64_t n, int64_t k, int rot_block) {
    (void)n;
    return m >= 1 && m <= kLayerRows && rot_block == 128 && k >= 256 && k % 128 == 0 && k <= 8192;
}

hipError_t launch_skinny_layer(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const float *bias,
                               int64_t m, int64_t n, int64_t k, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                               hipStream_t stream) {
    // the most weight rows per wavefront (4, 2, 1) that still give 160 or
    // more workgroups of 16 wavefronts
    if ((n + 63) / 64 >= 160) return launch_layer_g<4>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    if ((n + 31) / 32 >= 160) return launch_layer_g<2>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    return launch_layer_g<1>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
}

}  // namespace ck4
