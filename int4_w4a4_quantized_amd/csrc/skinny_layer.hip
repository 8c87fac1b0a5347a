// The whole W4A4 layer for m <= 4 activation rows in one launch: rotate +
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
// LDS while its first weight loads are in flight. The steps are those of
// rotate_quant_kernel, through the same helpers (fwht.h, quant_codes.h): the
// same butterflies in the same order, the same scale division, the same
// quotient and rounding, so the codes and scales are bitwise the
// two-launch path's. Workgroup 0 also writes them out (x_q, x_scales), so a
// caller can reuse them. The GEMM is gemm_skinny_kernel's direct-load path:
// one 16-row weight tile per workgroup, KS wavefronts splitting K in 256-k
// steps (a half last step when K = 128 mod 256), the weight loaded straight
// into registers MAXS steps at a time, the activation fragments read from
// LDS (rows past m read as zeros), the partial sums added through LDS and
// the epilogue run by wavefront 0. Integer accumulation is exact, so the
// output is bitwise the two-launch path's too.
//
// Rotation mapping: thread t of the workgroup (T = 64 KS threads) owns the
// 16-element chunks t + jT of each row, j < CPR; a 128-element block is 8
// consecutive chunks in 8 consecutive lanes of one wavefront, as in the
// quantiser. Registers hold MR rows x CPR chunks (MR x CPR <= 4).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"
#include "fwht.h"
#include "int4_widen.h"
#include "quant_codes.h"

namespace ck4 {
namespace {

constexpr int kLayerRows = 4;  // activation rows the fused kernel takes

template <int KS, int MAXS, int MR, int CPR>
__global__ __launch_bounds__(64 * KS) void skinny_layer_kernel(const uint16_t *__restrict__ X, int64_t ldx, float c,
                                                               const int8_t *__restrict__ B,
                                                               const float *__restrict__ sb,
                                                               const float *__restrict__ bias, int M, int N, int K,
                                                               int8_t *__restrict__ XQ, float *__restrict__ SX,
                                                               uint16_t *__restrict__ Y, int64_t ldy) {
    constexpr int T = 64 * KS;
    constexpr int LPB = 8;     // chunks per 128-element rotation block
    constexpr int SLAB = 128;  // packed bytes of a row per 256-k step
    constexpr int RED_B = (KS - 1) * 64 * 16;
    constexpr int AMAX_B = kLayerRows * KS * 4;
    static_assert(MR * CPR <= 4 && MR <= kLayerRows, "rotation registers");
    // LDS: [partial sums (KS - 1) x 1 KB][row maxima][codes, M x K/2]
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    v4i *red = reinterpret_cast<v4i *>(dyn);
    float *amax_lds = reinterpret_cast<float *>(dyn + RED_B);
    uint8_t *xq = dyn + RED_B + AMAX_B;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 16;
    const int rows_b = min(16, N - n0);
    const int row_bytes = K / 2;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(B) + (int64_t)n0 * row_bytes, (short)0, rows_b * row_bytes, 0x00020000);
    const int frow = lane & 15;
    const int fgrp = lane >> 4;
    // weight loads: lane l reads row l & 15, 16 bytes at 16 (l >> 4) of each 64-byte half
    const uint32_t lane_off = (uint32_t)frow * (uint32_t)row_bytes + (uint32_t)(fgrp * 16);
    const int halves = K / 128;
    const int steps = (halves + 1) >> 1;
    const bool half_tail = halves & 1;
    const int per_wave = (steps + KS - 1) / KS;
    const int s_begin = wave * per_wave;
    const int s_end = min(steps, s_begin + per_wave);

    // MAXS steps of weight loads, always 2 MAXS instructions: a step past
    // this wavefront's last (or the missing half of a half step) gets an
    // offset beyond the buffer range, which the bounds check turns into a
    // load of zeros that moves no data. With a fixed count the compiler's
    // wait for the activation, loaded before them, leaves them in flight.
    constexpr uint32_t kOob = 0x40000000u;  // beyond any weight tile here (at most 1 MB)
    v4i wv[MAXS][2];
    auto load_w = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            const int s = s0 + t;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool real = s < s_end && !(h == 1 && half_tail && s == steps - 1);
                wv[t][h] = __builtin_amdgcn_raw_buffer_load_b128(rb, lane_off + (real ? 0u : kOob),
                                                                 s * SLAB + h * 64, 0);
            }
        }
    };

    // --- rotate + quantise the activation rows into LDS. The activation is
    // loaded first and the first weight steps right after it: memory loads
    // retire in order, so waiting for the activation does not wait for them.
    const int nchunks = K / kElems;
    const float c_lane = (__popc(lane & (LPB - 1)) & 1) ? -c : c;  // sign left by the cross-lane stages
    uint4 raw[MR][CPR][2];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
            const int ch = tid + j * T;
            if (r < M && ch < nchunks) {
                const uint4 *q = reinterpret_cast<const uint4 *>(X + (int64_t)r * ldx + (int64_t)ch * kElems);
                raw[r][j][0] = q[0];
                raw[r][j][1] = q[1];
            }
        }
    load_w(s_begin);
    float v[MR][CPR][kElems];
    float am[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
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
    for (int r = 0; r < MR; ++r) {
        const float a = wave_max(am[r]);
        if (lane == 0) amax_lds[r * KS + wave] = a;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        if (r >= M) continue;
        float a = amax_lds[r * KS];
#pragma unroll
        for (int w = 1; w < KS; ++w) a = fmaxf(a, amax_lds[r * KS + w]);
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

    // --- the GEMM over this wavefront's k-steps
    v4i acc = v4i{0, 0, 0, 0};
    const uint8_t *xrow = xq + (frow < M ? frow : 0) * row_bytes + fgrp * 16;
    for (int s0 = s_begin; s0 < s_end; s0 += MAXS) {
        if (s0 != s_begin) load_w(s0);
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            const int s = s0 + t;
            if (s >= s_end) break;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1 && half_tail && s == steps - 1) break;
                uint4 xp = *reinterpret_cast<const uint4 *>(xrow + s * SLAB + h * 64);
                if (frow >= M) xp = make_uint4(0u, 0u, 0u, 0u);
                const uint4 wp = make_uint4(wv[t][h].x, wv[t][h].y, wv[t][h].z, wv[t][h].w);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_lo(wp), widen_lo(xp), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_hi(wp), widen_hi(xp), acc, 0, 0, 0);
            }
        }
    }

    if (KS > 1) {
        if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
        __syncthreads();
        if (wave > 0) return;
#pragma unroll 1
        for (int w = 0; w < KS - 1; ++w) acc += red[w * 64 + lane];
    }

    // epilogue: lane holds acc[r] = 256 y[frow][n0 + 4 fgrp + r] before the scales
    const int m = frow;
    const int nb = n0 + 4 * fgrp;
    if (m >= M || nb >= N) return;
    float sam = 0.0f;
#pragma unroll
    for (int r = 0; r < MR; ++r)
        if (r == m) sam = am[r];
    uint16_t o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = nb + r < N ? nb + r : N - 1;
        float val = ((float)(acc[r] >> 8) * sam) * sb[n];
        if (bias) val = val + bias[n];
        o[r] = f32_to_bf16(val);
    }
    uint16_t *yr = Y + (int64_t)m * ldy + nb;
    if (nb + 3 < N) {
        *reinterpret_cast<uint2 *>(yr) =
            make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
    } else {
        for (int r = 0; r < 4 && nb + r < N; ++r) yr[r] = o[r];
    }
}

template <int KS, int MR, int CPR>
hipError_t launch_layer_cfg(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const float *bias,
                            int64_t m, int64_t n, int64_t k, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                            hipStream_t stream) {
    constexpr int MAXS = 4;
    const size_t lds = (size_t)(KS - 1) * 1024 + kLayerRows * KS * 4 + (size_t)m * (size_t)(k / 2);
    const float c = (float)(1.0 / __builtin_sqrt(128.0));
    const dim3 grid((unsigned)((n + 15) / 16)), block(64 * KS);
    skinny_layer_kernel<KS, MAXS, MR, CPR><<<grid, block, lds, stream>>>(x, ldx, c, w, ws, bias, (int)m, (int)n,
                                                                         (int)k, xq, sx, y, ldy);
    return hipGetLastError();
}

template <int KS>
hipError_t launch_layer_ks(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const float *bias,
                           int64_t m, int64_t n, int64_t k, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                           hipStream_t stream) {
    const int64_t cpr = (k / kElems + 64 * KS - 1) / (64 * KS);  // chunks per row per thread
    if (cpr <= 1) return launch_layer_cfg<KS, 4, 1>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    if (cpr <= 2) return launch_layer_cfg<KS, 2, 2>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    return launch_layer_cfg<KS, 1, 4>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
}

// K-split wavefronts per workgroup, as the skinny GEMM chooses them: about
// one workgroup's worth of waves per SIMD whatever the number of 16-row tiles.
int layer_ks(int64_t n) {
    const int64_t tiles = (n + 15) / 16;
    return tiles >= 1024 ? 2 : tiles >= 512 ? 4 : 8;
}

}  // namespace

bool skinny_layer_fits(int64_t m, int64_t n, int64_t k, int rot_block) {
    if (m < 1 || m > kLayerRows || rot_block != 128 || k < 256 || k % 128 != 0) return false;
    const int64_t cpr = (k / kElems + 64 * layer_ks(n) - 1) / (64 * layer_ks(n));
    const int64_t mr = cpr <= 1 ? 4 : cpr <= 2 ? 2 : cpr <= 4 ? 1 : 0;
    return m <= mr && m * (k / 2) <= 32 * 1024;
}

hipError_t launch_skinny_layer(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const float *bias,
                               int64_t m, int64_t n, int64_t k, int8_t *xq, float *sx, uint16_t *y, int64_t ldy,
                               hipStream_t stream) {
    switch (layer_ks(n)) {
    case 2: return launch_layer_ks<2>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    case 4: return launch_layer_ks<4>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    default: return launch_layer_ks<8>(x, ldx, w, ws, bias, m, n, k, xq, sx, y, ldy, stream);
    }
}

}  // namespace ck4
