// Grouped int4 -> int8 weight decode for gfx950.
//
// What it computes ("[PR #97] HIP port of #90: grouped W4A8 over the INT8
// GEMM", What this adds: int4 codes with per-group fp32 or e4m3 scales are
// decoded to int8 codes that the rowwise int8 GEMM consumes, one lane turning
// 8 packed bytes into 16 int8 with one 16-byte store, optionally through a
// codebook staged in LDS; Chunk sizing: rows [n0, n0+nc) at a time). The int8
// GEMM applies one scale per row in its epilogue, so the decode re-expresses
// the group scales against a row scale:
//   s_row = (max_g s[row, g] * c) / 127
//   w8    = clamp(rint(val(u) * (s[row, g] / s_row)), -127, 127)      (all fp32)
// where u is the 4-bit code, val(u) = q (u as a two's-complement int4) and
// c = 7, or with a codebook val(u) = cb[u] and c = max |cb|. An all-zero row
// (s_row == 0) decodes to zeros. Groups are powers of two from 4 up.
//
// One workgroup per output row: the row scale is a workgroup max-reduction
// over that row's group scales, then each lane decodes 16-element chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"
#include "fp8_e4m3.h"

namespace ck4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int sext4(uint32_t nib) { return (int)(nib ^ 8u) - 8; }

template <bool E4M3, bool CB>
__global__ __launch_bounds__(kThreads) void w4a8_decode_kernel(const int8_t *__restrict__ wp,
                                                               const void *__restrict__ gs, int k, int group,
                                                               int64_t n0, int8_t *__restrict__ w8,
                                                               float *__restrict__ row_scales, Codebook cb) {
    __shared__ float red[kThreads / 64];
    __shared__ float lut[16];
    const int i = blockIdx.x;
    const int64_t row = n0 + i;
    const int tid = threadIdx.x;
    const int ng = k / group;
    auto sg = [&](int g) { return load_scale<E4M3>(gs, row * ng + g); };
    if (CB && tid < 16) lut[tid] = cb.v[tid];

    float smax = 0.0f;
    for (int g = tid; g < ng; g += kThreads) smax = fmaxf(smax, sg(g));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = smax;
    __syncthreads();  // also publishes the codebook
    smax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float srow = (smax * (CB ? cb.cmax : 7.0f)) / 127.0f;
    if (tid == 0) row_scales[i] = srow;

    const int nchunks = k / 16;
    const int8_t *src = wp + row * (int64_t)(k / 2);
    int8_t *dst = w8 + (int64_t)i * k;
    for (int ch = tid; ch < nchunks; ch += kThreads) {
        // multipliers of the chunk's groups: one for groups of 16 and wider,
        // else one per run of 4 elements (groups of 4 or 8)
        float mult[4];
        mult[0] = srow == 0.0f ? 0.0f : sg((ch * 16) / group) / srow;
        if (group >= 16) {
            mult[1] = mult[2] = mult[3] = mult[0];
        } else {
#pragma unroll
            for (int r = 1; r < 4; ++r) mult[r] = srow == 0.0f ? 0.0f : sg((ch * 16 + 4 * r) / group) / srow;
        }
        const uint2 p = *reinterpret_cast<const uint2 *>(src + ch * 8);
        const uint32_t words[2] = {p.x, p.y};
        uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t u = (words[e >> 3] >> (4 * (e & 7))) & 0xFu;
            const float val = CB ? lut[u] : (float)sext4(u);
            float t = rintf(val * mult[e >> 2]);
            t = fminf(fmaxf(t, -127.0f), 127.0f);
            out[e >> 2] |= ((uint32_t)(int)t & 0xFFu) << (8 * (e & 3));
        }
        *reinterpret_cast<uint4 *>(dst + ch * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    }
}

template <bool E4M3>
void launch_decode_typed(const int8_t *w_packed, const void *group_scales, int64_t k, int group, int64_t n0,
                         int64_t nc, int8_t *w8, float *row_scales, hipStream_t stream, const Codebook &cb) {
    if (cb.on)
        w4a8_decode_kernel<E4M3, true><<<dim3((unsigned)nc), dim3(kThreads), 0, stream>>>(
            w_packed, group_scales, (int)k, group, n0, w8, row_scales, cb);
    else
        w4a8_decode_kernel<E4M3, false><<<dim3((unsigned)nc), dim3(kThreads), 0, stream>>>(
            w_packed, group_scales, (int)k, group, n0, w8, row_scales, cb);
}

}  // namespace

hipError_t launch_w4a8_decode(const int8_t *w_packed, const void *group_scales, bool scale_e4m3, int64_t k, int group,
                              int64_t n0, int64_t nc, int8_t *w8, float *row_scales, hipStream_t stream,
                              const Codebook &cb) {
    if (scale_e4m3)
        launch_decode_typed<true>(w_packed, group_scales, k, group, n0, nc, w8, row_scales, stream, cb);
    else
        launch_decode_typed<false>(w_packed, group_scales, k, group, n0, nc, w8, row_scales, stream, cb);
    return hipGetLastError();
}

}  // namespace ck4

// ---------------------------------------------------------------------------
// Fused grouped W4A8 linear for skinny M (M <= 64): the decode above and the
// rowwise int8 GEMM in one kernel, with the decoded int8 weight never leaving
// VGPRs. The int8 codes are the same fp32 operations as the decode kernel, so
// the int32 accumulators, row scales and outputs are identical to decoding
// first. ([PR #97] What this adds decodes a chunk of columns to an int8
// buffer that stays in cache for the GEMM; here the "chunk" is one MFMA
// fragment and the cache is the register file.)
//
// A workgroup owns 16*FNW weight rows; KS wavefronts split K and add their
// int32 partial sums through LDS. The per-code decode costs about five VALU
// instructions (byte convert, fma, clamp, rounding add, byte gather), since
// the kernel is bound by VALU issue rather than by the weight stream.
namespace ck4 {
namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));

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

// Operand layout: a k-step is 256 k. Lane l (row l & 15, part p = l >> 4)
// owns the 64 contiguous k [256 s + 64 p, 256 s + 64 p + 64) of its weight row
// and of its activation row; the MFMA of slice h (0..3) takes 16 of them,
// [.. + 16 h, .. + 16 h + 16), as its 16 bytes. Both operands use the same
// assignment, so each slice's 64 products are 64 distinct k and the four
// slices cover the step. A lane's 64 k lie in one weight group when the group
// is at least 64 wide, which makes the scale division once per step.
// SG = 0 for groups of 16 and wider; SG = 8 or 4 for those narrow groups
// (a multiplier per 8-code word, or per half word). CB: codes index the
// codebook cb.
template <int FM, int FNW, int KS, int MAXS, bool E4M3, int SG, bool CB>
__global__ __launch_bounds__(64 * KS) void w4a8_fused_kernel(const int8_t *__restrict__ X, const float *__restrict__ sx,
                                                           const int8_t *__restrict__ W,
                                                           const void *__restrict__ gs, int M, int N, int K,
                                                           int group, uint16_t *__restrict__ Y, int64_t ldy,
                                                           Codebook cb) {
    constexpr int NGV = SG == 0 ? 4 : 64 / SG;  // group scales per lane and k-step
    __shared__ v4i_t red[KS - 1][FNW][FM][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16 * FNW;
    const int frow = lane & 15;
    const int part = lane >> 4;
    const int ng = K / group;
    const int wrow_bytes = K / 2;
    const int rows_b = min(16 * FNW, N - n0);
    const bool one_group = group >= 64;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(X), (short)0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(W) + (int64_t)n0 * wrow_bytes, (short)0, rows_b * wrow_bytes, 0x00020000);

    // Row scale of this lane's weight rows, (max group scale * 7) / 127: the
    // four lanes of a row split its groups, then combine.
    float srow[FNW];
    int64_t gsr[FNW];  // index of the row's first group scale
#pragma unroll
    for (int i = 0; i < FNW; ++i) {
        const int n = min(n0 + i * 16 + frow, N - 1);
        gsr[i] = (int64_t)n * ng;
        float smax = 0.0f;
        for (int g = part; g < ng; g += 4) smax = fmaxf(smax, load_scale<E4M3>(gs, gsr[i] + g));
        smax = fmaxf(smax, __shfl_xor(smax, 16, 64));
        smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
        srow[i] = (smax * (CB ? cb.cmax : 7.0f)) / 127.0f;
    }

    const int steps = K / 256;
    const int per_wave = (steps + KS - 1) / KS;
    const int s_begin = wave * per_wave;
    const int s_end = min(steps, s_begin + per_wave);

    v4i_t acc[FNW][FM];
#pragma unroll
    for (int i = 0; i < FNW; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i_t{0, 0, 0, 0};

    for (int s0 = s_begin; s0 < s_end; s0 += MAXS) {
        // every load of this chunk first: weights, group scales, activations
        v4i_t wv[MAXS][FNW][2];
        float gv[MAXS][FNW][NGV];
        v4i_t xv[MAXS][FM][4];
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            const int s = s0 + t;
            if (s < s_end) {
                const int kb = s * 256 + part * 64;  // first k of this lane's span
#pragma unroll
                for (int i = 0; i < FNW; ++i) {
                    const uint32_t off = (uint32_t)(i * 16 + frow) * (uint32_t)wrow_bytes + (uint32_t)(kb / 2);
                    wv[t][i][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
                    wv[t][i][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 16, 0);
                    if constexpr (SG != 0) {
#pragma unroll
                        for (int c = 0; c < NGV; ++c) gv[t][i][c] = load_scale<E4M3>(gs, gsr[i] + kb / SG + c);
                    } else if (one_group) {
                        const float g0 = load_scale<E4M3>(gs, gsr[i] + kb / group);
#pragma unroll
                        for (int h = 0; h < 4; ++h) gv[t][i][h] = g0;
                    } else {
#pragma unroll
                        for (int h = 0; h < 4; ++h) gv[t][i][h] = load_scale<E4M3>(gs, gsr[i] + (kb + 16 * h) / group);
                    }
                }
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const uint32_t off = (uint32_t)(j * 16 + frow) * (uint32_t)K + (uint32_t)kb;
#pragma unroll
                    for (int h = 0; h < 4; ++h) xv[t][j][h] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 16 * h, 0);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            if (s0 + t >= s_end) break;
#pragma unroll
            for (int i = 0; i < FNW; ++i) {
                const uint32_t words[8] = {(uint32_t)wv[t][i][0][0], (uint32_t)wv[t][i][0][1],
                                           (uint32_t)wv[t][i][0][2], (uint32_t)wv[t][i][0][3],
                                           (uint32_t)wv[t][i][1][0], (uint32_t)wv[t][i][1][1],
                                           (uint32_t)wv[t][i][1][2], (uint32_t)wv[t][i][1][3]};
                if constexpr (SG != 0) {
                    // groups of 8 or 4: a multiplier per word or per half word
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        uint2 d[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int wi = 2 * h + e;
                            const int ga = SG == 8 ? wi : 2 * wi, gb = SG == 8 ? wi : 2 * wi + 1;
                            const float ma = srow[i] == 0.0f ? 0.0f : gv[t][i][ga] / srow[i];
                            const float mb = SG == 8 ? ma : (srow[i] == 0.0f ? 0.0f : gv[t][i][gb] / srow[i]);
                            if constexpr (CB) {
                                const uint4 ta = code_table_cb(ma, cb);
                                d[e] = SG == 8 ? decode8_table(words[wi], ta)
                                               : decode8_table2(words[wi], ta, code_table_cb(mb, cb));
                            } else {
                                d[e] = decode8_2(words[wi], ma, -8.0f * ma, mb, -8.0f * mb);
                            }
                        }
                        const v4i_t w8 = v4i_t{(int)d[0].x, (int)d[0].y, (int)d[1].x, (int)d[1].y};
#pragma unroll
                        for (int j = 0; j < FM; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[t][j][h], acc[i][j], 0, 0, 0);
                    }
                    continue;
                }
                if (one_group) {
                    // one multiplier for the lane's 64 codes: table decode
                    const float mu = srow[i] == 0.0f ? 0.0f : gv[t][i][0] / srow[i];
                    uint4 tab;
                    if constexpr (CB) tab = code_table_cb(mu, cb);
                    else tab = code_table(mu);
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint2 a = decode8_table(words[2 * h], tab);
                        const uint2 b = decode8_table(words[2 * h + 1], tab);
                        const v4i_t w8 = v4i_t{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
#pragma unroll
                        for (int j = 0; j < FM; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[t][j][h], acc[i][j], 0, 0, 0);
                    }
                    continue;
                }
                // groups of 16 and 32: a multiplier per 16 codes
                if constexpr (CB) {
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint4 tab = code_table_cb(srow[i] == 0.0f ? 0.0f : gv[t][i][h] / srow[i], cb);
                        const uint2 a = decode8_table(words[2 * h], tab);
                        const uint2 b = decode8_table(words[2 * h + 1], tab);
                        const v4i_t w8 = v4i_t{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
#pragma unroll
                        for (int j = 0; j < FM; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[t][j][h], acc[i][j], 0, 0, 0);
                    }
                    continue;
                }
                // per-code decode
                float mult[4], m8[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    mult[h] = srow[i] == 0.0f ? 0.0f : gv[t][i][h] / srow[i];
                    m8[h] = -8.0f * mult[h];
                }
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint2 a = decode8(words[2 * h], mult[h], m8[h]);
                    const uint2 b = decode8(words[2 * h + 1], mult[h], m8[h]);
                    const v4i_t w8 = v4i_t{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
#pragma unroll
                    for (int j = 0; j < FM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[t][j][h], acc[i][j], 0, 0, 0);
                }
            }
        }
    }

    if (KS > 1) {
        if (wave > 0) {
#pragma unroll
            for (int i = 0; i < FNW; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) red[wave - 1][i][j][lane] = acc[i][j];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll 1
        for (int w = 0; w < KS - 1; ++w)
#pragma unroll
            for (int i = 0; i < FNW; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] += red[w][i][j][lane];
    }

    // Epilogue: lane holds acc[i][j][r] = y[m][n], m = 16j + (l & 15),
    // n = n0 + 16i + 4(l >> 4) + r; the weight scale of row n is its s_row,
    // which lives in lane (n - n0 - 16i) of the same 16-lane group.
#pragma unroll
    for (int i = 0; i < FNW; ++i) {
        float sw4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sw4[r] = __shfl(srow[i], 4 * part + r, 64);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = j * 16 + frow;
            const int nb = n0 + i * 16 + 4 * part;
            if (m >= M || nb >= N) continue;
            const float sam = sx[m];
            uint16_t o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = bf16_rne(((float)acc[i][j][r] * sam) * sw4[r]);
            uint16_t *yr = Y + (int64_t)m * ldy + nb;
            if (nb + 3 < N) {
                *reinterpret_cast<uint2 *>(yr) =
                    make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
            } else {
                for (int r = 0; r < 4 && nb + r < N; ++r) yr[r] = o[r];
            }
        }
    }
}

template <int FM, int FNW, int MAXS, bool E4M3, int SG, bool CB>
hipError_t launch_fused_cfg(const int8_t *x, const float *sx, const int8_t *w, const void *gs, int64_t m, int64_t n,
                            int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream, const Codebook &cb) {
    const int64_t groups = (n + 16 * FNW - 1) / (16 * FNW);
    dim3 grid((unsigned)groups);
    if constexpr (SG != 0 || CB) {
        // narrow groups and codebooks: one K split (4 wavefronts) for every width
        w4a8_fused_kernel<FM, FNW, 4, MAXS, E4M3, SG, CB><<<grid, dim3(256), 0, stream>>>(
            x, sx, w, gs, (int)m, (int)n, (int)k, group, y, ldy, cb);
    } else if (groups >= 1024) {
        w4a8_fused_kernel<FM, FNW, 2, MAXS, E4M3, 0, false><<<grid, dim3(128), 0, stream>>>(
            x, sx, w, gs, (int)m, (int)n, (int)k, group, y, ldy, cb);
    } else if (groups >= 512) {
        w4a8_fused_kernel<FM, FNW, 4, MAXS, E4M3, 0, false><<<grid, dim3(256), 0, stream>>>(
            x, sx, w, gs, (int)m, (int)n, (int)k, group, y, ldy, cb);
    } else {
        w4a8_fused_kernel<FM, FNW, 8, MAXS, E4M3, 0, false><<<grid, dim3(512), 0, stream>>>(
            x, sx, w, gs, (int)m, (int)n, (int)k, group, y, ldy, cb);
    }
    return hipGetLastError();
}

template <bool E4M3, int SG, bool CB>
hipError_t launch_fused(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed, const void *group_scales,
                        int64_t m, int64_t n, int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream,
                        const Codebook &cb) {
    if (m <= 16)
        return launch_fused_cfg<1, 1, 2, E4M3, SG, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy,
                                                        stream, cb);
    if (m <= 32)
        return launch_fused_cfg<2, 1, 2, E4M3, SG, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy,
                                                        stream, cb);
    // 64-row activations: two weight tiles per workgroup (half the
    // activation re-reads) when the weight has fewer than 512 tiles; with
    // more, the extra workgroups win (N = 5120: 33.1 -> 25.4 us, N = 12288:
    // 26.4 -> 32.3 us at M = 64)
    if ((n + 15) / 16 < 512)
        return launch_fused_cfg<4, 2, 1, E4M3, SG, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y,
                                                        ldy, stream, cb);
    return launch_fused_cfg<4, 1, 1, E4M3, SG, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy,
                                                    stream, cb);
}

template <bool E4M3, bool CB>
hipError_t launch_fused_groups(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                               const void *group_scales, int64_t m, int64_t n, int64_t k, int group, uint16_t *y,
                               int64_t ldy, hipStream_t stream, const Codebook &cb) {
    if (group == 4)
        return launch_fused<E4M3, 4, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream, cb);
    if (group == 8)
        return launch_fused<E4M3, 8, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream, cb);
    return launch_fused<E4M3, 0, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream, cb);
}

template <bool E4M3>
hipError_t launch_fused_cb(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed, const void *group_scales,
                           int64_t m, int64_t n, int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream,
                           const Codebook &cb) {
    if (cb.on)
        return launch_fused_groups<E4M3, true>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream,
                                               cb);
    return launch_fused_groups<E4M3, false>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream,
                                            cb);
}

}  // namespace

hipError_t launch_w4a8_fused(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                             const void *group_scales, bool scale_e4m3, int64_t m, int64_t n, int64_t k, int group,
                             uint16_t *y, int64_t ldy, hipStream_t stream, const Codebook &cb) {
    if (scale_e4m3)
        return launch_fused_cb<true>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream, cb);
    return launch_fused_cb<false>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream, cb);
}

}  // namespace ck4
