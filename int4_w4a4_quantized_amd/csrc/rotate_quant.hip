// Fused ConvRot rotation + symmetric quantisation + packing, one row per
// wavefront (or per workgroup for long rows), for gfx950.
//
// What it computes ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with
// fused CUDA kernels", Description: the activation kernel rotates, takes the
// row scale, quantises to int4 and packs in a single pass; weights are stored
// as int4 code pairs, the even element in the low nibble, with one fp32 scale
// per row):
//   r = x * blockdiag(H_b, ..., H_b) * fp32(1/sqrt(b))     (fp32, b = rot_block)
//   s = absmax(r) / qmax                                  (fp32 divide)
//   q = clamp(rint(r / s), -qmax, qmax)                    (fp32 quotient, ties to even)
// with H_b the Sylvester Hadamard matrix and the butterflies taken with
// ascending stride, so the fp32 rotation is one fixed sequence of roundings.
//
// Data layout in registers: each lane owns "chunks" of 16 contiguous elements
// of the row. Chunk c of a row covers elements [16c, 16c + 16); chunk c is
// owned by thread c mod T of the row's T threads. A row of up to 4096
// elements belongs to one wavefront (T = 64, four rows per workgroup), so its
// absmax needs no barrier and every row of a 4608-row batch is resident at
// once; a longer row, or a row of 2048 elements or more in a batch of at
// most 2048 rows, of 4096 elements, or quantised to FP6 codes, belongs to a
// whole workgroup (T = blockDim). A Hadamard
// block of b elements is b/16 consecutive chunks, which sit in b/16
// consecutive lanes of one wavefront (T is a multiple of 64 and b <= 1024).
// Butterfly strides 1..8 are inside a lane; stride 16*m pairs lane L with
// lane L ^ m. The whole row stays in VGPRs between the rotation and the
// quantisation, so HBM is read once and written once.
//
// Cross-lane butterflies with one instruction per element. A butterfly keeps
// a + b in the lower lane and a - b in the upper one. Each lane instead keeps
// u = sigma * v for a known sign sigma and computes u' = u + k * u_partner
// with k = -1 in the upper lane and +1 in the lower one: one fused
// multiply-add whose product is exact (k = +-1), so u' is the correctly
// rounded sum, equal to sigma' times the butterfly output because IEEE
// round-to-nearest commutes with negation. After all cross-lane stages,
// sigma = (-1)^popcount(lane & (b/16 - 1)); it is folded into the final
// multiply by the normalisation constant, so the rotated values are bitwise
// those of the plain butterflies (up to the sign of an exact zero). The
// partner value comes through ds_swizzle (strides 16 to 256) or ds_bpermute
// (512), which use the LDS crossbar and leave the VALU to the arithmetic.
//
// The quotient r / s without a divide per element. With y = RN(1/s) computed
// once per row by the IEEE divide, q0 = RN(r y), e = fma(-q0, s, r) (exact),
// q1 = fma(e, y, q0) is the correctly rounded r / s (Markstein's division
// theorem); it is used when s is a normal number in [2^-120, 2^120], where no
// step overflows or underflows, and the IEEE divide is used otherwise.
// Rounding to the nearest integer (ties to even) is one fp32 addition of
// 1.5 * 2^23: for |q1| < 2^22 the sum's bit pattern is 0x4B400000 + rint(q1),
// whose low byte is the two's-complement int8 code and whose low nibble is
// the int4 code. |q1| <= qmax (1 + 2^-23) when s is normal, so no clamp is
// needed on that path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"
#include "fp8_e4m3.h"
#include "fwht.h"
#include "quant_codes.h"

namespace ck4 {
namespace {

constexpr int kMaxChunks = 4;  // chunks per thread: k <= 16 * 256 * 4 = 16384
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef int v6i_t __attribute__((ext_vector_type(6)));
constexpr int kThreads = 256;
// The kernel is instantiated per chunks-per-thread count NCH (1..4), so a row
// of K <= 4096 keeps 16 values per lane in VGPRs and the occupancy stays high.

// Stochastic rounding with a caller-supplied draw uv in [0, 1):
// clamp(floor(RN(r / s) + uv), -qmax, qmax) in fp32, biased like code_exact.
template <int BIAS>
__device__ __forceinline__ uint32_t code_sr(float r, float s, float uv, float qmax) {
    if (s == 0.0f) return (uint32_t)BIAS;
    const float x = r / s;
    float t = floorf(x + uv);
    t = fminf(fmaxf(t, -qmax), qmax);
    return (uint32_t)((int)t + BIAS);
}

// Codebook code of r / s, biased like code_exact<8> (the low byte is u ^ 8,
// so pack8_biased stores the index u): the entry u nearest to t = r / s
// (IEEE quotient; t = 0 when s == 0) by the fp32 distance |t - v[u]|, the
// lowest index among equal distances.
__device__ __forceinline__ uint32_t code_codebook(float r, float s, const Codebook &cb) {
    const float t = s == 0.0f ? 0.0f : r / s;
    float best = fabsf(t - cb.v[0]);
    uint32_t u = 0;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        const float d = fabsf(t - cb.v[i]);
        if (d < best) {
            best = d;
            u = (uint32_t)i;
        }
    }
    return u ^ 8u;
}

// Scale of one weight group: absmax / qdiv, or its E4M3 rounding (stored as
// a byte, and the decoded value is what the codes use). Stored by the caller's
// `store` flag at scales[si].
__device__ __forceinline__ float group_scale(float gmax, float qdiv, bool e4m3, bool store, float *scales,
                                             int64_t si) {
    float s = gmax / qdiv;
    if (e4m3) {
        const uint32_t b = e4m3_encode(s);
        s = e4m3_decode(b);
        if (store) reinterpret_cast<uint8_t *>(scales)[si] = (uint8_t)b;
    } else if (store) {
        scales[si] = s;
    }
    return s;
}

// out_kind: 0 packed int4, 1 int8 codes, 2 fp32 rotation, 3 bf16 rotation in MFMA fragment order,
// 4 FP6 operand image, 5 its compact form.
// WAVE_ROW: each wavefront owns one row (K <= 64 * 16 * NCH), so the row
// absmax is a wavefront reduction with no LDS and no barrier, and a 256-thread
// workgroup handles 4 rows; otherwise the workgroup owns one row.
template <typename TIn, int OUT, int NCH, bool WAVE_ROW, int LPB>
__global__ __launch_bounds__(kThreads) void rotate_quant_kernel(const TIn *__restrict__ x, int64_t rows, int64_t ldx,
                                                                  int k, float c, int group, void *__restrict__ out,
                                                                  int64_t ldo, float *__restrict__ scales,
                                                                  WeightOpts wo) {
    __shared__ float red[kThreads / 64];
    const int lane = threadIdx.x & 63;
    int64_t wg = blockIdx.x;
    if constexpr (OUT == 4 || OUT == 5) {
        // FP6 blocks span 16 rows: 4 workgroups of 4 rows, or 16 workgroups
        // of one row. Workgroup ids are dealt round-robin to the 8 XCDs
        // (id & 7), each with its own L2; remap so that the workgroups of a
        // block share an XCD and their partial 24-byte writes of each line
        // meet in one L2.
        const int64_t b = blockIdx.x, j = b >> 3;
        if (WAVE_ROW && (gridDim.x & 31) == 0 && blockDim.x == 256) wg = ((j >> 2) * 8 + (b & 7)) * 4 + (j & 3);
        if (!WAVE_ROW && (gridDim.x & 127) == 0) wg = ((j >> 4) * 8 + (b & 7)) * 16 + (j & 15);
    }
    const int64_t row = WAVE_ROW ? wg * (blockDim.x / 64) + (threadIdx.x >> 6) : wg;
    if (WAVE_ROW && row >= rows) return;  // whole wavefronts only; this mode has no barrier
    const int tid = WAVE_ROW ? lane : (int)threadIdx.x;
    const int nthreads = WAVE_ROW ? 64 : (int)blockDim.x;
    const int nchunks = k / kElems;
    const TIn *xr = x + (int64_t)row * ldx;
    // the sign carried by the cross-lane stages, folded into the scale
    const float c_lane = (__popc(lane & (LPB - 1)) & 1) ? -c : c;

    float v[NCH][kElems];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int ch = tid + j * nthreads;
        if (ch < nchunks) {
            load_chunk(xr + (int64_t)ch * kElems, v[j]);
            fwht_in_lane(v[j]);
            fwht_cross_lane<LPB>(v[j], lane);
#pragma unroll
            for (int i = 0; i < kElems; ++i) {
                v[j][i] = v[j][i] * c_lane;
                amax = fmaxf(amax, fabsf(v[j][i]));
            }
        }
    }

    if constexpr (OUT == 2) {
        float *o = reinterpret_cast<float *>(out) + (int64_t)row * ldo;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int ch = tid + j * nthreads;
            if (ch < nchunks) {
                float4 *d = reinterpret_cast<float4 *>(o + (int64_t)ch * kElems);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    d[i] = make_float4(v[j][4 * i], v[j][4 * i + 1], v[j][4 * i + 2], v[j][4 * i + 3]);
            }
        }
        return;
    } else if constexpr (OUT == 3) {
        // the rotation rounded once to bf16 (nearest even), stored in MFMA
        // fragment order: 16-row x 32-column tiles of 512 values, tile
        // (row / 16, col / 32) at ((row / 16) * (k / 32) + col / 32) * 512,
        // element (i, c) of a tile at (16 ((c >> 2) & 3) + i) * 8 + 4 (c >> 4) + (c & 3).
        // A 16-value chunk is half a tile row: four runs of 4 values, 8 bytes each.
        uint16_t *o = reinterpret_cast<uint16_t *>(out) + ((row >> 4) * (int64_t)(k / 32)) * 512 + (row & 15) * 8;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int ch = tid + j * nthreads;
            if (ch < nchunks) {
                uint16_t *tile = o + (int64_t)(ch >> 1) * 512 + 4 * (ch & 1);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[j][4 * q]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[j][4 * q + 1]) << 16);
                    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[j][4 * q + 2]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[j][4 * q + 3]) << 16);
                    *reinterpret_cast<uint2 *>(tile + 16 * q * 8) = make_uint2(lo, hi);
                }
            }
        }
        return;
    } else {
        const float qmax = OUT == 0 || OUT == 4 || OUT == 5 ? 7.0f : 127.0f;
        constexpr int BIAS = OUT == 0 ? 8 : 0;
        float s_row = 0.0f, y_row = 0.0f;
        bool fast_row = false;
        if (group == 0) {
            // absmax over the whole row: wavefront reduction, then across waves.
            amax = wave_max(amax);
            if constexpr (!WAVE_ROW) {
                if (lane == 0) red[tid >> 6] = amax;
                __syncthreads();
                amax = red[0];
                for (int w = 1; w < nthreads / 64; ++w) amax = fmaxf(amax, red[w]);
            }
            s_row = amax / qmax;
            fast_row = s_row >= 0x1p-120f && s_row <= 0x1p120f;
            y_row = fast_row ? 1.0f / s_row : 0.0f;
            if (tid == 0) scales[row] = s_row;
        }
        if constexpr (OUT == 4 || OUT == 5) {
            // int4 codes as FP6 E2M3 values q/8 (sign bit 5, |q| in bits 0-2: a
            // subnormal, exact), in the MFMA operand image: a 16-value chunk is
            // 96 bits at byte 12 (ch & 1) of lane image 16 ((ch >> 1) & 3) + (row & 15)
            // of block (row / 16, ch / 8), 1536 bytes per block, fields LSB-first.
            // q is formed as an integer-valued float (the rounding add of 1.5 * 2^23
            // and its subtraction are exact for |q| <= 7), and the hardware
            // converter packs two chunks at once: it divides by its scale (8) and
            // interleaves its sources (field 2i from the first, 2i + 1 from the
            // second), so the even elements of both chunks go in the first source.
            // The compact form (OUT == 5) keeps 8 of each chunk's 12 bytes: its
            // dwords V0, V1, V2 become V0 | (V1 & Z0), V2 | (V1 & Z2) (Z0, Z2 the
            // zero exponent bits of V0 and V2), in 1024-byte blocks of 16-byte
            // lane images.
            constexpr int BLK = OUT == 5 ? 1024 : 1536;
            constexpr int IMG = BLK / 64;
            constexpr int CHB = IMG / 2;  // bytes of a 16-value chunk
            uint8_t *o = reinterpret_cast<uint8_t *>(out) + (row >> 4) * (int64_t)(k / 128) * BLK + (row & 15) * IMG;
            float qf[NCH][kElems];
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                if (fast_row) {
#pragma unroll
                    for (int i = 0; i < kElems; ++i) {
                        const float q0 = v[j][i] * y_row;
                        const float e = __builtin_fmaf(-q0, s_row, v[j][i]);
                        const float q1 = __builtin_fmaf(e, y_row, q0);
                        qf[j][i] = (q1 + 12582912.0f) - 12582912.0f;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < kElems; ++i)
                        qf[j][i] = s_row == 0.0f ? 0.0f : fminf(fmaxf(rintf(v[j][i] / s_row), -qmax), qmax);
                }
            }
#pragma unroll
            for (int j = 0; j < NCH; j += 2) {
                const int j1 = j + 1 < NCH ? j + 1 : j;  // an odd count pairs the last chunk with itself
                v16f_t ev, od;
#pragma unroll
                for (int i = 0; i < kElems / 2; ++i) {
                    ev[i] = qf[j][2 * i];
                    od[i] = qf[j][2 * i + 1];
                    ev[8 + i] = qf[j1][2 * i];
                    od[8 + i] = qf[j1][2 * i + 1];
                }
                const v6i_t p6 = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 8.0f);
                const int ch0 = tid + j * nthreads, ch1 = tid + j1 * nthreads;
                uint8_t *d0 = o + (int64_t)(ch0 >> 3) * BLK + ((ch0 >> 1) & 3) * 16 * IMG + (ch0 & 1) * CHB;
                uint8_t *d1 = o + (int64_t)(ch1 >> 3) * BLK + ((ch1 >> 1) & 3) * 16 * IMG + (ch1 & 1) * CHB;
                if constexpr (OUT == 5) {
                    constexpr uint32_t Z0 = 0x18618618u, Z2 = 0x61861861u;
                    const uint32_t a1 = (uint32_t)p6[1], b1 = (uint32_t)p6[4];
                    if (ch0 < nchunks)
                        *reinterpret_cast<uint2 *>(d0) = make_uint2((uint32_t)p6[0] | (a1 & Z0), (uint32_t)p6[2] | (a1 & Z2));
                    if (j1 != j && ch1 < nchunks)
                        *reinterpret_cast<uint2 *>(d1) = make_uint2((uint32_t)p6[3] | (b1 & Z0), (uint32_t)p6[5] | (b1 & Z2));
                } else {
                    if (ch0 < nchunks) *reinterpret_cast<uint3 *>(d0) = make_uint3(p6[0], p6[1], p6[2]);
                    if (j1 != j && ch1 < nchunks) *reinterpret_cast<uint3 *>(d1) = make_uint3(p6[3], p6[4], p6[5]);
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int ch = tid + j * nthreads;
            if (ch >= nchunks) continue;
            uint32_t code[kElems];
            // stochastic rounding (weights only): one draw per element
            float uv[kElems];
            const bool sr = sizeof(TIn) == 4 && wo.u != nullptr;
            if (sr) {
                const float4 *up = reinterpret_cast<const float4 *>(wo.u + row * wo.ldu + (int64_t)ch * kElems);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 t = up[i];
                    uv[4 * i] = t.x;
                    uv[4 * i + 1] = t.y;
                    uv[4 * i + 2] = t.z;
                    uv[4 * i + 3] = t.w;
                }
            }
            if (group == 0 && sr) {
#pragma unroll
                for (int i = 0; i < kElems; ++i) code[i] = code_sr<BIAS>(v[j][i], s_row, uv[i], qmax);
            } else if (group == 0) {
                if (fast_row) {
#pragma unroll
                    for (int i = 0; i < kElems; ++i) code[i] = code_fast<BIAS>(v[j][i], s_row, y_row);
                } else {
#pragma unroll
                    for (int i = 0; i < kElems; ++i) code[i] = code_exact<BIAS>(v[j][i], s_row, qmax);
                }
            } else if constexpr (sizeof(TIn) == 4) {
                // Grouped weight codes (offline preparation: the IEEE divide
                // throughout). sv[i] is the scale of element i of the chunk.
                const float qdiv = wo.cb.on ? wo.cb.cmax : qmax;
                const int64_t gbase = (int64_t)row * (k / group);
                float sv[kElems];
                if (group >= kElems) {
                    // one scale per `group` elements = group/16 consecutive lanes
                    float gmax = 0.0f;
#pragma unroll
                    for (int i = 0; i < kElems; ++i) gmax = fmaxf(gmax, fabsf(v[j][i]));
                    for (int off = 1; off < group / kElems; off <<= 1) gmax = fmaxf(gmax, __shfl_xor(gmax, off, 64));
                    const int lanes_per_group = group / kElems;
                    const float sg = group_scale(gmax, qdiv, wo.scale_e4m3, (ch % lanes_per_group) == 0, scales,
                                                 gbase + ch / lanes_per_group);
#pragma unroll
                    for (int i = 0; i < kElems; ++i) sv[i] = sg;
                } else {
                    // groups of 4 or 8 inside the chunk: absmax of each run of 4
                    float gm[kElems / 4];
#pragma unroll
                    for (int sb = 0; sb < kElems / 4; ++sb) {
                        gm[sb] = 0.0f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) gm[sb] = fmaxf(gm[sb], fabsf(v[j][4 * sb + i]));
                    }
                    const int per_chunk = kElems / group;
#pragma unroll
                    for (int sb = 0; sb < kElems / 4; ++sb) {
                        // group 8: run sb joins its partner sb ^ 1
                        const float gmax = group == 8 ? fmaxf(gm[sb], gm[sb ^ 1]) : gm[sb];
                        const int gi = group == 8 ? sb >> 1 : sb;
                        const bool first = group == 8 ? (sb & 1) == 0 : true;
                        const float sg = group_scale(gmax, qdiv, wo.scale_e4m3, first, scales,
                                                     gbase + (int64_t)ch * per_chunk + gi);
#pragma unroll
                        for (int i = 0; i < 4; ++i) sv[4 * sb + i] = sg;
                    }
                }
                if (wo.cb.on) {
#pragma unroll
                    for (int i = 0; i < kElems; ++i) code[i] = code_codebook(v[j][i], sv[i], wo.cb);
                } else if (sr) {
#pragma unroll
                    for (int i = 0; i < kElems; ++i) code[i] = code_sr<BIAS>(v[j][i], sv[i], uv[i], qmax);
                } else {
#pragma unroll
                    for (int i = 0; i < kElems; ++i) code[i] = code_exact<BIAS>(v[j][i], sv[i], qmax);
                }
            }
            if constexpr (OUT == 0) {
                const uint32_t w0 = pack8_biased(code), w1 = pack8_biased(code + 8);
                int8_t *o = reinterpret_cast<int8_t *>(out) + (int64_t)row * ldo + (int64_t)ch * (kElems / 2);
                *reinterpret_cast<uint2 *>(o) = make_uint2(w0, w1);
            } else {
                int8_t *o = reinterpret_cast<int8_t *>(out) + (int64_t)row * ldo + (int64_t)ch * kElems;
                *reinterpret_cast<uint4 *>(o) =
                    make_uint4(pack4_bytes(code), pack4_bytes(code + 4), pack4_bytes(code + 8), pack4_bytes(code + 12));
            }
        }
    }
}

template <typename TIn, int OUT, bool WAVE_ROW, int LPB>
void launch_lpb(const TIn *x, int nch, dim3 grid, dim3 block, int64_t rows, int64_t ldx, int k, float c, int group,
                void *out, int64_t ldo, float *scales, WeightOpts wo, hipStream_t stream) {
    switch (nch) {
    case 1:
        rotate_quant_kernel<TIn, OUT, 1, WAVE_ROW, LPB><<<grid, block, 0, stream>>>(x, rows, ldx, k, c, group, out,
                                                                                     ldo, scales, wo);
        break;
    case 2:
        rotate_quant_kernel<TIn, OUT, 2, WAVE_ROW, LPB><<<grid, block, 0, stream>>>(x, rows, ldx, k, c, group, out,
                                                                                     ldo, scales, wo);
        break;
    case 3:
        rotate_quant_kernel<TIn, OUT, 3, WAVE_ROW, LPB><<<grid, block, 0, stream>>>(x, rows, ldx, k, c, group, out,
                                                                                     ldo, scales, wo);
        break;
    default:
        rotate_quant_kernel<TIn, OUT, 4, WAVE_ROW, LPB><<<grid, block, 0, stream>>>(x, rows, ldx, k, c, group, out,
                                                                                     ldo, scales, wo);
        break;
    }
}

template <typename TIn, int OUT, bool WAVE_ROW>
void launch_out(const TIn *x, int nch, dim3 grid, dim3 block, int64_t rows, int64_t ldx, int k, int lanes_per_block,
                float c, int group, void *out, int64_t ldo, float *scales, WeightOpts wo, hipStream_t stream) {
    switch (lanes_per_block) {
    case 1: launch_lpb<TIn, OUT, WAVE_ROW, 1>(x, nch, grid, block, rows, ldx, k, c, group, out, ldo, scales, wo, stream); break;
    case 2: launch_lpb<TIn, OUT, WAVE_ROW, 2>(x, nch, grid, block, rows, ldx, k, c, group, out, ldo, scales, wo, stream); break;
    case 4: launch_lpb<TIn, OUT, WAVE_ROW, 4>(x, nch, grid, block, rows, ldx, k, c, group, out, ldo, scales, wo, stream); break;
    case 8: launch_lpb<TIn, OUT, WAVE_ROW, 8>(x, nch, grid, block, rows, ldx, k, c, group, out, ldo, scales, wo, stream); break;
    case 16: launch_lpb<TIn, OUT, WAVE_ROW, 16>(x, nch, grid, block, rows, ldx, k, c, group, out, ldo, scales, wo, stream); break;
    case 32: launch_lpb<TIn, OUT, WAVE_ROW, 32>(x, nch, grid, block, rows, ldx, k, c, group, out, ldo, scales, wo, stream); break;
    default: launch_lpb<TIn, OUT, WAVE_ROW, 64>(x, nch, grid, block, rows, ldx, k, c, group, out, ldo, scales, wo, stream); break;
    }
}

template <typename TIn, int OUT>
void launch_mode(const TIn *x, int nch, bool wave_row, int64_t rows, int64_t ldx, int k, int lanes_per_block, float c,
                 int group, void *out, int64_t ldo, float *scales, WeightOpts wo, hipStream_t stream) {
    if (wave_row) {
        const dim3 grid((unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64))), block(kThreads);
        launch_out<TIn, OUT, true>(x, nch, grid, block, rows, ldx, k, lanes_per_block, c, group, out, ldo, scales,
                                   wo, stream);
    } else {
        const int nchunks = k / kElems;
        int threads = (nchunks + nch - 1) / nch;
        threads = (threads + 63) / 64 * 64;
        const dim3 grid((unsigned)rows), block((unsigned)threads);
        launch_out<TIn, OUT, false>(x, nch, grid, block, rows, ldx, k, lanes_per_block, c, group, out, ldo, scales,
                                    wo, stream);
    }
}

template <typename TIn>
hipError_t launch_typed(const TIn *x, int64_t rows, int64_t k, int64_t ldx, int rot_block, int out_kind, int group,
                        void *out, int64_t ldo, float *scales, WeightOpts wo, hipStream_t stream) {
    const int nchunks = (int)(k / kElems);
    // A row fits one wavefront when it is at most 64 lanes x kMaxChunks
    // chunks. Rows of 128 chunks or more are spread over a workgroup of up to
    // four wavefronts instead (same arithmetic, same bits) where that
    // measured faster: with few rows, where the GPU is mostly idle and each
    // row's latency chain (loads, butterflies, absmax, codes) is the time
    // (K = 3072, 1-2048 rows: 4.1-5.2 -> 2.6-4.7 us); at 256 chunks (K =
    // 4096: 4608 rows 11.6 -> 11.3 us); and for the FP6 codes at any count
    // (K = 3072, 4608 rows: 9.8 -> 9.5 us). Packed int4 codes of 4608 rows at
    // K = 3072 stay a wavefront per row (8.4 against 8.5 us); K = 1024 gains
    // nothing.
    const bool wg_row = nchunks >= 128 && (rows <= 2048 || nchunks >= 256 || out_kind == 4 || out_kind == 5);
    const bool wave_row = nchunks <= 64 * kMaxChunks && !wg_row;
    const int per_thread = wave_row ? (nchunks + 63) / 64 : (nchunks + kThreads - 1) / kThreads;  // 1..kMaxChunks
    const float c = (float)(1.0 / __builtin_sqrt((double)rot_block));
    const int lanes_per_block = rot_block / kElems;
    if (out_kind == 0)
        launch_mode<TIn, 0>(x, per_thread, wave_row, rows, ldx, (int)k, lanes_per_block, c, group, out, ldo, scales,
                            wo, stream);
    else if (out_kind == 1)
        launch_mode<TIn, 1>(x, per_thread, wave_row, rows, ldx, (int)k, lanes_per_block, c, group, out, ldo, scales,
                            wo, stream);
    else if (out_kind == 3)
        launch_mode<TIn, 3>(x, per_thread, wave_row, rows, ldx, (int)k, lanes_per_block, c, group, out, ldo, scales,
                            wo, stream);
    else if (out_kind == 4)
        launch_mode<TIn, 4>(x, per_thread, wave_row, rows, ldx, (int)k, lanes_per_block, c, group, out, ldo, scales,
                            wo, stream);
    else if (out_kind == 5)
        launch_mode<TIn, 5>(x, per_thread, wave_row, rows, ldx, (int)k, lanes_per_block, c, group, out, ldo, scales,
                            wo, stream);
    else if constexpr (sizeof(TIn) == 4)
        return hipErrorInvalidValue;  // fp32 rows: codes or the bf16 rotation only
    else
        launch_mode<TIn, 2>(x, per_thread, wave_row, rows, ldx, (int)k, lanes_per_block, c, group, out, ldo, scales,
                            wo, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant(const void *x, int in_kind, int64_t rows, int64_t k, int64_t ldx, int rot_block,
                               int out_kind, int group, void *out, int64_t ldo, float *scales, hipStream_t stream,
                               WeightOpts wo) {
    if (in_kind == 0)
        return launch_typed(static_cast<const uint16_t *>(x), rows, k, ldx, rot_block, out_kind, group, out, ldo,
                            scales, WeightOpts{}, stream);
    return launch_typed(static_cast<const float *>(x), rows, k, ldx, rot_block, out_kind, group, out, ldo, scales, wo,
                        stream);
}

}  // namespace ck4
