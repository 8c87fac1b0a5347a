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
// Groups of 32 codes or more with rows of up to 8192 codes take a wavefront
// per row instead (w4a8_decode_rows_kernel below).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "ck4_kernels.h"
#include "fp8_e4m3.h"
#include "w4a8_codes.h"

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

// The same decode with a wavefront per row, for groups of 32 codes or more
// and rows of up to 8192 codes: lane l takes the 32-code chunks l, l + 64,
// ... (CPL of them), one 16-byte load of codes and one group-scale load
// each, all issued before the first is used; since every group has a chunk,
// the wavefront maximum of the lane's scales is the row's, with no barrier.
// A chunk's 16 possible int8 codes are tabulated once for its multiplier
// with the same fp32 steps (w4a8_codes.h) and looked up per code, and its 32
// codes leave as two 16-byte stores. Four rows per workgroup.
template <int CPL, bool E4M3>
__global__ __launch_bounds__(256) void w4a8_decode_rows_kernel(const int8_t *__restrict__ wp,
                                                               const void *__restrict__ gs, int k, int group,
                                                               int64_t n0, int nc, int8_t *__restrict__ w8,
                                                               float *__restrict__ row_scales) {
    constexpr int SB = E4M3 ? 1 : 4;  // bytes per group scale
    constexpr uint32_t kOob = 0x40000000u;  // beyond any row here: the load returns zeros
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (i >= nc) return;  // whole wavefronts; no barrier in this kernel
    const int64_t row = n0 + i;
    const int row_bytes = k / 2;
    const int nch = k / 32;
    const int ng = k / group;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(static_cast<const int8_t *>(gs) + row * ng * SB), (short)0, ng * SB, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(wp + row * row_bytes), (short)0, row_bytes, 0x00020000);
    float sg[CPL];
    uint4 w[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;  // chunk c of 32 codes lies in group 32 c / group
        const uint32_t off = c < nch ? (uint32_t)(((32 * c) / group) * SB) : kOob;
        if constexpr (E4M3) sg[j] = e4m3_decode(__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0));
        else sg[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        typedef int v4i_d __attribute__((ext_vector_type(4)));
        const v4i_d t = __builtin_amdgcn_raw_buffer_load_b128(rb, c < nch ? (uint32_t)c * 16u : kOob, 0, 0);
        w[j] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
    }
    float smax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) smax = fmaxf(smax, sg[j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off, 64));
    const float srow = (smax * 7.0f) / 127.0f;
    if (lane == 0) row_scales[i] = srow;
    int8_t *dst = w8 + (int64_t)i * k;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if (c >= nch) continue;
        const uint4 tab = code_table(srow == 0.0f ? 0.0f : sg[j] / srow);
        const uint2 d0 = decode8_table(w[j].x, tab), d1 = decode8_table(w[j].y, tab);
        const uint2 d2 = decode8_table(w[j].z, tab), d3 = decode8_table(w[j].w, tab);
        *reinterpret_cast<uint4 *>(dst + c * 32) = make_uint4(d0.x, d0.y, d1.x, d1.y);
        *reinterpret_cast<uint4 *>(dst + c * 32 + 16) = make_uint4(d2.x, d2.y, d3.x, d3.y);
    }
}

template <int CPL>
void launch_decode_rows(const int8_t *w_packed, const void *group_scales, bool scale_e4m3, int64_t k, int group,
                        int64_t n0, int64_t nc, int8_t *w8, float *row_scales, hipStream_t stream) {
    const dim3 grid((unsigned)((nc + 3) / 4)), block(256);
    if (scale_e4m3)
        w4a8_decode_rows_kernel<CPL, true><<<grid, block, 0, stream>>>(w_packed, group_scales, (int)k, group, n0,
                                                                       (int)nc, w8, row_scales);
    else
        w4a8_decode_rows_kernel<CPL, false><<<grid, block, 0, stream>>>(w_packed, group_scales, (int)k, group, n0,
                                                                        (int)nc, w8, row_scales);
}

}  // namespace

hipError_t launch_w4a8_decode(const int8_t *w_packed, const void *group_scales, bool scale_e4m3, int64_t k, int group,
                              int64_t n0, int64_t nc, int8_t *w8, float *row_scales, hipStream_t stream,
                              const Codebook &cb) {
    if (!cb.on && group >= 32 && k % 128 == 0 && k <= 8192) {
        // the wavefront-per-row form (chunks of 32 codes in one group)
        switch ((k / 32 + 63) / 64) {
        case 1: launch_decode_rows<1>(w_packed, group_scales, scale_e4m3, k, group, n0, nc, w8, row_scales, stream); break;
        case 2: launch_decode_rows<2>(w_packed, group_scales, scale_e4m3, k, group, n0, nc, w8, row_scales, stream); break;
        case 3: launch_decode_rows<3>(w_packed, group_scales, scale_e4m3, k, group, n0, nc, w8, row_scales, stream); break;
        default: launch_decode_rows<4>(w_packed, group_scales, scale_e4m3, k, group, n0, nc, w8, row_scales, stream); break;
        }
        return hipGetLastError();
    }
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
// int32 partial sums through LDS. Codes are decoded through a per-lane table
// of the 16 int8 codes of one multiplier (groups of 64 and wider), or per code
// (narrower groups).
namespace ck4 {
namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));

// One k-step of one 16-row weight tile: the lane's 64 packed codes (8 words,
// element 2j in the low nibble of byte j of its span) decoded to int8 codes
// and multiplied against the FM activation fragments of the step's four
// slices. gv holds the lane's group scales of the step (SG = 0: one per
// 16-code slice; SG = 8 / 4: one per word / half word), srow its row scale.
// Every path below forms the same fp32 values as the decode kernel.
template <int FM, int NGV, int SG, bool CB>
__device__ __forceinline__ void w4a8_tile_step(const uint32_t (&words)[8], const float (&gv)[NGV], float srow,
                                               bool one_group, const v4i_t (&xv)[FM][4], v4i_t (&acc)[FM],
                                               const Codebook &cb) {
    if constexpr (SG != 0) {
        // groups of 8 or 4: a multiplier per word or per half word
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint2 d[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int wi = 2 * h + e;
                const int ga = SG == 8 ? wi : 2 * wi, gb = SG == 8 ? wi : 2 * wi + 1;
                const float ma = srow == 0.0f ? 0.0f : gv[ga] / srow;
                const float mb = SG == 8 ? ma : (srow == 0.0f ? 0.0f : gv[gb] / srow);
                if constexpr (CB) {
                    const uint4 ta = code_table_cb(ma, cb);
                    d[e] = SG == 8 ? decode8_table(words[wi], ta) : decode8_table2(words[wi], ta, code_table_cb(mb, cb));
                } else {
                    d[e] = decode8_2(words[wi], ma, -8.0f * ma, mb, -8.0f * mb);
                }
            }
            const v4i_t w8 = v4i_t{(int)d[0].x, (int)d[0].y, (int)d[1].x, (int)d[1].y};
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[j][h], acc[j], 0, 0, 0);
        }
        return;
    } else {
        if (one_group) {
            // one multiplier for the lane's 64 codes: table decode
            const float mu = srow == 0.0f ? 0.0f : gv[0] / srow;
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
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[j][h], acc[j], 0, 0, 0);
            }
            return;
        }
        // groups of 16 and 32: a multiplier per 16 codes
        if constexpr (CB) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint4 tab = code_table_cb(srow == 0.0f ? 0.0f : gv[h] / srow, cb);
                const uint2 a = decode8_table(words[2 * h], tab);
                const uint2 b = decode8_table(words[2 * h + 1], tab);
                const v4i_t w8 = v4i_t{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[j][h], acc[j], 0, 0, 0);
            }
            return;
        } else {
            // per-code decode
            float mult[4], m8[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                mult[h] = srow == 0.0f ? 0.0f : gv[h] / srow;
                m8[h] = -8.0f * mult[h];
            }
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint2 a = decode8(words[2 * h], mult[h], m8[h]);
                const uint2 b = decode8(words[2 * h + 1], mult[h], m8[h]);
                const v4i_t w8 = v4i_t{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8, xv[j][h], acc[j], 0, 0, 0);
            }
        }
    }
}

// The dynamic LDS of w4a8_staged_kernel (its group-scale table).
extern __shared__ uint32_t w4a8_stab[];

// f(integral_constant<int, T>) for T = 0 .. sizeof...(T) - 1, unrolled.
template <typename F, int... T>
__device__ __forceinline__ void for_each_slot(F &&f, std::integer_sequence<int, T...>) {
    (f(std::integral_constant<int, T>{}), ...);
}

// Wait until at most C vector memory operations of this wavefront are outstanding.
template <int C>
__device__ __forceinline__ void vm_wait_le() {
    static_assert(C >= 0 && C <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((C & 15) | ((C >> 4) << 14) | 0x0f70);
}

// Operand layout: a k-step is 256 k. Lane l (row l & 15, part p = l >> 4)
// owns the 64 contiguous k [256 s + 64 p, 256 s + 64 p + 64) of its weight row
// and of its activation row; the MFMA of slice h (0..3) takes 16 of them,
// [.. + 16 h, .. + 16 h + 16), as its 16 bytes. Both operands use the same
// assignment, so each slice's 64 products are 64 distinct k and the four
// slices cover the step. A lane's 64 k lie in one weight group when the group
// is at least 64 wide, which makes the scale division once per step.
//
// Loading the operands straight into that layout puts four rows in each group
// of four lanes (the MFMA row order), which costs the address unit about four
// times a coalesced load. Instead each wavefront copies its k-steps global ->
// LDS with buffer_load ... lds into a ring of NSLOT slots, NSLOT - 1 steps
// ahead of the step it computes: the 16 FNW weight rows of a step (128 bytes
// each, 8 rows per instruction) and AR activation rows (256 bytes each, 4 rows
// per instruction; AR = 4 serves m <= 4, and fragment rows past AR read staged
// rows, which only reach outputs that are never stored). Each 16-byte chunk
// index is XORed with (row & 7), so the eight lanes of a fragment read that
// the LDS serves together hit distinct banks. Fragments are then read from
// LDS in the layout above. Group scales come straight from global memory, as
// raw bits issued with each step's copies. G64: groups of 64 and wider (one
// scale per lane and step).
template <int AR, int FNW, int KS, int NSLOT, bool E4M3, int SG, bool CB, bool G64>
__global__ __launch_bounds__(64 * KS) void w4a8_staged_kernel(const int8_t *__restrict__ X,
                                                            const float *__restrict__ sx,
                                                            const int8_t *__restrict__ W,
                                                            const void *__restrict__ gs, int M, int N, int K,
                                                            int group, uint16_t *__restrict__ Y, int64_t ldy,
                                                            Codebook cb, int tab) {
    constexpr int FM = (AR + 15) / 16;
    constexpr int NGV = SG == 0 ? 4 : 64 / SG;             // scales a tile step needs per lane
    constexpr int NS = SG != 0 ? NGV : (G64 ? 1 : 4);      // scale loads per tile and step
    constexpr int WB = 16 * FNW * 128;                     // weight bytes of a step
    constexpr int XB = AR * 256;                           // activation bytes of a step
    constexpr int SLOT = WB + XB;
    constexpr int W_INS = WB / 1024, X_INS = (XB + 1023) / 1024;
    // A step issues its group-scale loads, then its INS copies. Every
    // iteration issues exactly one step (past the wavefront's last step, a
    // copy out of the buffers' range: it moves no data), so when a step is
    // computed, the NSLOT - 1 steps after it have been issued. Memory
    // operations retire in order, so its copies have landed once at most
    // (NSLOT - 1) x INS operations are outstanding (counting only the copies
    // stays right however the compiler groups the scale loads; the counter
    // holds 63, and a smaller bound only waits longer).
    constexpr int INS = W_INS + X_INS;
    constexpr int VM_AHEAD = (NSLOT - 1) * INS < 63 ? (NSLOT - 1) * INS : 63;
    constexpr int RING = KS * NSLOT * SLOT;
    constexpr int RED = (KS - 1) * FNW * FM * 64 * 16;
    static_assert(AR == 4 || AR % 16 == 0, "activation rows");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[RING > RED ? RING : RED];
    // tab != 0: w4a8_stab holds the raw group-scale bits of the workgroup's
    // 16 FNW rows, [row][ng], then the per-wavefront row maxima, [KS][16 FNW]
    uint32_t *const stab = w4a8_stab;

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
    uint8_t *ring = lds + wave * NSLOT * SLOT;

    // copy lanes: weights 8 rows x 8 chunks, activations 4 rows x 16 chunks
    const int wrow = lane >> 3;
    const uint32_t w_off = (uint32_t)wrow * (uint32_t)wrow_bytes + (uint32_t)(((lane & 7) ^ (wrow & 7)) * 16);
    const int xrow = lane >> 4;

    int64_t gsr[FNW];  // index of the first group scale of this lane's weight rows
    float srow[FNW];   // row scales, set once the first copies are issued
#pragma unroll
    for (int i = 0; i < FNW; ++i) gsr[i] = (int64_t)min(n0 + i * 16 + frow, N - 1) * ng;

    // K in 128-k halves of a step: an odd count ends in a half step, whose
    // copy window is moved back by half a step (so it stays inside the rows)
    // and whose first-half lanes (parts 0 and 1) multiply zeros
    const int steps = (K / 128 + 1) >> 1;
    const bool half_tail = (K / 128) & 1;
    auto kfirst = [&](int s) __attribute__((always_inline)) {
        return s * 256 - (half_tail && s == steps - 1 ? 128 : 0);
    };
    const int per_wave = (steps + KS - 1) / KS;
    const int s_begin = wave * per_wave;
    const int nsteps = max(0, min(steps, s_begin + per_wave) - s_begin);

    v4i_t acc[FNW][FM];
#pragma unroll
    for (int i = 0; i < FNW; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i_t{0, 0, 0, 0};
    uint32_t gb[NSLOT][FNW][NS];  // raw group-scale bits, per slot

    auto load_bits = [&](int64_t idx) __attribute__((always_inline)) -> uint32_t {
        if constexpr (E4M3) return static_cast<const uint8_t *>(gs)[idx];
        else return static_cast<const uint32_t *>(gs)[idx];
    };
    // group scales of step s (of the kernel) and its copies into slot
    // `dst`; s past this wavefront's last step (`real` false): the scales of
    // the kernel's last step, and copies past the end of the buffers' range
    // (the buffer bounds check turns them into no-ops)
    auto issue = [&](int s, bool real, uint8_t *__restrict__ dst, uint32_t (&g)[FNW][NS])
                     __attribute__((always_inline)) {
        const int k0 = kfirst(real ? s : steps - 1);  // first k of the step's window
        const uint32_t oob = real ? 0u : 0x40000000u;  // > any buffer range here (at most 8 MB)
        const int kb = k0 + part * 64;                 // first k of this lane's span
        if (!tab) {
#pragma unroll
            for (int i = 0; i < FNW; ++i) {
                if constexpr (SG != 0) {
#pragma unroll
                    for (int c = 0; c < NS; ++c) g[i][c] = load_bits(gsr[i] + kb / SG + c);
                } else if constexpr (G64) {
                    g[i][0] = load_bits(gsr[i] + kb / group);
                } else {
#pragma unroll
                    for (int h = 0; h < 4; ++h) g[i][h] = load_bits(gsr[i] + (kb + 16 * h) / group);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < W_INS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void *)(dst + q * 1024), 16,
                                                     (uint32_t)(q * 8) * (uint32_t)wrow_bytes + w_off +
                                                         (uint32_t)(k0 / 2) + oob,
                                                     0, 0, 0);
#pragma unroll
        for (int q = 0; q < X_INS; ++q) {
            const int r = q * 4 + xrow;  // activation row of this lane's chunk
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void *)(dst + WB + q * 1024), 16,
                (uint32_t)r * (uint32_t)K + (uint32_t)(((lane & 15) ^ (r & 7)) * 16) + (uint32_t)k0 + oob, 0, 0,
                0);
        }
    };
    auto compute = [&](const uint8_t *__restrict__ cur, const uint32_t (&g)[FNW][NS], bool tail)
                       __attribute__((always_inline)) {
        v4i_t xv[FM][4];
        const bool dead = tail && part < 2;  // this lane's k were counted in the previous step
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int r = AR < 16 ? (frow & (AR - 1)) : j * 16 + frow;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                xv[j][h] = *reinterpret_cast<const v4i_t *>(cur + WB + r * 256 + (((4 * part + h) ^ (r & 7)) * 16));
                if (dead) xv[j][h] = v4i_t{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < FNW; ++i) {
            const int r = i * 16 + frow;
            const uint4 a = *reinterpret_cast<const uint4 *>(cur + r * 128 + (((2 * part) ^ (r & 7)) * 16));
            const uint4 b = *reinterpret_cast<const uint4 *>(cur + r * 128 + (((2 * part + 1) ^ (r & 7)) * 16));
            const uint32_t words[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            float gv[NGV];
#pragma unroll
            for (int c = 0; c < NGV; ++c) {
                const uint32_t bits = g[i][SG == 0 && G64 ? 0 : c];
                if constexpr (E4M3) gv[c] = e4m3_decode(bits);
                else gv[c] = __uint_as_float(bits);
            }
            w4a8_tile_step<FM, NGV, SG, CB>(words, gv, srow[i], one_group, xv, acc[i], cb);
        }
    };
    // step idx (0-based in this wave) computes from slot T; first step
    // idx + NSLOT - 1 goes into the slot step idx - 1 was read from (those
    // reads have completed: their results were used)
    auto body = [&](int idx, auto t_c) __attribute__((always_inline)) {
        constexpr int T = decltype(t_c)::value;
        constexpr int TN = (T + NSLOT - 1) % NSLOT;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        issue(s_begin + idx + NSLOT - 1, idx + NSLOT - 1 < nsteps, ring + TN * SLOT, gb[TN]);
        vm_wait_le<VM_AHEAD>();
        asm volatile("" ::: "memory");  // no LDS read moves above the wait
        if (tab) {
            // this step's group scales from the table, at the indices issue() loads them from
            const int kb = kfirst(s_begin + idx) + part * 64;
#pragma unroll
            for (int i = 0; i < FNW; ++i) {
                const int trow = (i * 16 + frow) * ng;
#pragma unroll
                for (int c = 0; c < NS; ++c) {
                    const int gi = SG != 0 ? kb / SG + c : G64 ? kb / group : (kb + 16 * c) / group;
                    gb[T][i][c] = w4a8_stab[trow + gi];
                }
            }
        }
        compute(ring + T * SLOT, gb[T], half_tail && s_begin + idx == steps - 1);
    };
    // Row scale of this lane's weight rows, (max group scale * cmax) / 127.
    // The first loads per row are issued before the first copies, and all of
    // them before any is used, so that they cost one memory latency that
    // overlaps the copies'. Table mode: the wavefronts split the groups (wave
    // w, part p: groups 4 w + p + 4 KS u), keep their raw bits in the table
    // for the steps, and meet in one barrier for the row maxima. Otherwise
    // each wavefront loads all of its rows' groups (part p: groups p + 4 u)
    // and the steps load their scales again.
    constexpr int RB = 16;
    const int g_first = tab ? wave * 4 + part : part;
    const int g_step = tab ? 4 * KS : 4;
    uint32_t rs[FNW][RB];
#pragma unroll
    for (int i = 0; i < FNW; ++i)
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const int g = g_first + g_step * u;
            rs[i][u] = g < ng ? load_bits(gsr[i] + g) : 0u;
        }
    // steps 0 .. NSLOT - 2 of this wave into slots 0 .. NSLOT - 2
    for_each_slot(
        [&](auto t_c) __attribute__((always_inline)) {
            constexpr int T = decltype(t_c)::value;
            if constexpr (T < NSLOT - 1) issue(s_begin + T, T < nsteps, ring + T * SLOT, gb[T]);
        },
        std::make_integer_sequence<int, NSLOT>{});
    auto scale_of = [](uint32_t bits) __attribute__((always_inline)) -> float {
        if constexpr (E4M3) return e4m3_decode(bits);
        else return __uint_as_float(bits);
    };
    if (tab) {
        float smax[FNW];
#pragma unroll
        for (int i = 0; i < FNW; ++i) {
            smax[i] = 0.0f;
            const int trow = (i * 16 + frow) * ng;
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                const int g = g_first + g_step * u;
                if (g < ng) {
                    stab[trow + g] = rs[i][u];
                    smax[i] = fmaxf(smax[i], scale_of(rs[i][u]));
                }
            }
            for (int g = g_first + g_step * RB; g < ng; g += g_step) {
                const uint32_t b = load_bits(gsr[i] + g);
                stab[trow + g] = b;
                smax[i] = fmaxf(smax[i], scale_of(b));
            }
        }
        const int rmax = 16 * FNW * ng;  // [KS][16 FNW] row maxima after the table (fp32 bits)
#pragma unroll
        for (int i = 0; i < FNW; ++i) {
            float m = fmaxf(smax[i], __shfl_xor(smax[i], 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (part == 0) stab[rmax + wave * 16 * FNW + i * 16 + frow] = __float_as_uint(m);
        }
        __syncthreads();  // the table and every wavefront's maxima are in LDS
#pragma unroll
        for (int i = 0; i < FNW; ++i) {
            float m = __uint_as_float(stab[rmax + i * 16 + frow]);
#pragma unroll
            for (int w = 1; w < KS; ++w) m = fmaxf(m, __uint_as_float(stab[rmax + w * 16 * FNW + i * 16 + frow]));
            srow[i] = (m * (CB ? cb.cmax : 7.0f)) / 127.0f;
        }
    } else {
        float rsf[FNW][RB];
#pragma unroll
        for (int i = 0; i < FNW; ++i)
#pragma unroll
            for (int u = 0; u < RB; ++u) rsf[i][u] = scale_of(rs[i][u]);
        float smax[FNW];
#pragma unroll
        for (int i = 0; i < FNW; ++i) {
            smax[i] = 0.0f;
#pragma unroll
            for (int u = 0; u < RB; ++u) smax[i] = fmaxf(smax[i], rsf[i][u]);
        }
        for (int g0 = part + 4 * RB; g0 < ng; g0 += 32) {
            float v[FNW][8];
#pragma unroll
            for (int i = 0; i < FNW; ++i)
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    v[i][u] = g0 + 4 * u < ng ? load_scale<E4M3>(gs, gsr[i] + g0 + 4 * u) : 0.0f;
#pragma unroll
            for (int i = 0; i < FNW; ++i)
#pragma unroll
                for (int u = 0; u < 8; ++u) smax[i] = fmaxf(smax[i], v[i][u]);
        }
#pragma unroll
        for (int i = 0; i < FNW; ++i) {
            float m = fmaxf(smax[i], __shfl_xor(smax[i], 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            srow[i] = (m * (CB ? cb.cmax : 7.0f)) / 127.0f;
        }
    }
    for (int idx = 0; idx < nsteps; idx += NSLOT)
        for_each_slot(
            [&](auto t_c) __attribute__((always_inline)) {
                if (idx + decltype(t_c)::value < nsteps) body(idx + decltype(t_c)::value, t_c);
            },
            std::make_integer_sequence<int, NSLOT>{});

    vm_wait_le<0>();  // the copies issued past the last step have retired, too
    v4i_t *red = reinterpret_cast<v4i_t *>(lds);  // [KS - 1][FNW][FM][64], over the copy slots
    if (KS > 1) {
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __syncthreads();  // every wavefront is done with its slots
        if (wave > 0) {
#pragma unroll
            for (int i = 0; i < FNW; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) red[(((wave - 1) * FNW + i) * FM + j) * 64 + lane] = acc[i][j];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll 1
        for (int w = 0; w < KS - 1; ++w)
#pragma unroll
            for (int i = 0; i < FNW; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] += red[((w * FNW + i) * FM + j) * 64 + lane];
    }

    // Epilogue (as the direct kernel): lane holds acc[i][j][r] = y[m][n],
    // m = 16j + (l & 15), n = n0 + 16i + 4(l >> 4) + r.
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

template <int AR, int FNW, int KS, int NSLOT, bool E4M3, int SG, bool CB>
hipError_t launch_staged_cfg(const int8_t *x, const float *sx, const int8_t *w, const void *gs, int64_t m, int64_t n,
                             int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream, const Codebook &cb) {
    const dim3 grid((unsigned)((n + 16 * FNW - 1) / (16 * FNW))), block(64 * KS);
    // The group-scale table (raw bits of the workgroup's rows, plus the
    // wavefronts' row maxima) when it is small and the LDS has room for it.
    constexpr int FM = (AR + 15) / 16;
    constexpr size_t SLOT = 16 * FNW * 128 + AR * 256;
    constexpr size_t RING = (size_t)KS * NSLOT * SLOT, RED = (size_t)(KS - 1) * FNW * FM * 64 * 16;
    constexpr size_t STATIC = RING > RED ? RING : RED;
    const size_t table = (size_t)16 * FNW * (size_t)(k / group) * 4;
    const size_t dyn = table + (size_t)KS * 16 * FNW * 4;
    // only where it keeps as many workgroups per CU as the ring alone allows
    constexpr size_t kLds = 160 * 1024;
    const int tab = table <= 16384 && kLds / (STATIC + dyn) == kLds / STATIC ? 1 : 0;
    if (SG == 0 && group >= 64)
        w4a8_staged_kernel<AR, FNW, KS, NSLOT, E4M3, SG, CB, true><<<grid, block, tab ? dyn : 0, stream>>>(
            x, sx, w, gs, (int)m, (int)n, (int)k, group, y, ldy, cb, tab);
    else
        w4a8_staged_kernel<AR, FNW, KS, NSLOT, E4M3, SG, CB, false><<<grid, block, tab ? dyn : 0, stream>>>(
            x, sx, w, gs, (int)m, (int)n, (int)k, group, y, ldy, cb, tab);
    return hipGetLastError();
}

#define CK4_STAGED(AR, FNW, KS, NSLOT) \
    launch_staged_cfg<AR, FNW, KS, NSLOT, E4M3, SG, CB>(x, sx, w, gs, m, n, k, group, y, ldy, stream, cb)

template <bool E4M3, int SG, bool CB>
hipError_t launch_staged(const int8_t *x, const float *sx, const int8_t *w, const void *gs, int64_t m, int64_t n,
                         int64_t k, int group, uint16_t *y, int64_t ldy, hipStream_t stream, const Codebook &cb) {
    // With 512 or more weight tiles of 16 rows the workgroups are numerous
    // enough to fill the CUs with two K splits each; with fewer, four at
    // m <= 16, two with one weight tile above (N = 12288 / 5120 at K = 3072 /
    // 5120, 32 weight copies: the measured best of the staged configurations
    // at every m; deeper rings than these lost, as did more K splits).
    const bool many = (n + 15) / 16 >= 512;
    if (m <= 4) return CK4_STAGED(4, 1, 4, 3);
    if (m <= 16) return many ? CK4_STAGED(16, 1, 2, 3) : CK4_STAGED(16, 1, 4, 3);
    if (m <= 32) return many ? CK4_STAGED(32, 2, 2, 3) : CK4_STAGED(32, 1, 2, 3);
    return many ? CK4_STAGED(64, 2, 2, 2) : CK4_STAGED(64, 1, 2, 2);
}
#undef CK4_STAGED

template <bool E4M3, bool CB>
hipError_t launch_fused_groups(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                               const void *group_scales, int64_t m, int64_t n, int64_t k, int group, uint16_t *y,
                               int64_t ldy, hipStream_t stream, const Codebook &cb) {
    if (group == 4)
        return launch_staged<E4M3, 4, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy,
                                                   stream, cb);
    if (group == 8)
        return launch_staged<E4M3, 8, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy,
                                                   stream, cb);
    return launch_staged<E4M3, 0, CB>(x_q8, x_scales, w_packed, group_scales, m, n, k, group, y, ldy, stream,
                                               cb);
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

// The decode buffer of ck4_linear_w4a8_grouped_noalloc: a file-scope device
// array, so that entry point allocates nothing. Each device that runs the
// library holds its own copy until the process ends. Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void *g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
}  // namespace

hipError_t noalloc_scratch(int dev, void **ptr) {
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev]() {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    *ptr = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

}  // namespace ck4
