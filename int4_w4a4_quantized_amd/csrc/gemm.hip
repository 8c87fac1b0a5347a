// Integer GEMM on the gfx950 int8 matrix cores, with the rank-one epilogue.
//
// What it computes ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with
// fused CUDA kernels", Description: s4.s4 GEMM with carried int32
// accumulators, |acc| <= 49 K, and the per-row / per-column scales applied
// once after the K loop):
//   acc[m, n] = sum_k a[m, k] * b[n, k]                    (exact, int32)
//   y[m, n]   = bf16(((float)acc * sa[m]) * sb[n] (+ bias[n]))
// a = quantised activations, b = quantised weights, both K-major.
//
// gfx950 has no int4 matrix instruction (the assembler rejects every i4 MFMA
// mnemonic), so int4 operands are widened in registers and fed to
// v_mfma_i32_16x16x64_i8. The widening uses two facts:
//  * for a packed byte B (low nibble = code of element 2j, high = 2j+1),
//    B & 0xF0 read as int8 is exactly 16 * hi, and (B << 4) & 0xF0 is exactly
//    16 * lo, so a 32-bit word of 8 codes widens to two words of 4 int8 each
//    with one AND (high) and one shift + AND (low): the products carry a factor
//    256, removed by an exact arithmetic shift after the K loop
//    (|256 acc| <= 12544 K < 2^31 for K <= 131072);
//  * the low-nibble words hold the even k and the high-nibble words the odd
//    k; both operands are split the same way, and a permutation of k shared
//    by both operands leaves every dot product unchanged ([PR #63]: both
//    operands share the fragment k-permutation).
//
// Two kernels: a large-tile kernel that stages both operands in LDS (M > 64)
// and a skinny kernel that streams the weight straight into registers
// (M <= 64). In both, the MFMA's first operand is the weight fragment and its
// second the activation fragment, so each lane's 4 accumulators are 4
// consecutive output columns of one row.
//
// Optional LoRA up-projection (dynamic LoRA, "Comfy-INT4-HIPtest" README, LoRA
// modes): with t = the bf16 down-projected activation [M, R] and b = the bf16
// up-projection [N, R], both in MFMA fragment order, the epilogue adds
// sum_j t[m, j] b[n, j] to the fp32 value of y before the bf16 rounding, with
// v_mfma_f32_16x16x32_bf16 whose result layout matches the int8 one (first
// operand b rows, second t rows), so the sum accumulates straight onto the
// lane's 4 outputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"
#include "int4_widen.h"
#include "lora_up.h"
#include "tile_map.h"

namespace ck4 {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kRowBytes = 128;          // bytes of each row per K step


template <bool S4, int BM, int BN, int WGM, int WGN, int WPE, bool OUT_I32, bool LORA>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WGM * WGN, 64 * WGM * WGN),
                          amdgpu_waves_per_eu(WPE, WPE))) void
gemm_big_kernel(const int8_t *__restrict__ A, const int8_t *__restrict__ B, const float *__restrict__ sa,
                const float *__restrict__ sb, const float *__restrict__ bias, int M, int N, int row_bytes,
                int halves, void *__restrict__ Y, int64_t ldy, int tiles_n, int tiles_total, int xcd_m,
                LoraUp lora) {
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM;
    constexpr int WTN = BN / WGN;
    constexpr int FM = WTM / 16;
    constexpr int FN = WTN / 16;
    constexpr int STAGE = (BM + BN) * kRowBytes;
    constexpr int NINSTR = (BM + BN) / 8;  // one wave instruction fills 8 rows x 128 bytes
    constexpr int PER_WAVE = (NINSTR + NW - 1) / NW;
    static_assert(BM % 8 == 0 && BN % 8 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "bad tile");
    __shared__ __attribute__((aligned(1024))) uint4 smem[2 * STAGE / 16];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_n, tiles_total, xcd_m, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN;
    const int wn = wave - wm * WGN;

    // K in 64-byte halves of a 128-byte step; an odd count ends in a half
    // step, whose copy window is moved back by half a step (so it stays inside
    // the row) and of which only the second half is multiplied
    const int ksteps = (halves + 1) >> 1;
    const bool half_tail = halves & 1;
    auto kbyte = [&](int s) { return s * kRowBytes - (half_tail && s == ksteps - 1 ? kRowBytes / 2 : 0); };

    const int rows_a = min(BM, M - m0);
    const int rows_b = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(A) + (int64_t)m0 * row_bytes, (short)0, rows_a * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(B) + (int64_t)n0 * row_bytes, (short)0, rows_b * row_bytes, 0x00020000);

    // Lane l of a staging instruction fills LDS slot l of an 8-row group:
    // row 8q + (l >> 3), physical chunk l & 7, holding logical chunk
    // (l & 7) ^ (row & 7) of that row.
    const uint32_t lane_off =
        (uint32_t)(lane >> 3) * (uint32_t)row_bytes + (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
    auto issue_stage = [&](uint4 *dst, int s) {
        char *base = reinterpret_cast<char *>(dst);
#pragma unroll
        for (int t = 0; t < PER_WAVE; ++t) {
            const int q = t * NW + wave;
            if (q < NINSTR) {
                const bool is_a = q < BM / 8;
                const int qr = is_a ? q : q - BM / 8;
                // the row (lane and instruction parts) in the VGPR offset, which the
                // descriptor's range check covers, so rows past M or N read as zeros;
                // the k offset within the row in soffset
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    is_a ? ra : rb, (__attribute__((address_space(3))) void *)(base + q * 1024), 16,
                    lane_off + (uint32_t)(qr * 8) * (uint32_t)row_bytes, (uint32_t)kbyte(s), 0, 0);
            }
        }
    };

    v4i acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // LDS byte offsets of this lane's fragment rows (row & 7 == lane & 7).
    const int frow = lane & 15;
    const int fgrp = lane >> 4;
    const int a_row0 = (wm * WTM + frow) * kRowBytes;
    const int b_row0 = (BM + wn * WTN + frow) * kRowBytes;
    const int chunk_off0 = ((0 * 4 + fgrp) ^ (lane & 7)) * 16;
    const int chunk_off1 = ((1 * 4 + fgrp) ^ (lane & 7)) * 16;

    // The epilogue's scales, fetched before the K loop so their latency hides.
    float sa_r[FM], sb_r[FN][4];
    if constexpr (!OUT_I32) {
#pragma unroll
        for (int j = 0; j < FM; ++j) sa_r[j] = sa[min(m0 + wm * WTM + j * 16 + frow, M - 1)];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sb_r[i][r] = sb[min(n0 + wn * WTN + i * 16 + 4 * fgrp + r, N - 1)];
    }

    // One stage = two 64-byte halves. Per half: the FN weight fragments are
    // read and widened once. The activation fragments flow through a
    // three-deep pipeline: while the MFMAs of fragment j run, fragment j+1 is
    // widened and fragment j+2 is read from LDS. The scheduling groups put two
    // VALU instructions between consecutive MFMAs, so the widening of the next
    // fragment hides under the matrix-core time of the current one.
    auto compute_stage = [&](const uint4 *src, bool tail) {
        const char *base = reinterpret_cast<const char *>(src);
        auto xptr = [&](int j, int coff) {
            return reinterpret_cast<const uint4 *>(base + a_row0 + j * 16 * kRowBytes + coff);
        };
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h == 0 && tail) continue;  // a half step: its k are the window's second half
            __builtin_amdgcn_sched_barrier(0);
            const int coff = h ? chunk_off1 : chunk_off0;
            uint4 wb[FN];
#pragma unroll
            for (int i = 0; i < FN; ++i)
                wb[i] = *reinterpret_cast<const uint4 *>(base + b_row0 + i * 16 * kRowBytes + coff);
            if constexpr (S4) {
                uint4 xraw = *xptr(0, coff);
                uint4 xnext = FM > 1 ? *xptr(1, coff) : xraw;
                v4i wl[FN], wh[FN];
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    wl[i] = widen_lo(wb[i]);
                    wh[i] = widen_hi(wb[i]);
                }
                v4i xl = widen_lo(xraw);
                v4i xh = widen_hi(xraw);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    v4i nl = xl, nh = xh;
                    if (j + 1 < FM) {
                        const uint4 cur = xnext;
                        if (j + 2 < FM) xnext = *xptr(j + 2, coff);
                        nl = widen_lo(cur);
                        nh = widen_hi(cur);
                    }
#pragma unroll
                    for (int i = 0; i < FN; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl[i], xl, acc[i][j], 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < FN; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh[i], xh, acc[i][j], 0, 0, 0);
                    if (j + 1 < FM) {
                        // the LDS read first: it has the whole iteration to land
                        if (j + 2 < FM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                        for (int t = 0; t < 2 * FN; ++t) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    xl = nl;
                    xh = nh;
                }
            } else {
                uint4 xnext = *xptr(0, coff);
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const uint4 xcur = xnext;
                    if (j + 1 < FM) xnext = *xptr(j + 1, coff);
#pragma unroll
                    for (int i = 0; i < FN; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(wb[i]), as_v4i(xcur), acc[i][j],
                                                                          0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // The stage body issues the DMA for stage s+1 into one LDS half and reads
    // stage s from the other. Passing the two halves as __restrict__ pointers
    // of an inlined function tells the compiler they never alias, so it does
    // not make the fragment reads wait for the DMA.
    auto body = [&](uint4 *__restrict__ dst, const uint4 *__restrict__ src, int s) {
        if (s + 1 < ksteps) issue_stage(dst, s + 1);
        compute_stage(src, half_tail && s == ksteps - 1);
    };
    issue_stage(smem, 0);
    for (int s = 0; s < ksteps; ++s) {
        __builtin_amdgcn_s_waitcnt(0);  // this thread's stage-s loads have landed
        __syncthreads();                // ... and every thread's; stage s-1 is no longer read
        uint4 *cur = smem + (s & 1) * (STAGE / 16);
        uint4 *nxt = smem + ((s + 1) & 1) * (STAGE / 16);
        body(nxt, cur, s);
    }

    if constexpr (OUT_I32) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int m = m0 + wm * WTM + j * 16 + frow;
            if (m >= M) continue;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int nb = n0 + wn * WTN + i * 16 + 4 * fgrp;
                if (nb >= N) continue;
                int a4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) a4[r] = S4 ? (acc[i][j][r] >> 8) : acc[i][j][r];
                int32_t *yr = reinterpret_cast<int32_t *>(Y) + (int64_t)m * ldy + nb;
                if (nb + 3 < N) {
                    *reinterpret_cast<int4 *>(yr) = make_int4(a4[0], a4[1], a4[2], a4[3]);
                } else {
                    for (int r = 0; r < 4 && nb + r < N; ++r) yr[r] = a4[r];
                }
            }
        }
    } else {
        // Rank-one epilogue, staged through LDS so that the tile leaves as
        // whole rows: y = bf16((acc * sa[m]) * sb[n] (+ bias[n])) into a
        // [BM][BN + 8] bf16 tile, then 16-byte row-contiguous stores.
        // With LoRA, the fp32 values of the whole wave tile are formed first and
        // the up-projection accumulates onto them on the matrix cores.
        constexpr int LD = BN + 8;
        static_assert(BM * LD * 2 <= 2 * STAGE, "output tile does not fit in LDS");
        uint16_t *tile_lds = reinterpret_cast<uint16_t *>(smem);
        v4f yv[LORA ? FN : 1][LORA ? FM : 1];
        if constexpr (LORA) {
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int a = S4 ? (acc[i][j][r] >> 8) : acc[i][j][r];
                        float v = ((float)a * sa_r[j]) * sb_r[i][r];
                        if (bias) v = v + bias[min(n0 + wn * WTN + i * 16 + 4 * fgrp + r, N - 1)];
                        yv[i][j][r] = v;
                    }
            lora_up<FN, FM>(yv, lora, n0 + wn * WTN, m0 + wm * WTM, N, M, lane);
        }
        __syncthreads();  // every wave has finished reading the last stage
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int ml = wm * WTM + j * 16 + frow;
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int nl = wn * WTN + i * 16 + 4 * fgrp;
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (LORA) {
                        o[r] = f32_to_bf16(yv[i][j][r]);
                    } else {
                        const int a = S4 ? (acc[i][j][r] >> 8) : acc[i][j][r];
                        float v = ((float)a * sa_r[j]) * sb_r[i][r];
                        if (bias) v = v + bias[min(n0 + nl + r, N - 1)];
                        o[r] = f32_to_bf16(v);
                    }
                }
                *reinterpret_cast<uint2 *>(tile_lds + ml * LD + nl) =
                    make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
            }
        }
        __syncthreads();
        constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
        for (int c = threadIdx.x; c < BM * CPR; c += NW * 64) {
            const int r = c / CPR;
            const int cn = (c - r * CPR) * 8;
            const int m = m0 + r;
            const int n = n0 + cn;
            if (m >= M || n >= N) continue;
            const uint4 v = *reinterpret_cast<const uint4 *>(tile_lds + r * LD + cn);
            uint16_t *yr = reinterpret_cast<uint16_t *>(Y) + (int64_t)m * ldy + n;
            if (n + 7 < N && ((reinterpret_cast<uintptr_t>(yr) & 15) == 0)) {
                *reinterpret_cast<uint4 *>(yr) = v;
            } else if (n + 7 < N) {
                // rows of y are 8-byte aligned (ldy % 4 == 0), 16-byte only if ldy % 8 == 0
                reinterpret_cast<uint2 *>(yr)[0] = make_uint2(v.x, v.y);
                reinterpret_cast<uint2 *>(yr)[1] = make_uint2(v.z, v.w);
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    if (n + t < N) yr[t] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
            }
        }
    }
}

template <bool S4, int BM, int BN, int WGM, int WGN, int WPE>
hipError_t launch_big(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                      int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy, hipStream_t stream,
                      LoraUp lora) {
    const int64_t row_bytes = S4 ? k / 2 : k;
    const int halves = (int)(row_bytes / (kRowBytes / 2));
    const int tiles_m = (int)((m + BM - 1) / BM);
    const int tiles_n = (int)((n + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    const int xcd_m = pick_xcd_m(tiles_m, tiles_n, BM, BN);
    dim3 grid((unsigned)total), block(64 * WGM * WGN);
    if (out_i32)
        gemm_big_kernel<S4, BM, BN, WGM, WGN, WPE, true, false><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, (int)row_bytes, halves, y, ldy, tiles_n, total, xcd_m, lora);
    else if (lora.rank > 0)
        gemm_big_kernel<S4, BM, BN, WGM, WGN, WPE, false, true><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, (int)row_bytes, halves, y, ldy, tiles_n, total, xcd_m, lora);
    else
        gemm_big_kernel<S4, BM, BN, WGM, WGN, WPE, false, false><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, (int)row_bytes, halves, y, ldy, tiles_n, total, xcd_m, lora);
    return hipGetLastError();
}

// Skinny kernel (M <= 64): bound by streaming the weight from HBM. A
// workgroup owns 16*FNW weight rows; its KS wavefronts split K between them,
// up to MAXS k-steps (128 bytes of every row each) in flight per wavefront.
// Two ways to bring a step in:
//  * direct (LDS_STAGE false): every load of a chunk straight from global
//    memory into VGPRs in the MFMA operand layout (lane l: row l & 15, 16
//    bytes at 16 (l >> 4) of each 64-byte half), so compute starts as soon as
//    the first step lands and no LDS limits residency;
//  * staged (LDS_STAGE true, used when the activation has 64 rows and its
//    fragments are four of every five loads): the 16*FNW weight rows and
//    16*FM activation rows of each step are copied global -> LDS with
//    buffer_load ... lds into the wavefront's own slots, 8 rows x 128 bytes
//    per instruction, and the fragments are read from LDS. The copies are
//    coalesced (each group of four lanes reads one 64-byte segment), whereas
//    the direct loads put four rows in each group of four lanes, which costs
//    the address unit about four times the cycles per load. As in the large
//    kernel the 16-byte chunk index is XORed with (row & 7), so a fragment read
//    hits 16 distinct banks.
// Rows past M or N read as zeros (range-checked vector offsets). The KS
// partial accumulators are summed through LDS and one wavefront runs the
// epilogue.
template <bool S4, int FM, int FNW, int KS, int MAXS, bool LDS_STAGE, bool OUT_I32, bool LORA>
__global__ __launch_bounds__(64 * KS) void gemm_skinny_kernel(
    const int8_t *__restrict__ A, const int8_t *__restrict__ B, const float *__restrict__ sa,
    const float *__restrict__ sb, const float *__restrict__ bias, int M, int N, int row_bytes, int halves,
    void *__restrict__ Y, int64_t ldy, LoraUp lora) {
    constexpr int SLAB = 128;  // bytes of each row per k-step: 256 k for s4, 128 k for s8
    constexpr int ROWS = 16 * (FNW + FM);  // staged rows per step: weights, then activations
    constexpr int SLOT = ROWS * SLAB;
    constexpr int NINS = ROWS / 8;  // copy instructions per step, 8 rows x 128 bytes each
    constexpr int RING = LDS_STAGE ? KS * MAXS * SLOT : 0;
    constexpr int RED = (KS - 1) * FNW * FM * 64 * 16;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[RING > RED ? RING : RED];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16 * FNW;
    const int rows_b = min(16 * FNW, N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(A), (short)0, M * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(B) + (int64_t)n0 * row_bytes, (short)0, rows_b * row_bytes, 0x00020000);
    const int frow = lane & 15;
    const int fgrp = lane >> 4;
    // direct loads: lane l reads row l & 15, 16 bytes at 16 (l >> 4) of each 64-byte half
    const uint32_t lane_off = (uint32_t)frow * (uint32_t)row_bytes + (uint32_t)(fgrp * 16);
    // copy lane: row 8q + (l >> 3) of the step's rows, logical chunk (l & 7) ^ (row & 7)
    const int crow = lane >> 3;
    const uint32_t c_off = (uint32_t)(((lane & 7) ^ crow) * 16);
    uint8_t *ring = lds + wave * MAXS * SLOT;
    // K in 64-byte halves of a step (as the large kernel): a half last step
    // copies a window moved back by half a step and multiplies its second
    // half; the direct loads read its first half where it lies
    const int steps = (halves + 1) >> 1;
    const bool half_tail = halves & 1;

    const int per_wave = (steps + KS - 1) / KS;
    const int s_begin = wave * per_wave;
    const int s_end = min(steps, s_begin + per_wave);

    v4i acc[FNW][FM];
#pragma unroll
    for (int i = 0; i < FNW; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    if constexpr (LDS_STAGE) {
        for (int s0 = s_begin; s0 < s_end; s0 += MAXS) {
            // the previous chunk's fragment reads have completed before its slots are overwritten
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    #pragma unroll
            for (int t = 0; t < MAXS; ++t) {
                const int s = s0 + t;
                if (s < s_end) {
    #pragma unroll
                    for (int q = 0; q < NINS; ++q) {
                        const bool is_w = q < 2 * FNW;
                        const int r = (is_w ? q : q - 2 * FNW) * 8 + crow;  // row within weights / activations
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            is_w ? rb : ra, (__attribute__((address_space(3))) void *)(ring + t * SLOT + q * 1024), 16,
                            (uint32_t)r * (uint32_t)row_bytes +
                                (uint32_t)(s * SLAB - (half_tail && s == steps - 1 ? SLAB / 2 : 0)) + c_off,
                            0, 0, 0);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wavefront's copies have landed
            asm volatile("" ::: "memory");        // and no LDS read moves above that wait
    #pragma unroll
            for (int t = 0; t < MAXS; ++t) {
                if (s0 + t >= s_end) break;
                const uint8_t *slot = ring + t * SLOT;
                const bool tail = half_tail && s0 + t == steps - 1;
    #pragma unroll
                for (int h = 0; h < SLAB / 64; ++h) {
                    if (h == 0 && tail) continue;
                    const int coff = ((4 * h + fgrp) ^ (frow & 7)) * 16;
                    uint4 wv[FNW], xv[FM];
    #pragma unroll
                    for (int i = 0; i < FNW; ++i)
                        wv[i] = *reinterpret_cast<const uint4 *>(slot + (i * 16 + frow) * SLAB + coff);
    #pragma unroll
                    for (int j = 0; j < FM; ++j)
                        xv[j] = *reinterpret_cast<const uint4 *>(slot + (16 * FNW + j * 16 + frow) * SLAB + coff);
                    if constexpr (S4) {
    #pragma unroll
                        for (int i = 0; i < FNW; ++i) {
                            const v4i wl = widen_lo(wv[i]), wh = widen_hi(wv[i]);
    #pragma unroll
                            for (int j = 0; j < FM; ++j) {
                                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl, widen_lo(xv[j]), acc[i][j], 0, 0, 0);
                                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh, widen_hi(xv[j]), acc[i][j], 0, 0, 0);
                            }
                        }
                    } else {
    #pragma unroll
                        for (int i = 0; i < FNW; ++i)
    #pragma unroll
                            for (int j = 0; j < FM; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(wv[i]), as_v4i(xv[j]), acc[i][j],
                                                                                  0, 0, 0);
                    }
                }
            }
        }
    } else {
        for (int s0 = s_begin; s0 < s_end; s0 += MAXS) {
            v4i wv[MAXS][FNW][SLAB / 64], xv[MAXS][FM][SLAB / 64];
    #pragma unroll
            for (int t = 0; t < MAXS; ++t) {
                const int s = s0 + t;
                if (s < s_end) {
    #pragma unroll
                    for (int h = 0; h < SLAB / 64; ++h) {
                        if (h == 1 && half_tail && s == steps - 1) break;
    #pragma unroll
                        for (int i = 0; i < FNW; ++i)
                            wv[t][i][h] = __builtin_amdgcn_raw_buffer_load_b128(
                                rb, lane_off + (uint32_t)(i * 16) * (uint32_t)row_bytes, s * SLAB + h * 64, 0);
    #pragma unroll
                        for (int j = 0; j < FM; ++j)
                            xv[t][j][h] = __builtin_amdgcn_raw_buffer_load_b128(
                                ra, lane_off + (uint32_t)(j * 16) * (uint32_t)row_bytes, s * SLAB + h * 64, 0);
                    }
                }
            }
    #pragma unroll
            for (int t = 0; t < MAXS; ++t) {
                if (s0 + t >= s_end) break;
    #pragma unroll
                for (int h = 0; h < SLAB / 64; ++h) {
                    if (h == 1 && half_tail && s0 + t == steps - 1) break;
                    if constexpr (S4) {
    #pragma unroll
                        for (int i = 0; i < FNW; ++i) {
                            const uint4 wp = make_uint4(wv[t][i][h].x, wv[t][i][h].y, wv[t][i][h].z, wv[t][i][h].w);
                            const v4i wl = widen_lo(wp), wh = widen_hi(wp);
    #pragma unroll
                            for (int j = 0; j < FM; ++j) {
                                const uint4 xp =
                                    make_uint4(xv[t][j][h].x, xv[t][j][h].y, xv[t][j][h].z, xv[t][j][h].w);
                                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl, widen_lo(xp), acc[i][j], 0, 0, 0);
                                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh, widen_hi(xp), acc[i][j], 0, 0, 0);
                            }
                        }
                    } else {
    #pragma unroll
                        for (int i = 0; i < FNW; ++i)
    #pragma unroll
                            for (int j = 0; j < FM; ++j)
                                acc[i][j] =
                                    __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[t][i][h], xv[t][j][h], acc[i][j], 0, 0, 0);
                    }
                }
            }
        }
    }

    v4i *red = reinterpret_cast<v4i *>(lds);  // [KS - 1][FNW][FM][64], over the copy slots
    if (KS > 1) {
        __syncthreads();  // every wavefront is done with its copy slots
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

    // With LoRA, every fragment's fp32 values are formed first (clamped rows,
    // so the whole wavefront runs the up-projection MFMAs) and the stores below
    // round them.
    v4f yv[LORA ? FNW : 1][LORA ? FM : 1];
    if constexpr (LORA) {
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const float sam = sa[min(j * 16 + frow, M - 1)];
#pragma unroll
            for (int i = 0; i < FNW; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = min(n0 + i * 16 + 4 * fgrp + r, N - 1);
                    const int a = S4 ? (acc[i][j][r] >> 8) : acc[i][j][r];
                    float v = ((float)a * sam) * sb[n];
                    if (bias) v = v + bias[n];
                    yv[i][j][r] = v;
                }
        }
        lora_up<FNW, FM>(yv, lora, n0, 0, N, M, lane);
    }

#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m = j * 16 + frow;
        if (m >= M) continue;
        const float sam = OUT_I32 ? 0.0f : sa[m];
#pragma unroll
        for (int i = 0; i < FNW; ++i) {
            const int nb = n0 + i * 16 + 4 * fgrp;
            if (nb >= N) continue;
            int a4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a4[r] = S4 ? (acc[i][j][r] >> 8) : acc[i][j][r];
            if constexpr (OUT_I32) {
                int32_t *yr = reinterpret_cast<int32_t *>(Y) + (int64_t)m * ldy + nb;
                if (nb + 3 < N) {
                    *reinterpret_cast<int4 *>(yr) = make_int4(a4[0], a4[1], a4[2], a4[3]);
                } else {
                    for (int r = 0; r < 4 && nb + r < N; ++r) yr[r] = a4[r];
                }
            } else {
                uint16_t *yr = reinterpret_cast<uint16_t *>(Y) + (int64_t)m * ldy + nb;
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (LORA) {
                        o[r] = f32_to_bf16(yv[i][j][r]);
                    } else {
                        const int n = nb + r < N ? nb + r : N - 1;
                        float v = ((float)a4[r] * sam) * sb[n];
                        if (bias) v = v + bias[n];
                        o[r] = f32_to_bf16(v);
                    }
                }
                if (nb + 3 < N) {
                    *reinterpret_cast<uint2 *>(yr) =
                        make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
                } else {
                    for (int r = 0; r < 4 && nb + r < N; ++r) yr[r] = o[r];
                }
            }
        }
    }
}

// Skinny GEMM for 4 < M <= 64 (packed int4, bf16 epilogue) with the waves of
// a workgroup splitting N instead of K: wave w owns the 16 weight rows
// 16 (NW blockIdx + w) and all of K, and the workgroup's waves share one LDS
// copy of the activation, so each workgroup reads the activation once for
// 16 NW weight rows (the K-split kernel above reads it once per 16). Both
// operands move through a ring of three chunks of CS k-steps (two in flight
// while one is read), copied global -> LDS with buffer_load ... lds (8 rows
// x 128 bytes per instruction, 16-byte chunks XOR-swizzled by row as above),
// the copies of a chunk split over the waves. Memory operations retire in
// order, so waiting for all but the next chunks' copies leaves exactly the
// current chunk complete; every operand then comes from LDS. No partial sums
// are exchanged.
template <bool S4, int FM, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_shared_kernel(
    const int8_t *__restrict__ A, const int8_t *__restrict__ B, const float *__restrict__ sa,
    const float *__restrict__ sb, const float *__restrict__ bias, int M, int N, int row_bytes, int halves,
    uint16_t *__restrict__ Y, int64_t ldy) {
    constexpr int SLAB = 128;                 // bytes of a row per k-step
    constexpr int CS = 2;                     // k-steps per chunk
    constexpr int AROWS = 16 * FM;            // activation rows (padded)
    constexpr int ROWS = AROWS + 16 * NW;     // staged rows per k-step: activation, then weights
    constexpr int STEP_B = ROWS * SLAB;       // LDS bytes of one k-step
    constexpr int NINS = ROWS / 8 * CS;       // copy instructions per chunk
    constexpr int PER = (NINS + NW - 1) / NW; // per wave (surplus slots repeat another wave's)
    static_assert(NINS >= NW && 2 * PER <= 63, "copy plan");
    static_assert(S4, "packed int4 operands only (both are widened)");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * CS * STEP_B];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw0 = blockIdx.x * NW * 16;                 // the workgroup's first weight row
    const int rows_w = min(16 * NW, N - nw0);             // weight rows that exist
    const bool has_rows = 16 * wave < rows_w;             // this wave's rows exist
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(A), (short)0, M * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(B) + (int64_t)nw0 * row_bytes, (short)0, rows_w * row_bytes, 0x00020000);
    const int frow = lane & 15;
    const int fgrp = lane >> 4;
    const int crow = lane >> 3;
    const uint32_t c_off = (uint32_t)(((lane & 7) ^ crow) * 16);
    // K in 64-byte halves (as the large kernel): a half last step copies a
    // window moved back by half a step and multiplies its second half
    const int steps = (halves + 1) >> 1;
    const bool half_tail = halves & 1;
    const int nch = (steps + CS - 1) / CS;

    v4i acc[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[j] = v4i{0, 0, 0, 0};

    // this wave's share of chunk c's copies into `slot` (steps past the last
    // repeat the last step; they are never read)
    auto issue = [&](int c, uint8_t *slot) {
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            int q = t * NW + wave;
            if (q >= NINS) q -= NW;
            const int st = q / (ROWS / 8), rg = q % (ROWS / 8);
            const int s = min(c * CS + st, steps - 1);
            const bool is_a = 8 * rg < AROWS;
            const int r = (is_a ? 8 * rg : 8 * rg - AROWS) + crow;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                is_a ? ra : rb, (__attribute__((address_space(3))) void *)(slot + st * STEP_B + rg * 1024), 16,
                (uint32_t)r * (uint32_t)row_bytes +
                    (uint32_t)(s * SLAB - (half_tail && s == steps - 1 ? SLAB / 2 : 0)) + c_off,
                0, 0, 0);
        }
    };
    // wait for chunk c (`later` next chunks' copies may stay in flight), then
    // every wave's part of it has landed
    auto wait_chunk = [&](int later) {
        constexpr int P1 = PER, P2 = 2 * PER;
        if (later == 2) __builtin_amdgcn_s_waitcnt((P2 & 15) | ((P2 >> 4) << 14) | 0x0f70);
        else if (later == 1) __builtin_amdgcn_s_waitcnt((P1 & 15) | ((P1 >> 4) << 14) | 0x0f70);
        else __builtin_amdgcn_s_waitcnt(0x0f70);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto compute = [&](int c, const uint8_t *slot) {
#pragma unroll
        for (int st = 0; st < CS; ++st) {
            if (c * CS + st >= steps) break;
            const bool tail = half_tail && c * CS + st == steps - 1;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 0 && tail) continue;
                const int coff = ((4 * h + fgrp) ^ (frow & 7)) * 16;
                const uint8_t *sp = slot + st * STEP_B;
                const uint4 wp = *reinterpret_cast<const uint4 *>(sp + (AROWS + 16 * wave + frow) * SLAB + coff);
                const v4i wl = widen_lo(wp), wh = widen_hi(wp);
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const uint4 xp = *reinterpret_cast<const uint4 *>(sp + (j * 16 + frow) * SLAB + coff);
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl, widen_lo(xp), acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh, widen_hi(xp), acc[j], 0, 0, 0);
                }
            }
        }
        // every wave is done reading the slot before it is filled again
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // one chunk: copy chunk c + 2 into the slot chunk c - 1 used (every wave
    // has left it at the barrier ending chunk c - 1), wait for chunk c,
    // compute. The slots arrive as __restrict__ parameters of an inlined
    // function, so the compiler knows the copies in flight do not write the
    // slot being read and adds no wait of its own for them.
    auto body = [&](int c, const uint8_t *__restrict__ cur, uint8_t *__restrict__ nxt2) {
        if (c + 2 < nch) issue(c + 2, nxt2);
        wait_chunk(c + 2 < nch ? 2 : (c + 1 < nch ? 1 : 0));
        compute(c, cur);
    };
    uint8_t *slot0 = lds, *slot1 = lds + CS * STEP_B, *slot2 = lds + 2 * CS * STEP_B;
    issue(0, slot0);
    if (nch > 1) issue(1, slot1);
    for (int c = 0; c < nch; c += 3) {
        body(c, slot0, slot2);
        if (c + 1 >= nch) break;
        body(c + 1, slot1, slot0);
        if (c + 2 >= nch) break;
        body(c + 2, slot2, slot1);
    }

    if (!has_rows) return;
    const int n0 = nw0 + 16 * wave;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m = j * 16 + frow;
        if (m >= M) continue;
        const float sam = sa[m];
        const int nb = n0 + 4 * fgrp;
        if (nb >= N) continue;
        uint16_t o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = nb + r < N ? nb + r : N - 1;
            float v = ((float)(acc[j][r] >> 8) * sam) * sb[n];
            if (bias) v = v + bias[n];
            o[r] = f32_to_bf16(v);
        }
        uint16_t *yr = Y + (int64_t)m * ldy + nb;
        if (nb + 3 < N) {
            *reinterpret_cast<uint2 *>(yr) =
                make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        } else {
            for (int r = 0; r < 4 && nb + r < N; ++r) yr[r] = o[r];
        }
    }
}

template <int FM, int NW>
hipError_t launch_skinny_shared_nw(const int8_t *a, const int8_t *b, const float *sa, const float *sb,
                                   const float *bias, int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy,
                                   hipStream_t stream) {
    const int64_t tiles = (n + 15) / 16;
    const dim3 grid((unsigned)((tiles + NW - 1) / NW)), block(64 * NW);
    gemm_skinny_shared_kernel<true, FM, NW><<<grid, block, 0, stream>>>(a, b, sa, sb, bias, (int)m, (int)n,
                                                                         (int)(k / 2), (int)(k / 128), y, ldy);
    return hipGetLastError();
}

// waves per workgroup: about one workgroup per CU on the weight tiles
template <int FM>
hipError_t launch_skinny_shared(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                                int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy, hipStream_t stream) {
    const int64_t per_cu = ((n + 15) / 16) / 256;
    if (per_cu >= 4) return launch_skinny_shared_nw<FM, 4>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    if (per_cu == 3) return launch_skinny_shared_nw<FM, 3>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    return launch_skinny_shared_nw<FM, 2>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
}

// MAXS: k-steps in flight per wavefront. Direct loads: 4, or 2 with a 64-row
// activation (the VGPR budget of 2 waves per SIMD). Staged: 1 to 4, about
// 20 KB of copy slots per wavefront, so that a CU's 160 KB of LDS holds eight
// wavefronts, and at most 128 KB per workgroup.
template <int FM, int FNW, int KS, bool LDS_STAGE>
constexpr int skinny_maxs() {
    if constexpr (!LDS_STAGE) {
        return FM >= 4 ? 2 : 4;
    } else {
        constexpr int slot = 16 * (FNW + FM) * 128;
        constexpr int m1 = (20 * 1024) / slot;
        constexpr int m2 = (128 * 1024) / (KS * slot);
        constexpr int m = m1 < m2 ? m1 : m2;
        return m < 1 ? 1 : (m > 4 ? 4 : m);
    }
}

template <bool S4, int FM, int FNW, int KS>
hipError_t launch_skinny_cfg(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                             int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy,
                             hipStream_t stream, LoraUp lora) {
    constexpr bool STG = FM >= 4;
    constexpr int MAXS = skinny_maxs<FM, FNW, KS, STG>();
    const int64_t row_bytes = S4 ? k / 2 : k;
    const int halves = (int)(row_bytes / 64);
    dim3 grid((unsigned)((n + 16 * FNW - 1) / (16 * FNW))), block(64 * KS);
    if (out_i32)
        gemm_skinny_kernel<S4, FM, FNW, KS, MAXS, STG, true, false><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, (int)row_bytes, halves, y, ldy, lora);
    else if (lora.rank > 0)
        gemm_skinny_kernel<S4, FM, FNW, KS, MAXS, STG, false, true><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, (int)row_bytes, halves, y, ldy, lora);
    else
        gemm_skinny_kernel<S4, FM, FNW, KS, MAXS, STG, false, false><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, (int)row_bytes, halves, y, ldy, lora);
    return hipGetLastError();
}

// KS: enough wavefronts in flight to keep HBM busy (about 2K or more).
template <bool S4, int FM, int FNW>
hipError_t launch_skinny_ks(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                            int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy, hipStream_t stream,
                            LoraUp lora) {
    const int64_t groups = (n + 16 * FNW - 1) / (16 * FNW);
    if (groups >= 1024)
        return launch_skinny_cfg<S4, FM, FNW, 2>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    if (groups >= 512)
        return launch_skinny_cfg<S4, FM, FNW, 4>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    return launch_skinny_cfg<S4, FM, FNW, 8>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
}

template <bool S4>
hipError_t launch_skinny(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                         int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy, hipStream_t stream,
                         LoraUp lora) {
    if constexpr (S4) {
        // the shared-activation kernel needs two or more weight tiles per CU;
        // at M <= 4 the activation is too small for sharing it to pay
        if (m > 4 && m <= 16 && !out_i32 && lora.rank == 0 && (n + 15) / 16 >= 512)
            return launch_skinny_shared<1>(a, b, sa, sb, bias, m, n, k, static_cast<uint16_t *>(y), ldy, stream);
    }
    if (m <= 16) return launch_skinny_ks<S4, 1, 1>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    if constexpr (S4) {
        if (m > 32 && !out_i32 && lora.rank == 0 && (n + 15) / 16 >= 512)
            return launch_skinny_shared<4>(a, b, sa, sb, bias, m, n, k, static_cast<uint16_t *>(y), ldy, stream);
        if (m > 16 && !out_i32 && lora.rank == 0 && (n + 15) / 16 >= 512)
            return launch_skinny_shared<2>(a, b, sa, sb, bias, m, n, k, static_cast<uint16_t *>(y), ldy, stream);
    }
    if (m <= 32) return launch_skinny_ks<S4, 2, 1>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    return launch_skinny_ks<S4, 4, 1>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
}

template <bool S4>
hipError_t launch_s(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias, int64_t m,
                    int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy, hipStream_t stream,
                    LoraUp lora) {
    if (m <= 64) return launch_skinny<S4>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    // 288 x 192 tiles (one workgroup per CU) or 128 x 128 tiles (two per CU).
    // Packed int4: whichever needs less time by the rounds of workgroups over
    // the 256 CUs (on the part a round of large tiles takes about 8/5 the time
    // of a round of small ones at the same K: 40 against 25 us at K = 3072).
    // int8 operands: large tiles once there are 192 of them.
    const int64_t big_tiles = ((m + 287) / 288) * ((n + 191) / 192);
    const int64_t big_rounds = (big_tiles + 255) / 256;
    const int64_t small_rounds = (((m + 127) / 128) * ((n + 127) / 128) + 511) / 512;
    if (S4 ? 5 * small_rounds > 8 * big_rounds : big_tiles >= 192)
        return launch_big<S4, 288, 192, 2, 4, 2>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    return launch_big<S4, 128, 128, 2, 2, 2>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
}

}  // namespace

hipError_t launch_gemm(bool s4, const int8_t *a, const int8_t *b, const float *sa, const float *sb,
                       const float *bias, int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy,
                       hipStream_t stream, LoraUp lora) {
    if (out_i32 || lora.t == nullptr) lora.rank = 0;
    if (s4) return launch_s<true>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    return launch_s<false>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
}

}  // namespace ck4
