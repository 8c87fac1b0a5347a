// W4A4 GEMM on the gfx950 FP6 matrix cores, with the rank-one epilogue.
//
// What it computes is the s4.s4 GEMM of "[PR #63] int4_tensorwise: W4A4
// layout (+ConvRot) with fused CUDA kernels" (Description: carried integer
// accumulators, |acc| <= 49 K, per-row and per-column scales applied once
// after the K loop):
//   acc[m, n] = sum_k qa[m, k] * qb[n, k]
//   y[m, n]   = bf16(((float)acc * sa[m]) * sb[n] (+ bias[n]))
// bit for bit as the int8-MFMA kernel computes it, at twice its matrix rate.
//
// Why it is exact. Every int4 code q in [-7, 7] is exactly the FP6 E2M3
// value q / 8: exponent field 0 (a subnormal), mantissa |q|, sign bit 5. The
// product of two codes is q_a q_b / 64, and each partial sum of
// v_mfma_scale_f32_16x16x128_f8f6f4 (block scales 2^0) is an integer multiple
// of 2^-6 of magnitude <= 49 K / 64, which fp32 holds exactly for K <=
// 131072 (49 * 131072 < 2^24); so the fp32 accumulator is acc / 64 exactly,
// whatever the order of the additions, and acc * 64 is the integer
// accumulator as a float, as the int8 kernel converts it.
//
// Operand layout (FP6 fragment order, written by the quantiser's FP6 output):
// rows padded to a multiple of 16, K a multiple of 128; the 16-row x 128-k
// block (r / 16, k / 128) is 1536 bytes at ((r / 16) * (K / 128) + k / 128) *
// 1536, holding the 64 lane images of the MFMA operand: lane l = 16 g + i
// (row i, k group g) has 24 bytes at 24 l with the 32 codes of k = 128 kb +
// 32 g + t at bits 6 t, least significant bit first. A block is therefore
// one contiguous copy, and a fragment read (lane l reads 24 bytes at 24 l)
// touches every LDS bank once per 16 lanes.
//
// Compact operands (C4). The two exponent bits of every code are zero, so
// a lane image can travel in 16 bytes instead of 24 (1024-byte blocks, lane
// l at 16 l) and be expanded in registers with 8 bitwise instructions after
// its 16-byte LDS read (expand_c4). The copies then move two thirds of the
// bytes: 189 MB instead of 283 MB from L2 per launch on the square layer.
//
// Tiling: 288 x 192 output tiles (one per CU on the 4608 x 3072 layer), 8
// waves of 144 x 48 (9 x 3 MFMA fragments; the first MFMA operand is the
// weight fragment, so each lane's 4 accumulators are 4 consecutive output
// columns of one row). Where it takes fewer rounds of workgroups, 96 x 128
// tiles of 4 waves (48 x 64, 3 x 4 fragments), two workgroups per CU. One k
// step is 128 k (on the large tile: 30 blocks, 45 KB, or 30 KB compact),
// copied global -> LDS with buffer_load ... lds into a ring of 3 stages (4
// for compact operands), NST - 1 steps ahead of the MFMAs. Rows past the padded operands read as zeros through the buffer
// descriptors' range check (the block offset is in the copy's vector offset).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ck4_kernels.h"
#include "lora_up.h"
#include "tile_map.h"

namespace ck4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// bytes of one 16-row x 128-k operand block: 1536 for the FP6 image, 1024
// for the compact form (C4)
template <bool C4>
constexpr int blk_bytes() { return C4 ? 1024 : 1536; }

// s_waitcnt immediates: vmcnt <= n and lgkmcnt == 0, or vmcnt <= n alone.
constexpr int vm_lgkm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

typedef int v6i __attribute__((ext_vector_type(6)));

// One lane's 24-byte operand image (8-byte aligned): six registers, the
// part of the MFMA's eight-register operand that FP6 reads.
__device__ __forceinline__ v6i load_frag(const uint8_t *p) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    const uint2 b = *reinterpret_cast<const uint2 *>(p + 8);
    const uint2 c = *reinterpret_cast<const uint2 *>(p + 16);
    return v6i{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y};
}

// The compact form of an FP6 operand image. Every code is a subnormal
// (exponent bits 3-4 of its 6-bit field are zero), so the 96-bit image W of
// 16 codes, split in dwords V0 = W[0:32), V1 = W[32:64), V2 = W[64:96), has
// its 32 zero bits at fixed places: V0's at kZ0 (bits 3-4 of the fields of
// codes 0-4), V2's at kZ2, and V1's 21 data bits exactly at kZ0 | kZ2. So
// D0 = V0 | (V1 & kZ0) and D1 = V2 | (V1 & kZ2) hold the 16 codes in 8 bytes,
// and V0 = D0 & ~kZ0, V2 = D1 & ~kZ2, V1 = (D0 & kZ0) | (D1 & kZ2): four
// bitwise instructions restore 12 bytes of MFMA operand.
constexpr uint32_t kZ0 = 0x18618618u;
constexpr uint32_t kZ2 = 0x61861861u;
typedef int v4i __attribute__((ext_vector_type(4)));

// One lane's 16-byte compact image (16-byte aligned).
__device__ __forceinline__ v4i load_frag_c4(const uint8_t *p) { return *reinterpret_cast<const v4i *>(p); }

__device__ __forceinline__ v6i expand_c4(v4i d) {
    const uint32_t d0 = (uint32_t)d[0], d1 = (uint32_t)d[1], d2 = (uint32_t)d[2], d3 = (uint32_t)d[3];
    return v6i{(int)(d0 & ~kZ0), (int)((d0 & kZ0) | (d1 & kZ2)), (int)(d1 & ~kZ2),
               (int)(d2 & ~kZ0), (int)((d2 & kZ0) | (d3 & kZ2)), (int)(d3 & ~kZ2)};
}

template <bool C4>
struct FragT;
template <>
struct FragT<false> {
    typedef v6i type;
    static __device__ __forceinline__ v6i load(const uint8_t *p) { return load_frag(p); }
    static __device__ __forceinline__ v6i op(v6i f) { return f; }
};
template <>
struct FragT<true> {
    typedef v4i type;
    static __device__ __forceinline__ v4i load(const uint8_t *p) { return load_frag_c4(p); }
    static __device__ __forceinline__ v6i op(v4i f) { return expand_c4(f); }
};

__device__ __forceinline__ v4f mfma_fp6(v6i w, v6i x, v4f acc) {
    // cbsz = blgp = 2: both operands FP6 E2M3; scale bytes 127 = 2^0; the two
    // operand registers past the sixth are not read
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_shufflevector(w, w, 0, 1, 2, 3, 4, 5, -1, -1),
                                                            __builtin_shufflevector(x, x, 0, 1, 2, 3, 4, 5, -1, -1),
                                                            acc, 2, 2, 0, 127, 0, 127);
}

template <int BM, int BN, int WGM, int WGN, int WPE, int NST, bool OUT_I32, bool LORA, bool C4>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WGM * WGN, 64 * WGM * WGN),
                          amdgpu_waves_per_eu(WPE, WPE))) void
gemm_fp6_kernel(const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const float *__restrict__ sa,
                const float *__restrict__ sb, const float *__restrict__ bias, int M, int N, int kb,
                void *__restrict__ Y, int64_t ldy, int tiles_n, int tiles_total, int xcd_m, LoraUp lora) {
    constexpr int kBlk = blk_bytes<C4>();
    constexpr int kBlkChunks = kBlk / 16;  // 16-byte copy chunks per block
    constexpr int kLaneBytes = kBlk / 64;  // one lane's operand image
    using Frag = FragT<C4>;
    using frag_t = typename Frag::type;
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM;
    constexpr int WTN = BN / WGN;
    constexpr int FM = WTM / 16;
    constexpr int FN = WTN / 16;
    constexpr int BLK_A = BM / 16;
    constexpr int BLK_B = BN / 16;
    constexpr int STAGE = (BLK_A + BLK_B) * kBlk;
    constexpr int NINS_A = BLK_A * kBlkChunks / 64;  // copy instructions (64 x 16 bytes) per step
    constexpr int NINS = (BLK_A + BLK_B) * kBlkChunks / 64;
    constexpr int PER_WAVE = (NINS + NW - 1) / NW;
    constexpr int LD = BN + 8;  // bf16 epilogue tile row pitch
    constexpr int LDS_BYTES = NST * STAGE > BM * LD * 2 ? NST * STAGE : BM * LD * 2;
    static_assert(BM % 16 == 0 && BN % 16 == 0 && WTM % 16 == 0 && WTN % 16 == 0, "bad tile");
    static_assert((BLK_A * kBlkChunks) % 64 == 0 && (BLK_B * kBlkChunks) % 64 == 0, "bad copy split");
    static_assert(NST >= 2, "need two stages");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_n, tiles_total, xcd_m, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN;
    const int wn = wave - wm * WGN;

    // the row blocks of this tile that exist in the (16-row padded) operands
    const int64_t rowblk = (int64_t)kb * kBlk;
    const int blk_a = min(BLK_A, (M + 15) / 16 - m0 / 16);
    const int blk_b = min(BLK_B, (N + 15) / 16 - n0 / 16);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(A) + (int64_t)(m0 / 16) * rowblk, (short)0, (int)(blk_a * rowblk), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(B) + (int64_t)(n0 / 16) * rowblk, (short)0, (int)(blk_b * rowblk), 0x00020000);

    // Copy plan of one step: 16-byte chunk c = 64 q + lane of the stage,
    // block c / 96 (A blocks first), byte 16 (c % 96) of it. Every wave issues
    // PER_WAVE instructions so that its vmcnt arithmetic is uniform; the
    // surplus slots repeat an instruction of another wave (same bytes to the
    // same place).
    uint32_t voff[PER_WAVE];
    int qi[PER_WAVE];
#pragma unroll
    for (int t = 0; t < PER_WAVE; ++t) {
        int q = t * NW + wave;
        if (q >= NINS) q -= NW;
        qi[t] = q;
        const bool is_a = q < NINS_A;
        const int c = (is_a ? q : q - NINS_A) * 64 + lane;
        voff[t] = (uint32_t)(c / kBlkChunks) * (uint32_t)rowblk + (uint32_t)((c % kBlkChunks) * 16);
    }
    auto issue_stage = [&](uint8_t *dst, int s) {
#pragma unroll
        for (int t = 0; t < PER_WAVE; ++t) {
            const bool is_a = qi[t] < NINS_A;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb,
                                                     (__attribute__((address_space(3))) void *)(dst + qi[t] * 1024),
                                                     16, (int)voff[t], s * kBlk, 0, 0);
        }
    };

    v4f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int frow = lane & 15;
    const int fgrp = lane >> 4;

    // LDS offsets of this lane's fragment images in a stage.
    const int a_off = wm * FM * kBlk + lane * kLaneBytes;
    const int b_off = (BLK_A + wn * FN) * kBlk + lane * kLaneBytes;
    auto stage_ptr = [&](int s) { return smem + (s % NST) * STAGE; };
    // Every wave issues the same number of copy instructions per step, and
    // the prologue always fills NST - 1 slots (past the last step it repeats
    // the last step into a slot no step reads), so "step s has landed" is one
    // constant vmcnt: the NST - 3 later steps issued after it may stay in
    // flight.
    static_assert(NST >= 3, "the pipeline keeps two steps ahead of the MFMAs");
    constexpr int kAheadWait = (NST - 3) * PER_WAVE;

    // Software pipeline over k steps. The FN weight fragments of a step are
    // held in registers; the FM activation fragments stream through a ring of
    // D + 1 registers, each read D fragments ahead of the MFMAs that use it,
    // and the stream runs on into the next step without a pause: D fragments
    // before the end of step s the wave waits for step s + 1's copy and meets
    // the others at the barrier (after which step s - 1's slot is free for
    // the copy of step s + NST - 1), reads step s + 1's weight fragments into
    // the other weight set and continues the activation stream with step
    // s + 1. The next weight set moves into place at the end of the step (18
    // register moves, or the expansion of the compact images, against 27
    // MFMAs). Slots go through __restrict__ parameters of an inlined
    // function, so the compiler knows the slot being copied into is neither
    // of the slots being read.
    constexpr int D = 2;
    static_assert(FM % (D + 1) == 0 && FM > D, "the ring must realign at step boundaries");
    // compact operands (C4) stay compact in the ring and the next weight set
    // and are expanded where they are used: 8 bitwise instructions per
    // 16-byte image, against 3 MFMAs per activation fragment
    frag_t ring[D + 1];
    auto step = [&](auto more_c, const uint8_t *__restrict__ cur, const uint8_t *__restrict__ nxt,
                    uint8_t *__restrict__ dst, int s, v6i(&wb)[FN], frag_t(&wn)[FN]) {
        constexpr bool more = decltype(more_c)::value;  // step s + 1 exists
#pragma unroll
        for (int j = 0; j < FM; ++j) {
            const int jn = j + D;
            if (jn < FM) {
                ring[jn % (D + 1)] = Frag::load(cur + a_off + jn * kBlk);
            } else if constexpr (more) {
                if (jn == FM) {
                    // this wave's copy of step s + 1 has landed; the ring's
                    // reads of step s may stay in flight across the barrier
                    __builtin_amdgcn_s_waitcnt(vm_wait(kAheadWait));
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    // past the last step the copy repeats the last step into
                    // the free slot (never read), which keeps the step
                    // branch-free
                    issue_stage(dst, min(s + NST - 1, kb - 1));
#pragma unroll
                    for (int i = 0; i < FN; ++i) wn[i] = Frag::load(nxt + b_off + i * kBlk);
                }
                ring[jn % (D + 1)] = Frag::load(nxt + a_off + (jn - FM) * kBlk);
            }
            const v6i x = Frag::op(ring[j % (D + 1)]);
#pragma unroll
            for (int i = 0; i < FN; ++i) acc[i][j] = mfma_fp6(wb[i], x, acc[i][j]);
            // keep the schedule as written: loads hoisted further would only
            // raise register pressure
            __builtin_amdgcn_sched_barrier(0);
        }
    };

#pragma unroll
    for (int p = 0; p < NST - 1; ++p) issue_stage(stage_ptr(p), min(p, kb - 1));
    // step 0 has landed in every wave's part (a bare s_barrier: __syncthreads
    // would also drain the later steps' copies; the empty asm keeps the LDS
    // reads below it)
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(kAheadWait + PER_WAVE));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    v6i w0[FN];
    frag_t w1[FN];
#pragma unroll
    for (int i = 0; i < FN; ++i) w0[i] = Frag::op(Frag::load(stage_ptr(0) + b_off + i * kBlk));
#pragma unroll
    for (int j = 0; j < D; ++j) ring[j] = Frag::load(stage_ptr(0) + a_off + j * kBlk);
    using more_t = std::integral_constant<bool, true>;
    using last_t = std::integral_constant<bool, false>;
    for (int s = 0; s + 1 < kb; ++s) {
        step(more_t{}, stage_ptr(s), stage_ptr(s + 1), stage_ptr(s + NST - 1), s, w0, w1);
#pragma unroll
        for (int i = 0; i < FN; ++i) w0[i] = Frag::op(w1[i]);
    }
    step(last_t{}, stage_ptr(kb - 1), stage_ptr(kb), stage_ptr(kb + NST - 2), kb - 1, w0, w1);
    // the repeat copies past the last step (into slots no one reads) must
    // land before the epilogue reuses the LDS for its tile
    __builtin_amdgcn_s_waitcnt(vm_wait(0));

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
                for (int r = 0; r < 4; ++r) a4[r] = (int)(acc[i][j][r] * 64.0f);
                int32_t *yr = reinterpret_cast<int32_t *>(Y) + (int64_t)m * ldy + nb;
                if (nb + 3 < N) {
                    *reinterpret_cast<int4 *>(yr) = make_int4(a4[0], a4[1], a4[2], a4[3]);
                } else {
                    for (int r = 0; r < 4 && nb + r < N; ++r) yr[r] = a4[r];
                }
            }
        }
    } else {
        // Rank-one epilogue through LDS, so the tile leaves as whole rows:
        // y = bf16((acc * sa[m]) * sb[n] (+ bias[n])) with acc = 64 x the fp32
        // accumulator (exact), into a [BM][BN + 8] bf16 tile, then 16-byte
        // row-contiguous stores. The factor 64 goes into the row scale:
        // f * (64 sa) and (64 f) * sa are the same rounding of 64 f sa, because
        // 64 sa is exact; a row scale whose 64-fold overflows is capped at the
        // largest float, so that 0 stays 0 and any nonzero product still
        // overflows as (64 f) * sa does.
        // the scales are read after the K loop, whose registers are all in use
        float sa_r[FM], sb_r[FN][4];
#pragma unroll
        for (int j = 0; j < FM; ++j)
            sa_r[j] = fminf(sa[min(m0 + wm * WTM + j * 16 + frow, M - 1)] * 64.0f, 3.40282347e38f);
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sb_r[i][r] = sb[min(n0 + wn * WTN + i * 16 + 4 * fgrp + r, N - 1)];
        uint16_t *tile_lds = reinterpret_cast<uint16_t *>(smem);
        if constexpr (LORA) {
            // the fp32 values of the wave tile first, in place, then the LoRA
            // up projection accumulates onto them on the bf16 matrix cores
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = (acc[i][j][r] * sa_r[j]) * sb_r[i][r];
                        if (bias) v = v + bias[min(n0 + wn * WTN + i * 16 + 4 * fgrp + r, N - 1)];
                        acc[i][j][r] = v;
                    }
            lora_up<FN, FM>(acc, lora, n0 + wn * WTN, m0 + wm * WTM, N, M, lane);
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
                        o[r] = f32_to_bf16(acc[i][j][r]);
                    } else {
                        float v = (acc[i][j][r] * sa_r[j]) * sb_r[i][r];
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

template <int BM, int BN, int WGM, int WGN, int WPE, int NST, bool C4>
hipError_t launch_fp6(const uint8_t *a, const uint8_t *b, const float *sa, const float *sb, const float *bias,
                      int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy, hipStream_t stream,
                      LoraUp lora) {
    const int kb = (int)(k / 128);
    const int tiles_m = (int)((m + BM - 1) / BM);
    const int tiles_n = (int)((n + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    const int xcd_m = pick_xcd_m(tiles_m, tiles_n, BM, BN);
    dim3 grid((unsigned)total), block(64 * WGM * WGN);
    if (out_i32)
        gemm_fp6_kernel<BM, BN, WGM, WGN, WPE, NST, true, false, C4><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, kb, y, ldy, tiles_n, total, xcd_m, lora);
    else if (lora.rank > 0)
        gemm_fp6_kernel<BM, BN, WGM, WGN, WPE, NST, false, true, C4><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, kb, y, ldy, tiles_n, total, xcd_m, lora);
    else
        gemm_fp6_kernel<BM, BN, WGM, WGN, WPE, NST, false, false, C4><<<grid, block, 0, stream>>>(
            a, b, sa, sb, bias, (int)m, (int)n, kb, y, ldy, tiles_n, total, xcd_m, lora);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp6(const uint8_t *a, const uint8_t *b, const float *sa, const float *sb, const float *bias,
                           int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy, hipStream_t stream,
                           LoraUp lora, bool compact) {
    if (out_i32 || lora.t == nullptr) lora.rank = 0;
    const bool large = gemm_fp6_large_tile(m, n);
    // stages: 3 x 45 KB of FP6 blocks on the large tile; the compact blocks
    // (30 KB a step there) leave room for a fourth (3, 4 and 5 stages of
    // them measured alike on the square layer: 29.5-29.9 us)
    if (compact) {
        if (large) return launch_fp6<288, 192, 2, 4, 2, 4, true>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
        return launch_fp6<96, 128, 2, 2, 2, 4, true>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    }
    if (large) return launch_fp6<288, 192, 2, 4, 2, 3, false>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
    return launch_fp6<96, 128, 2, 2, 2, 3, false>(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy, stream, lora);
}

}  // namespace ck4
