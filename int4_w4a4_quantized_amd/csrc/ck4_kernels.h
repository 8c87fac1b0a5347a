// Internal launchers of the ck4 HIP kernels (gfx950). Not part of the C ABI:
// ck4_api.cpp validates arguments and then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck4 {

// A frozen 16-entry codebook of the grouped int4 weight, passed by value
// (it travels in the kernel arguments, so every wavefront reads it from
// scalar registers): code u stands for the value v[u] times the group scale.
// cmax = max |v[u]| > 0 takes the place of 7 in the scale formulas.
struct Codebook {
    float v[16] = {};
    float cmax = 0.0f;
    bool on = false;
};

// Options of the weight path (fp32 input) of launch_rotate_quant.
//   u, ldu      if u is not null: stochastic rounding with the draw
//               u[row * ldu + col] in [0, 1) for each element
//   scale_e4m3  grouped int4 only: group scales are stored as E4M3 bytes and
//               the codes use the decoded scale
//   cb          grouped int4 only: if cb.on, each code is the index of the
//               codebook entry nearest to r / s (ties to the lower index),
//               with s = absmax / cb.cmax
struct WeightOpts {
    const float *u = nullptr;
    int64_t ldu = 0;
    bool scale_e4m3 = false;
    Codebook cb = Codebook{};
};

// Rotation + quantisation of rows (one wavefront or one workgroup per row).
//   in_kind   0: bf16 input, 1: fp32 input
//   out_kind  0: packed int4 (+ scales), 1: int8 codes (+ scales), 2: fp32 rotation
//             (bf16 input only), 3: the rotation rounded to bf16, in MFMA fragment
//             order (rows a multiple of 16, k a multiple of 32; ldo unused), 4: int4
//             codes as FP6 E2M3 in the f8f6f4 MFMA operand image (group 0, k a
//             multiple of 128, rows padded to 16; ldo unused; see launch_gemm_fp6),
//             5: the same codes in the compact form of that image (see
//             launch_gemm_fp6, compact)
//   group     0: one scale per row; > 0: one scale per `group` elements (int4 only)
//   scales    fp32, or E4M3 bytes when wo.scale_e4m3
hipError_t launch_rotate_quant(const void *x, int in_kind, int64_t rows, int64_t k, int64_t ldx, int rot_block,
                               int out_kind, int group, void *out, int64_t ldo, float *scales, hipStream_t stream,
                               WeightOpts wo = WeightOpts{});

// MFMA fragment order of a bf16 matrix [rows, cols] (rows padded with whole
// 16-row blocks, cols a multiple of 32): 16-row x 32-column tiles of 512
// values, tile (r / 16, c / 32) at ((r / 16) * (cols / 32) + c / 32) * 512,
// element (i, c) of a tile at (16 ((c >> 2) & 3) + i) * 8 + 4 (c >> 4) + (c & 3).
//
// LoRA up-projection added in the bf16 epilogue of launch_gemm: t is the
// bf16 down-projected activation [m, rank], b the bf16 up-projection
// [n, rank], both in fragment order and 16-byte aligned; rank is a multiple
// of 32 (0 or t == nullptr: no LoRA term).
struct LoraUp {
    const uint16_t *t = nullptr;
    const uint16_t *b = nullptr;
    int rank = 0;
};

// Integer GEMM acc[m, n] = sum_k a[m, k] b[n, k] on int8 MFMA, with a rank-one
// bf16 epilogue (out_i32 == false) or an int32 store (out_i32 == true).
//   s4 true:  a, b packed int4 [rows, k/2]; false: int8 codes [rows, k].
//   lora      bf16 epilogue only: y += t b^T before the rounding
hipError_t launch_gemm(bool s4, const int8_t *a, const int8_t *b, const float *sa, const float *sb,
                       const float *bias, int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy,
                       hipStream_t stream, LoraUp lora = LoraUp{});

// The same GEMM and epilogue on FP6 operands: a and b hold the int4 codes as
// FP6 E2M3 values q / 8 in the f8f6f4 MFMA operand image (rotate_quant
// out_kind 4): rows padded to 16, k a multiple of 128, 16-row x 128-k blocks
// of 1536 bytes at ((r / 16) * (k / 128) + k / 128) * 1536, lane image
// 16 g + i (row i, k group g) of 24 bytes at 24 (16 g + i), code of k =
// 32 g + t at bits 6 t. Bit-identical to launch_gemm(s4 = true) on the same
// codes.
//
// compact: a and b hold the same images in the compact form (rotate_quant
// out_kind 5): 16-row x 128-k blocks of 1024 bytes at ((r / 16) * (k / 128) +
// k / 128) * 1024, lane image 16 g + i of 16 bytes at 16 (16 g + i), and in
// it the 96-bit FP6 image W of codes t = 0-15 (then of t = 16-31) as two
// dwords D0 = V0 | (V1 & 0x18618618), D1 = V2 | (V1 & 0x61861861), with
// V0, V1, V2 the dwords of W (the masks mark the zero exponent bits of V0
// and V2, where V1's data bits go).
hipError_t launch_gemm_fp6(const uint8_t *a, const uint8_t *b, const float *sa, const float *sb, const float *bias,
                           int64_t m, int64_t n, int64_t k, bool out_i32, void *y, int64_t ldy, hipStream_t stream,
                           LoraUp lora = LoraUp{}, bool compact = false);

// The output tile launch_gemm_fp6 uses for an m x n product (m, n in
// [1, 2^31)): true for 288 x 192 tiles (one workgroup per CU), false for
// 96 x 128 tiles of 4 waves (48 x 64 each, two workgroups per CU), whichever
// needs less time by the rounds of workgroups over the 256 CUs: on the part a
// round of large tiles takes about 16/9 the time of a round of small ones at
// the same K (30 against 17 us at K = 3072).
inline bool gemm_fp6_large_tile(int64_t m, int64_t n) {
    const int64_t big_rounds = (((m + 287) / 288) * ((n + 191) / 192) + 255) / 256;
    const int64_t small_rounds = (((m + 95) / 96) * ((n + 127) / 128) + 511) / 512;
    return 9 * small_rounds >= 16 * big_rounds;
}

// b (bf16 [n, rank], row stride ldb) to fragment order, zero rows padding n
// to a multiple of 16.
hipError_t launch_lora_pack(const uint16_t *b, int64_t n, int64_t rank, int64_t ldb, uint16_t *out,
                            hipStream_t stream);

// LoRA down-projection in the rotated basis: t[m, j] = bf16(alpha *
// sum_k bf16(rotate(x)[m, k]) a_rot[j, k]) with fp32 accumulation (the
// rotation too runs on the bf16 matrix cores, accumulating in fp32), x bf16
// [m, k] (row stride ldx), a_rot bf16 [rank, k] and t bf16 [m, rank] in
// fragment order (t: whole 16-row blocks).
// rank in {32, 64, 128, 256}; rot_block in {16, ..., 256}; k a multiple of
// max(128, rot_block).
hipError_t launch_lora_down(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, const uint16_t *a_rot,
                            int64_t rank, float alpha, uint16_t *t, hipStream_t stream);

// Grouped int4 -> int8 decode of weight rows [n0, n0 + nc). group_scales are
// fp32, or E4M3 bytes when scale_e4m3; group is a power of two >= 4; with
// cb.on the codes index the codebook instead of standing for q = -8..7.
hipError_t launch_w4a8_decode(const int8_t *w_packed, const void *group_scales, bool scale_e4m3, int64_t k, int group,
                              int64_t n0, int64_t nc, int8_t *w8, float *row_scales, hipStream_t stream,
                              const Codebook &cb = Codebook{});

// Fused grouped W4A8 linear for m <= 64 and k >= 256, k % 128 == 0 (decode in registers
// + int8 MFMA + epilogue), bit-identical to decode followed by the int8 GEMM.
hipError_t launch_w4a8_fused(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                             const void *group_scales, bool scale_e4m3, int64_t m, int64_t n, int64_t k, int group,
                             uint16_t *y, int64_t ldy, hipStream_t stream, const Codebook &cb = Codebook{});

// The fixed device buffer behind ck4_linear_w4a8_grouped_noalloc (a
// file-scope device array of kNoallocScratchBytes in w4a8_decode.hip): its
// device address on device `dev`, which must be the current device. The
// address is looked up once per device; the result (and error) is kept.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(int dev, void **ptr);

}  // namespace ck4
