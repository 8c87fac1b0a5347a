/*
 * ck4 -- W4A4 ConvRot linear layer for AMD MI355X (gfx950), C ABI.
 *
 * The layer (comfy-kitchen "[PR #63] int4_tensorwise: W4A4 layout (+ConvRot)
 * with fused CUDA kernels", Description):
 *   1. rotate activations along K with a block Hadamard transform (ConvRot),
 *   2. quantise each activation row to symmetric int4 (scale = absmax / 7,
 *      codes in [-7, 7]) and pack two codes per byte, low nibble first,
 *   3. multiply against int4 weights rotated and quantised the same way with
 *      an s4 x s4 GEMM accumulating in int32 (|acc| <= 49 K),
 *   4. apply the per-row activation scale and per-row weight scale once, in a
 *      rank-one epilogue, and write bf16.
 * The grouped W4A8 variant ("[PR #97] HIP port of #90: grouped W4A8 over the
 * INT8 GEMM", What this adds / Chunk sizing) decodes int4 weights with
 * per-group scales into int8 codes with one scale per row, and runs the
 * rowwise int8 GEMM against int8 activations.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or retains them.
 *  - Matrices are row-major; ld* arguments are row strides in ELEMENTS of the
 *    pointed-to type (bytes for int8 containers).
 *  - bf16 tensors are passed as uint16_t bit patterns (IEEE bfloat16).
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it; none synchronises the host. Device faults surface
 *    at the caller's next synchronisation.
 *  - Errors are returned, never thrown: CK4_ERR_INVALID for a null pointer,
 *    a non-positive size, a row stride smaller than the row, or a pointer or
 *    stride that breaks the stated alignment; CK4_ERR_UNSUPPORTED for a shape
 *    or option outside what the kernels implement (listed per call);
 *    CK4_ERR_DEVICE when no gfx950 device is current or a launch fails.
 *    Nothing is launched when validation fails. ck4_last_error() returns a
 *    thread-local description of the last failure.
 *  - There is no fallback path: an unsupported call fails.
 *
 * Citation tags used below (web pages, by title and section):
 *  [PR #63]  comfy-kitchen "[PR #63] int4_tensorwise: W4A4 layout (+ConvRot)
 *            with fused CUDA kernels".
 *  [PR #97]  comfy-kitchen "[PR #97] HIP port of #90: grouped W4A8 over the
 *            INT8 GEMM".
 *  [FAST]    "ComfyUI-INT4-Fast" extension listing.
 *  [HIPT]    "Comfy-INT4-HIPtest" README.
 */
#ifndef CK4_H
#define CK4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CK4_OK = 0,
    CK4_ERR_INVALID = 1,
    CK4_ERR_UNSUPPORTED = 2,
    CK4_ERR_DEVICE = 3
} ck4_status;

/* Library version string, e.g. "ck4 0.1.0 gfx950". */
const char *ck4_version(void);
/* Static description of a status code. */
const char *ck4_status_string(ck4_status s);
/* Thread-local description of the most recent failure on this thread ("" if
 * none). The pointer stays valid until the next ck4 call on this thread. */
const char *ck4_last_error(void);

/*
 * Offline weight preparation ([PR #63] Description: quantize_int4_convrot_weight;
 * [PR #97] What this adds: int4 codes with per-group scales).
 *
 *   w        fp32 [n, ldw], the unrotated weight (out_features x in_features).
 *   rot_block  Hadamard block along K: a power of two in [16, 1024], k % rot_block == 0.
 *   group    0: one scale per output row (W4A4 layout), w_scales is fp32 [n].
 *            g > 0: one scale per contiguous group of g elements along K
 *            (grouped W4A8 layout), w_scales is fp32 [n, k/g]; g must be a
 *            power of two in [4, 1024] dividing k ([PR #97] Testing: group sizes
 *            4 to 64 are decoded bit-exactly).
 *   w_packed int8 [n, k/2] (row stride k/2): codes in [-7, 7], element 2j of a
 *            row in the low nibble of byte j, element 2j+1 in the high nibble.
 * Each row is rotated in fp32 (butterfly strides ascending, then one multiply
 * by fp32(1/sqrt(rot_block))), scaled by absmax/7 (fp32 divide) and rounded
 * half to even after an fp32 divide; an all-zero row or group has scale 0
 * and codes 0.
 * Alignment: w and ldw*4 bytes 16-byte aligned; w_packed 8-byte aligned.
 * Unsupported: k > 16384.
 */
ck4_status ck4_quantize_weight_convrot(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                       int group, int8_t *w_packed, float *w_scales, void *stream);

/*
 * ck4_quantize_weight_convrot with stochastic instead of nearest rounding, for
 * requantising a weight after a LoRA patch is baked into it ([HIPT] LoRA
 * modes: "Stochastic").
 *   u, ldu  fp32 [n, ldu]: one draw in [0, 1) per weight element, supplied
 *           by the caller (the library has no random number generator).
 *           Values outside [0, 1) are not checked; the formula below applies.
 * Each code is clamp(floor(RN(r / s) + u), -7, 7) in fp32, with r the rotated
 * weight and s its row (group = 0) or group scale, absmax / 7; an all-zero
 * row or group has scale 0 and codes 0. Other arguments, layouts and errors as
 * ck4_quantize_weight_convrot; u and ldu*4 bytes 16-byte aligned.
 */
ck4_status ck4_quantize_weight_convrot_sr(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                          int group, const float *u, int64_t ldu, int8_t *w_packed, float *w_scales,
                                          void *stream);

/*
 * Offline weight preparation for the rowwise int8 (W8A8) ConvRot linear, the
 * int8 layout that the int4 layout extends downward ([PR #63] Description;
 * [FAST] Features: int8 layers in mixed checkpoints).
 *   w        fp32 [n, ldw], the unrotated weight.
 *   w_q8     int8 [n, k] (row stride k), codes in [-127, 127].
 *   w_scales fp32 [n], absmax / 127 of each rotated row.
 * Same rotation and rounding as ck4_quantize_weight_convrot; an all-zero row
 * has scale 0 and codes 0. The result feeds ck4_linear_w8a8 together with
 * ck4_rotate_quantize_act(bits = 8).
 * Alignment: w and ldw*4 bytes 16-byte aligned; w_q8 16-byte aligned.
 * Unsupported: k > 16384.
 */
ck4_status ck4_quantize_weight_convrot_int8(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                            int8_t *w_q8, float *w_scales, void *stream);

/*
 * Dynamic activation rotation + quantisation, one fused pass per row
 * ([PR #63] Description: fused activation kernel, FHT rotation + rowwise int4
 * quantize + pack; [PR #97] What this adds: the int8 quantiser with
 * convrot=True for the W4A8 path).
 *
 *   x        bf16 [m, ldx].
 *   bits     4: x_q is packed int8 [m, k/2] (row stride k/2), codes in [-7, 7],
 *               low nibble first, scale = absmax / 7;
 *            8: x_q is int8 [m, k] (row stride k), codes in [-127, 127],
 *               scale = absmax / 127.
 *   x_scales fp32 [m], one per row over the whole K.
 * Same rotation and rounding as ck4_quantize_weight_convrot.
 * Alignment: x and ldx*2 bytes 16-byte aligned; x_q 8-byte (bits 4) or
 * 16-byte (bits 8) aligned. Unsupported: k > 16384.
 */
ck4_status ck4_rotate_quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                   int bits, int8_t *x_q, float *x_scales, void *stream);

/*
 * The fp32 rotation alone: r[m, k] = x * blockdiag(H, ..., H) * fp32(1/sqrt(rot_block)),
 * the first stage of ck4_rotate_quantize_act (same kernel, fp32 store).
 * Also the input basis of a rotated low-rank side path ([FAST] Features:
 * dynamic LoRA patching with a Hadamard-rotated down projection).
 * r is fp32 [m, k], row stride k, 16-byte aligned.
 */
ck4_status ck4_rotate_act_f32(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, float *r,
                              void *stream);

/*
 * W4A4 linear: y = bf16((sum_k qx[m,k] qw[n,k]) * x_scales[m] * w_scales[n] + bias[n])
 * ([PR #63] Description: s4.s4 GEMM with int32 accumulators, rank-one
 * epilogue; scales factor out of the K loop).
 *
 *   x_q, x_scales  from ck4_rotate_quantize_act(bits = 4); reusing them for
 *                  several weights is the caller's choice ([PR #63]: q/k/v
 *                  projections share one quantised activation).
 *   w_packed, w_scales  from ck4_quantize_weight_convrot(group = 0).
 *   bias     fp32 [n] or NULL.
 *   y        bf16 [m, ldy]; only columns [0, n) of each row are written.
 * The epilogue is fp32 ((acc * x_scale) * w_scale + bias) rounded once to
 * bf16, nearest even.
 * Alignment: x_q and w_packed 16-byte aligned; y 8-byte aligned and ldy a
 * multiple of 4. Unsupported: k % 128 != 0, k < 256, k > 131072 (the rows are
 * walked in 256-k steps; k = 128 (mod 256) ends in a half step).
 */
ck4_status ck4_linear_w4a4(const int8_t *x_q, const float *x_scales, const int8_t *w_packed,
                           const float *w_scales, const float *bias, int64_t m, int64_t n, int64_t k,
                           uint16_t *y, int64_t ldy, void *stream);

/*
 * The whole W4A4 layer from bf16 activations in one call: x rotated with
 * 128-element Hadamard blocks, quantised to packed int4 with one scale per
 * row, multiplied by the packed weight, epilogue as ck4_linear_w4a4
 * ([PR #63] Description: the activation kernel rotates, takes the row
 * scale, quantises and packs in one pass; the GEMM then applies the row and
 * column scales once). The same arguments as ck4_rotate_quantize_act(bits =
 * 4) followed by ck4_linear_w4a4, and the same results bit for bit: x_q
 * [m, k/2] and x_scales [m] are written too (the caller's buffers; reuse
 * them for other projections of the same activation), and y.
 *
 * For m <= 2 with rot_block 128 one kernel does it all: each workgroup
 * rotates and quantises the m rows into its own LDS while its weight loads
 * are in flight, which saves the quantiser's launch at decode sizes. Other
 * shapes run the quantiser, then the GEMM, on `stream`.
 *   x        bf16 [m, ldx], ldx a multiple of 8, 16-byte aligned.
 *   w_packed, w_scales, bias, y, ldy  as ck4_linear_w4a4.
 *   x_q      int8 [m, k/2], row stride k/2, 16-byte aligned (output).
 *   x_scales fp32 [m] (output).
 * Unsupported: k % 128 != 0, k < 256, k > 16384, rot_block not a power of
 * two in [16, 1024] or not dividing k.
 */
ck4_status ck4_linear_w4a4_bf16(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                const int8_t *w_packed, const float *w_scales, const float *bias, int64_t n,
                                int8_t *x_q, float *x_scales, uint16_t *y, int64_t ldy, void *stream);

/*
 * The integer part of ck4_linear_w4a4 alone: acc[m, n] (int32, row stride
 * ldacc) = sum_k qx[m,k] qw[n,k], exact. Same kernel as ck4_linear_w4a4 with
 * an int32 store in place of the epilogue. Same alignment and shape rules;
 * acc 16-byte aligned and ldacc a multiple of 4.
 */
ck4_status ck4_gemm_w4a4_acc_i32(const int8_t *x_q, const int8_t *w_packed, int64_t m, int64_t n, int64_t k,
                                 int32_t *acc, int64_t ldacc, void *stream);

/*
 * W4A4 on the FP6 matrix cores (the same layer, [PR #63] Description, at
 * twice the int8 matrix rate of gfx950, which has no int4 matrix
 * instruction). Every int4 code q in [-7, 7] is exactly the FP6 E2M3 value
 * q / 8 (a subnormal: sign bit 5, |q| in bits 0-2), products of two codes
 * are q_a q_b / 64, and the fp32 accumulator holds 64 x the integer sum
 * exactly for k <= 131072, so ck4_linear_w4a4_fp6 gives the same bits as
 * ck4_linear_w4a4 on the same codes and scales. The codes take 6 bits
 * instead of 4 (1.5x the bytes): this is the layout for compute-bound calls
 * (m of a few hundred and more); the int4 layout stays the one for
 * weight-streaming calls (small m, where the extra weight bytes cost more
 * than the doubled matrix rate saves, and m <= 64 has a kernel of its own).
 *
 * FP6 operand layout ("q6", ck4_fp6_bytes(rows, k) bytes, 16-byte aligned):
 * rows padded to a multiple of 16 (the padding rows are never written by the
 * quantisers and never reach an output), k a multiple of 128. The 16-row x
 * 128-k block (r / 16, k / 128) is 1536 bytes at ((r / 16) * (k / 128) +
 * k / 128) * 1536; in it, row i = r % 16 and k group g = (k % 128) / 32 own
 * the 24 bytes at 24 (16 g + i), holding the codes of k % 32 = t at bits
 * 6 t, least significant bit first (the MFMA operand register image).
 *
 * ck4_rotate_quantize_act_fp6, ck4_quantize_weight_convrot_fp6: the codes and
 *   scales of ck4_rotate_quantize_act(bits = 4) and
 *   ck4_quantize_weight_convrot(group = 0) (same rotation, scale and
 *   rounding), written as q6. x bf16 [m, ldx] / w fp32 [n, ldw], 16-byte
 *   aligned rows; scales fp32 [rows].
 * ck4_linear_w4a4_fp6: y as ck4_linear_w4a4, from q6 operands.
 * ck4_gemm_w4a4_fp6_acc_i32: its integer accumulators (int32, as
 *   ck4_gemm_w4a4_acc_i32).
 * Unsupported: k % 128 != 0; k > 16384 for the quantisers, k > 131072 for the
 * GEMM; other errors as the int4 calls. ck4_fp6_bytes returns 0 for k not a
 * multiple of 128.
 */
size_t ck4_fp6_bytes(int64_t rows, int64_t k);
ck4_status ck4_rotate_quantize_act_fp6(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                       uint8_t *x_q6, float *x_scales, void *stream);
ck4_status ck4_quantize_weight_convrot_fp6(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                           uint8_t *w_q6, float *w_scales, void *stream);
ck4_status ck4_linear_w4a4_fp6(const uint8_t *x_q6, const float *x_scales, const uint8_t *w_q6,
                               const float *w_scales, const float *bias, int64_t m, int64_t n, int64_t k,
                               uint16_t *y, int64_t ldy, void *stream);
ck4_status ck4_gemm_w4a4_fp6_acc_i32(const uint8_t *x_q6, const uint8_t *w_q6, int64_t m, int64_t n, int64_t k,
                                     int32_t *acc, int64_t ldacc, void *stream);
/*
 * Compact FP6 operand layout ("q6c", ck4_fp6c_bytes(rows, k) = rows16 * k / 2
 * bytes, 16-byte aligned): the q6 image with the two exponent bits of every
 * code, always zero for |q| <= 7, squeezed out, so the matrix cores are fed
 * from two thirds of the bytes. Blocks (r / 16, k / 128) of 1024 bytes at
 * ((r / 16) * (k / 128) + k / 128) * 1024; row i and k group g own the 16
 * bytes at 16 (16 g + i). Let W be the 96-bit q6 image of the codes of
 * t = 0-15 (then of t = 16-31) with dwords V0 = W[0:32), V1 = W[32:64),
 * V2 = W[64:96). Its two dwords (little-endian, bytes 0-7, then 8-15) are
 *   D0 = V0 | (V1 & 0x18618618),  D1 = V2 | (V1 & 0x61861861);
 * the masks are the zero exponent bits of V0 and of V2, and V1's data bits
 * sit exactly at their union, so V0 = D0 & ~0x18618618,
 * V2 = D1 & ~0x61861861, V1 = (D0 & 0x18618618) | (D1 & 0x61861861).
 *
 * ck4_rotate_quantize_act_fp6c, ck4_quantize_weight_convrot_fp6c,
 * ck4_linear_w4a4_fp6c, ck4_gemm_w4a4_fp6c_acc_i32: the four q6 calls above on
 * q6c operands, with the same arguments, bits, alignment and errors
 * ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with fused CUDA
 * kernels", Description: the same per-row quantisation and s4.s4 GEMM).
 * ck4_fp6c_bytes returns 0 for k not a multiple of 128.
 */
size_t ck4_fp6c_bytes(int64_t rows, int64_t k);
ck4_status ck4_rotate_quantize_act_fp6c(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                        uint8_t *x_q6c, float *x_scales, void *stream);
ck4_status ck4_quantize_weight_convrot_fp6c(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                            uint8_t *w_q6c, float *w_scales, void *stream);
ck4_status ck4_linear_w4a4_fp6c(const uint8_t *x_q6c, const float *x_scales, const uint8_t *w_q6c,
                                const float *w_scales, const float *bias, int64_t m, int64_t n, int64_t k,
                                uint16_t *y, int64_t ldy, void *stream);
ck4_status ck4_gemm_w4a4_fp6c_acc_i32(const uint8_t *x_q6c, const uint8_t *w_q6c, int64_t m, int64_t n, int64_t k,
                                      int32_t *acc, int64_t ldacc, void *stream);
/*
 * The output tile (tile_m x tile_n, host ints) that ck4_linear_w4a4_fp6 and
 * ck4_gemm_w4a4_fp6_acc_i32 (and their compact-operand forms, _fp6c) use for
 * an m x n x k product: 288 x 192 with
 * eight waves, or 96 x 128 with four, whichever takes fewer estimated rounds
 * of workgroups over the 256 compute units. Host-only (launches nothing,
 * needs no device); the same shape errors as ck4_gemm_w4a4_fp6_acc_i32.
 * For benchmarks and tests that must know which kernel a shape reaches.
 */
ck4_status ck4_gemm_fp6_tile(int64_t m, int64_t n, int64_t k, int *tile_m, int *tile_n);

/*
 * Grouped int4 -> int8 weight decode of rows [n0, n0 + nc) ([PR #97] What
 * this adds: grouped int4 -> int8 weight decode; Chunk sizing: one chunk of
 * output columns at a time).
 *
 *   w_packed      int8 [n, k/2] codes from ck4_quantize_weight_convrot(group = g).
 *   group_scales  fp32 [n, k/g].
 *   w8            int8 [nc, k] (row stride k), codes in [-127, 127].
 *   row_scales    fp32 [nc].
 * s_row = (max_j s[row, j] * 7) / 127, w8 = clamp(rint(q * (s[row, j] / s_row)), -127, 127),
 * all fp32; an all-zero row gives s_row = 0 and w8 = 0.
 * Alignment: w_packed and w8 16-byte aligned. Unsupported: g not a power of two in
 * [4, 1024].
 */
ck4_status ck4_dequant_w4a8_grouped(const int8_t *w_packed, const float *group_scales, int64_t n, int64_t k,
                                    int group, int64_t n0, int64_t nc, int8_t *w8, float *row_scales,
                                    void *stream);

/*
 * Rowwise int8 linear: y = bf16(sum_k qx[m,k] qw[n,k] * x_scales[m] * w_scales[n] + bias[n])
 * with int8 codes on both sides (the int8 GEMM that the grouped W4A8 path
 * feeds, [PR #97] What this adds). Same epilogue as ck4_linear_w4a4.
 * x_q8 int8 [m, k] from ck4_rotate_quantize_act(bits = 8); w8 int8 [n, k].
 * Alignment as ck4_linear_w4a4. Unsupported: k % 128 != 0, k > 131072.
 */
ck4_status ck4_linear_w8a8(const int8_t *x_q8, const float *x_scales, const int8_t *w8, const float *w_scales,
                           const float *bias, int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy,
                           void *stream);

/*
 * Grouped W4A8 linear ([PR #97] What this adds, Chunk sizing): y =
 * bf16(sum_k qx[m,k] w8[n,k] * x_scales[m] * s_row[n]), with w8 and s_row the
 * decode of ck4_dequant_w4a8_grouped. Three execution paths give bit-identical
 * results:
 *   chunk_cols > 0  the pages' chunked path: for each chunk of `chunk_cols`
 *                   output columns, decode that slice of the weight into the
 *                   workspace and run the int8 GEMM writing the chunk's
 *                   column slice of y through ldy (a multiple of 16);
 *   chunk_cols < 0  one decode pass over all n, then one int8 GEMM;
 *   chunk_cols == 0 the default policy: for m <= 64 (env
 *                   CK4_W4A8_CHUNK_MAX_ROWS) and k >= 256, one fused kernel
 *                   that decodes in registers (no workspace); otherwise chunks
 *                   of the device L2 size / k rounded down to 128, clamped to
 *                   [1024, 4096] (env CK4_W4A8_CHUNK_COLS overrides the width)
 *                   when m <= 64, or a single pass for larger m.
 *   x_q8, x_scales  from ck4_rotate_quantize_act(bits = 8).
 *   w_packed, group_scales  from ck4_quantize_weight_convrot(group = g).
 *   workspace       device memory of at least ck4_w4a8_workspace_bytes(...)
 *                   bytes (16-byte aligned; may be NULL when that is 0); its
 *                   contents are scratch.
 * Unsupported: k % 128 != 0, g not a power of two in [4, 1024].
 */
size_t ck4_w4a8_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t chunk_cols);
ck4_status ck4_linear_w4a8_grouped(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                   const float *group_scales, int64_t m, int64_t n, int64_t k, int group,
                                   uint16_t *y, int64_t ldy, int64_t chunk_cols, void *workspace,
                                   size_t ws_bytes, void *stream);


/*
 * The whole grouped W4A8 layer from bf16 activations in one call ([PR #97]
 * What this adds: int8 activations from the same rotation with an absmax/127
 * row scale, against the decoded int4 weight): the same arguments as
 * ck4_rotate_quantize_act(bits = 8) followed by ck4_linear_w4a8_grouped (or
 * its E4M3 form) with chunk_cols = 0, and the same results bit for bit:
 * x_q8 [m, k] and x_scales [m] are written too (the caller's buffers), and y.
 * For m = 1 with n <= 8192, rot_block 128, k <= 8192 and groups of 32 or
 * more codes one kernel does it all: each workgroup
 * rotates and quantises the row into its own LDS while its weight loads are
 * in flight, which saves the quantiser's launch at decode sizes. Other
 * shapes run the quantiser, then the W4A8 linear, on `stream`.
 *   x               bf16 [m, ldx], ldx a multiple of 8, 16-byte aligned.
 *   w_packed        int8 [n, k/2] from ck4_quantize_weight_convrot(group = g)
 *                   or its E4M3 form.
 *   group_scales    fp32 [n, k/g], or (scale_e4m3 != 0) E4M3 bytes [n, k/g].
 *   x_q8            int8 [m, k], row stride k, 16-byte aligned (output).
 *   x_scales        fp32 [m] (output).
 *   y, ldy          as ck4_linear_w4a8_grouped.
 *   workspace       as ck4_linear_w4a8_grouped with chunk_cols = 0: at least
 *                   ck4_w4a8_workspace_bytes(m, n, k, 0) bytes, NULL when
 *                   that is 0.
 * Unsupported: k % 128 != 0, k < 256, k > 16384, rot_block not a power of
 * two in [16, 1024] or not dividing k, g not a power of two in [4, 1024].
 */
ck4_status ck4_linear_w4a8_grouped_bf16(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                        const int8_t *w_packed, const void *group_scales, int scale_e4m3, int64_t n,
                                        int group, int8_t *x_q8, float *x_scales, uint16_t *y, int64_t ldy,
                                        void *workspace, size_t ws_bytes, void *stream);

/*
 * ck4_linear_w4a8_grouped for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same three paths
 * and the same results bit for bit. The decode buffer of the chunked and
 * single-pass paths is a fixed device array inside the library,
 * CK4_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it runs on, held until the
 * process ends; the call allocates nothing. CK4_ERR_UNSUPPORTED when
 * ck4_w4a8_workspace_bytes(m, n, k, chunk_cols) exceeds that size (choose a
 * chunk width that fits). Every call on a GPU shares that GPU's array and
 * leaves the last call's decoded weights in it (each call writes all of the
 * buffer it reads, so nothing has to start at zero): calls that overlap in time
 * on one GPU (several streams or host threads) race and must be serialised by
 * the caller.
 */
#define CK4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ck4_status ck4_linear_w4a8_grouped_noalloc(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                           const float *group_scales, int64_t m, int64_t n, int64_t k, int group,
                                           uint16_t *y, int64_t ldy, int64_t chunk_cols, void *stream);

/*
 * Grouped W4A8 with FP8 E4M3 group scales ([PR #97] What this adds: group
 * scales in fp32 or e4m3, one decode for both). E4M3 is the OCP format: sign,
 * 4 exponent bits (bias 7), 3 mantissa bits, largest 448, no infinities.
 *
 * ck4_quantize_weight_convrot_e4m3: as ck4_quantize_weight_convrot with
 *   group > 0, except that each group scale absmax / 7 is rounded to E4M3
 *   (nearest, ties to even, saturating at 448), stored as one byte in
 *   group_scales uint8 [n, k/group], and the group's codes are
 *   clamp(rint(r / s8), -7, 7) against the value s8 that byte decodes to
 *   (a byte that decodes to 0 gives codes 0).
 * ck4_dequant_w4a8_grouped_e4m3, ck4_linear_w4a8_grouped_e4m3: as the fp32
 *   versions; each scale byte decodes exactly to fp32 first, so the decode
 *   and the linear are those of the decoded fp32 scales, bit for bit.
 */
ck4_status ck4_quantize_weight_convrot_e4m3(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                            int group, int8_t *w_packed, uint8_t *group_scales, void *stream);
ck4_status ck4_dequant_w4a8_grouped_e4m3(const int8_t *w_packed, const uint8_t *group_scales, int64_t n, int64_t k,
                                         int group, int64_t n0, int64_t nc, int8_t *w8, float *row_scales,
                                         void *stream);
ck4_status ck4_linear_w4a8_grouped_e4m3(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                        const uint8_t *group_scales, int64_t m, int64_t n, int64_t k, int group,
                                        uint16_t *y, int64_t ldy, int64_t chunk_cols, void *workspace,
                                        size_t ws_bytes, void *stream);

/*
 * Grouped W4A8 with a frozen 16-entry codebook ([PR #97] What this adds: an
 * optional codebook staged for the decode; On #96: a frozen codebook lookup
 * table, and a decode that is bit exact with a pinned codebook). The pages
 * give neither the codebook's values nor how codes map through it; these
 * calls take the plain reading: the 4-bit code u (0..15, as stored, low
 * nibble first) stands for codebook[u] times the group scale.
 *
 *   codebook     HOST pointer to 16 fp32 entries, read during the call and
 *                copied into the kernel arguments; every entry finite and
 *                cmax = max |codebook[u]| in [2^-64, 2^64], else
 *                CK4_ERR_INVALID. The same 16 values must be passed to the
 *                decode and the linear as to the preparation.
 *   scale_e4m3   0: group_scales fp32 [n, k/g]; 1: E4M3 bytes [n, k/g] (as
 *                ck4_quantize_weight_convrot_e4m3).
 *
 * ck4_quantize_weight_convrot_codebook: rotation as ck4_quantize_weight_convrot;
 *   per group s = absmax / cmax (fp32 divide; with scale_e4m3 rounded to
 *   E4M3 and the decoded byte used), t = r / s (fp32 divide; t = 0 when
 *   s == 0), and u = the index minimising the fp32 value |t - codebook[u]|,
 *   the lowest such index on ties.
 * ck4_dequant_w4a8_codebook: s_row = (max_j s[row, j] * cmax) / 127,
 *   w8 = clamp(rint(codebook[u] * (s[row, j] / s_row)), -127, 127), all fp32;
 *   an all-zero row decodes to zeros. Rows, chunks and layouts as
 *   ck4_dequant_w4a8_grouped.
 * ck4_linear_w4a8_codebook: as ck4_linear_w4a8_grouped on that decode (same
 *   three execution paths, bit-identical).
 * Group g: a power of two in [4, 1024] dividing k. Other arguments, alignment
 * and errors as the fp32-scale calls.
 */
ck4_status ck4_quantize_weight_convrot_codebook(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                                int group, const float *codebook, int scale_e4m3, int8_t *w_packed,
                                                void *group_scales, void *stream);
ck4_status ck4_dequant_w4a8_codebook(const int8_t *w_packed, const void *group_scales, int scale_e4m3,
                                     const float *codebook, int64_t n, int64_t k, int group, int64_t n0, int64_t nc,
                                     int8_t *w8, float *row_scales, void *stream);
ck4_status ck4_linear_w4a8_codebook(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                    const void *group_scales, int scale_e4m3, const float *codebook, int64_t m,
                                    int64_t n, int64_t k, int group, uint16_t *y, int64_t ldy, int64_t chunk_cols,
                                    void *workspace, size_t ws_bytes, void *stream);

/*
 * Dynamic LoRA side path ([HIPT] LoRA modes: the Dynamic mode keeps the LoRA
 * matrices apart and adds their product at run time; [FAST] Features:
 * Dynamic LoRA patching rotates the LoRA down projection with the same
 * Hadamard blocks, so that it stays coherent with the rotated activation).
 * For a LoRA y += alpha * (x A^T) B^T with A fp32 [rank, k] (down) and
 * B bf16 [n, rank] (up), the orthonormal rotation R of the quantiser gives
 * x A^T = (x R)(A R)^T, so the down projection runs on the rotated
 * activation.
 *
 * Fragment order. The LoRA operands live in device memory in the register
 * order of the bf16 matrix instructions, so that every wavefront load is one
 * contiguous 1 KB: a bf16 matrix Z [rows, cols] (cols a multiple of 32, rows
 * rounded up to a multiple of 16) is stored as 16-row x 32-column tiles of
 * 512 values, tile (r / 16, c / 32) at element offset
 * ((r / 16) * (cols / 32) + c / 32) * 512, and element (i, c) of a tile at
 * (16 * ((c >> 2) & 3) + i) * 8 + 4 * (c >> 4) + (c & 3).
 *
 *   ck4_lora_prepare_down  a_pack = bf16(A R) in fragment order ([rank, k],
 *       rank * k values): each row of a (fp32, row stride lda) rotated with
 *       the weight path's fp32 butterflies and rounded to bf16 (nearest
 *       even). Once per LoRA, like the weight preparation.
 *   ck4_lora_prepare_up  b_pack = b in fragment order ([n, rank] padded to
 *       n16 = 16 * ceil(n / 16) rows with zeros: n16 * rank values); b bf16
 *       [n, ldb] holds the up matrix, already scaled as the caller wants.
 *   ck4_lora_down  t_pack = t in fragment order ([m, rank] as 16 * ceil(m / 16)
 *       rows: rows >= m of the last block hold unspecified values), with
 *       t[m, j] = bf16(alpha * sum_k bf16((x R)[m, k]) (A R)[j, k]); x R is
 *       the product of x with the +-1 Hadamard blocks accumulated in fp32 and
 *       scaled by fp32(1 / sqrt(rot_block)) (the rotation of
 *       ck4_rotate_act_f32 up to fp32 rounding order); products and sums in
 *       fp32; x bf16 [m, ldx].
 *   ck4_linear_w4a4_lora  ck4_linear_w4a4 with the up projection fused into
 *       its epilogue: y = bf16(acc * x_scales[m] * w_scales[n] (+ bias[n])
 *       + sum_j t[m, j] b[n, j]); the fp32 value of the base layer and the
 *       LoRA sum are added in fp32 before the one bf16 rounding.
 * Several LoRAs active at once are one LoRA of their summed ranks: stack
 * their scaled down rows and up columns (zero rows and columns pad the stack
 * to a supported rank and add nothing).
 * rank: 32, 64, 128 or 256. Alignment: x, ldx*2, a_pack, b_pack, t_pack
 * 16 bytes; a and lda*4 16 bytes; b, ldb*2 8 bytes.
 * Unsupported: rot_block above 256; k not a multiple of max(128, rot_block)
 * for ck4_lora_down; otherwise as ck4_rotate_act_f32 and ck4_linear_w4a4.
 */
ck4_status ck4_lora_prepare_down(const float *a, int64_t rank, int64_t k, int64_t lda, int rot_block,
                                 uint16_t *a_pack, void *stream);
ck4_status ck4_lora_prepare_up(const uint16_t *b, int64_t n, int64_t rank, int64_t ldb, uint16_t *b_pack,
                               void *stream);
ck4_status ck4_lora_down(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, const uint16_t *a_pack,
                         int64_t rank, float alpha, uint16_t *t_pack, void *stream);
ck4_status ck4_linear_w4a4_lora(const int8_t *x_q, const float *x_scales, const int8_t *w_packed,
                                const float *w_scales, const float *bias, const uint16_t *t_pack,
                                const uint16_t *b_pack, int64_t rank, int64_t m, int64_t n, int64_t k, uint16_t *y,
                                int64_t ldy, void *stream);

/*
 * The same LoRA epilogue on the FP6 operand path (the FP6 block above):
 * ck4_linear_w4a4_lora from x_q6 and w_q6, bit for bit. Arguments, ranks,
 * alignment and errors as ck4_linear_w4a4_lora and ck4_linear_w4a4_fp6. For
 * the callers of the FP6 layout (compute-bound calls).
 */
ck4_status ck4_linear_w4a4_fp6_lora(const uint8_t *x_q6, const float *x_scales, const uint8_t *w_q6,
                                    const float *w_scales, const float *bias, const uint16_t *t_pack,
                                    const uint16_t *b_pack, int64_t rank, int64_t m, int64_t n, int64_t k,
                                    uint16_t *y, int64_t ldy, void *stream);
/*
 * The same LoRA epilogue on compact FP6 operands (the q6c layout above):
 * ck4_linear_w4a4_lora from x_q6c and w_q6c, bit for bit ([HIPT] LoRA modes:
 * Dynamic). Arguments, ranks, alignment and errors as ck4_linear_w4a4_fp6_lora.
 */
ck4_status ck4_linear_w4a4_fp6c_lora(const uint8_t *x_q6c, const float *x_scales, const uint8_t *w_q6c,
                                     const float *w_scales, const float *bias, const uint16_t *t_pack,
                                     const uint16_t *b_pack, int64_t rank, int64_t m, int64_t n, int64_t k,
                                     uint16_t *y, int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CK4_H */
