// The matrix-vector kernels for a few activation rows: the W4A4 GEMM
// (gemv_w4a4.hip), the whole W4A4 layer in one launch (skinny_layer.hip) and
// the fused grouped W4A8 linear (w4a8_gemv.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck4 {

// Whether (m, k) takes the kernel: 1 <= m <= 2, 256 <= k <= 16384, k % 128 == 0.
bool gemv_w4a4_fits(int64_t m, int64_t k);

// y bf16 [m, ldy] = the W4A4 linear of packed int4 x_q [m, k/2] and
// w_packed [n, k/2] with row scales x_scales [m], w_scales [n] and an
// optional bias [n]; bitwise the result of launch_gemm on the same operands.
hipError_t launch_gemv_w4a4(const int8_t *x_q, const float *x_scales, const int8_t *w_packed, const float *w_scales,
                            const float *bias, int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy,
                            hipStream_t stream);

// The whole W4A4 layer from bf16 activations in one launch (rotate with
// 128-blocks, quantise to packed int4, GEMM + epilogue) for m <= 2 rows:
// skinny_layer_fits says whether a shape takes it (1 <= m <= 2, rot_block
// 128, 256 <= k <= 8192, k % 128 == 0). Writes x_q [m, k/2] and x_scales [m]
// as the quantiser does, and y, bitwise as the quantiser followed by
// launch_gemm.
bool skinny_layer_fits(int64_t m, int64_t n, int64_t k, int rot_block);
hipError_t launch_skinny_layer(const uint16_t *x, int64_t ldx, const int8_t *w_packed, const float *w_scales,
                               const float *bias, int64_t m, int64_t n, int64_t k, int8_t *x_q, float *x_scales,
                               uint16_t *y, int64_t ldy, hipStream_t stream);

// Fused grouped W4A8 linear (int4 codes with fp32 or E4M3 group scales,
// decoded in registers, int8 activations) for the shapes w4a8_gemv_fits
// takes (m <= 2, n <= 8192, 256 <= k <= 8192, k % 128 == 0, groups of 32 or
// more codes, no codebook): y bf16 [m, ldy], bitwise the decode kernel
// followed by the int8 GEMM.
bool w4a8_gemv_fits(int64_t m, int64_t n, int64_t k, int group, bool codebook);
hipError_t launch_w4a8_gemv(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                            const void *group_scales, bool scale_e4m3, int64_t m, int64_t n, int64_t k, int group,
                            uint16_t *y, int64_t ldy, hipStream_t stream);

// The whole grouped W4A8 layer from bf16 activations in one launch (rotate
// with 128-blocks, quantise to int8 with s = absmax / 127, then the
// matrix-vector W4A8 product) for the shapes w4a8_layer_fits takes (m = 1,
// n <= 8192, rot_block 128, 256 <= k <= 8192, k % 128 == 0, groups of 32 or
// more codes, no codebook). Writes x_q8 [m, k] and
// x_scales [m] as the quantiser does, and y, bitwise as the quantiser
// followed by the W4A8 linear.
bool w4a8_layer_fits(int64_t m, int64_t n, int64_t k, int rot_block, int group, bool codebook, bool scale_e4m3);
hipError_t launch_w4a8_layer(const uint16_t *x, int64_t ldx, const int8_t *w_packed, const void *group_scales,
                             bool scale_e4m3, int64_t m, int64_t n, int64_t k, int group, int8_t *x_q8,
                             float *x_scales, uint16_t *y, int64_t ldy, hipStream_t stream);

}  // namespace ck4
