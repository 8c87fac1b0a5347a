// The matrix-vector W4A4 kernels for one or two activation rows: the GEMM
// (gemv_w4a4.hip) and the whole layer in one launch (skinny_layer.hip).
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

}  // namespace ck4
