// Grouped int4 -> int8 weight decode for gfx950.
//
// What it computes ("[PR #97] HIP port of #90: grouped W4A8 over the INT8
// GEMM", What this adds: int4 codes with per-group fp32 scales are decoded to
// int8 codes that the rowwise int8 GEMM consumes, one lane turning 8 packed
// bytes into 16 int8 with one 16-byte store; Chunk sizing: rows [n0, n0+nc)
// at a time). The int8 GEMM applies one scale per row in its epilogue, so the
// decode re-expresses the group scales against a row scale:
//   s_row = (max_g s[row, g] * 7) / 127
//   w8    = clamp(rint(q * (s[row, g] / s_row)), -127, 127)      (all fp32)
// An all-zero row (s_row == 0) decodes to zeros.
//
// One workgroup per output row: the row scale is a workgroup max-reduction
// over that row's group scales, then each lane decodes 16-element chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"

namespace ck4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int sext4(uint32_t nib) { return (int)(nib ^ 8u) - 8; }

__global__ __launch_bounds__(kThreads) void w4a8_decode_kernel(const int8_t *__restrict__ wp,
                                                               const float *__restrict__ gs, int k, int group,
                                                               int64_t n0, int8_t *__restrict__ w8,
                                                               float *__restrict__ row_scales) {
    __shared__ float red[kThreads / 64];
    const int i = blockIdx.x;
    const int64_t row = n0 + i;
    const int tid = threadIdx.x;
    const int ng = k / group;
    const float *sg = gs + row * ng;

    float smax = 0.0f;
    for (int g = tid; g < ng; g += kThreads) smax = fmaxf(smax, sg[g]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = smax;
    __syncthreads();
    smax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float srow = (smax * 7.0f) / 127.0f;
    if (tid == 0) row_scales[i] = srow;

    const int nchunks = k / 16;
    const int8_t *src = wp + row * (int64_t)(k / 2);
    int8_t *dst = w8 + (int64_t)i * k;
    for (int ch = tid; ch < nchunks; ch += kThreads) {
        const float mult = srow == 0.0f ? 0.0f : sg[(ch * 16) / group] / srow;
        const uint2 p = *reinterpret_cast<const uint2 *>(src + ch * 8);
        const uint32_t words[2] = {p.x, p.y};
        uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int q = sext4((words[e >> 3] >> (4 * (e & 7))) & 0xFu);
            float t = rintf((float)q * mult);
            t = fminf(fmaxf(t, -127.0f), 127.0f);
            out[e >> 2] |= ((uint32_t)(int)t & 0xFFu) << (8 * (e & 3));
        }
        *reinterpret_cast<uint4 *>(dst + ch * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    }
}

}  // namespace

hipError_t launch_w4a8_decode(const int8_t *w_packed, const float *group_scales, int64_t k, int group,
                              int64_t n0, int64_t nc, int8_t *w8, float *row_scales, hipStream_t stream) {
    w4a8_decode_kernel<<<dim3((unsigned)nc), dim3(kThreads), 0, stream>>>(w_packed, group_scales, (int)k, group,
                                                                          n0, w8, row_scales);
    return hipGetLastError();
}

}  // namespace ck4
