// W4A4 GEMM + epilogue for m <= 2 activation rows, as a matrix-vector
// product with coalesced weight loads, for gfx950.
//
// What it computes ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with
// fused CUDA kernels", Description: the s4 x s4 product with int32
// accumulation and the rank-one epilogue):
//   acc[m, n] = sum_k qx[m, k] qw[n, k]   (exact, int32)
//   y[m, n]   = bf16(((float)acc * sx[m]) * sw[n] (+ bias[n]))
// the same expression, in the same fp32 steps, as the GEMM kernels, so the
// outputs are bitwise theirs.
//
// With one or two activation rows the matrix cores have almost nothing to
// do; what costs is streaming the weight. The MFMA operand layout puts a
// different weight row in every lane of a group of four, which costs the
// address unit four times a coalesced load. Here consecutive lanes read
// consecutive 16-byte chunks of the same weight row (gemv_core.h): all loads
// of a wavefront's G rows are issued before the first is used, and the
// activation chunks with the same k stay in registers for every row. From
// three rows on, the K-split MFMA kernel, whose time hardly depends on m up
// to 16 rows, is the faster one (N = 12288, K = 3072, m = 4: 6.7 against
// 8.3 us), so this kernel takes m <= 2 only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv.h"
#include "gemv_core.h"

namespace ck4 {
namespace {

// MG activation rows held (m <= MG), NW wavefronts of G weight rows each,
// CPL chunks of 16 bytes per lane and row (row bytes <= 1024 CPL). The
// activation rows are read from memory once per workgroup into LDS (every
// wavefront needs all of them); the weight loads are issued right after
// them, so the wait for the activation leaves them in flight.
template <int NW, int MG, int G, int CPL>
__global__ __launch_bounds__(64 * NW) void gemv_w4a4_kernel(const int8_t *__restrict__ A,
                                                           const int8_t *__restrict__ B,
                                                           const float *__restrict__ sa,
                                                           const float *__restrict__ sb,
                                                           const float *__restrict__ bias, int M, int N, int K,
                                                           uint16_t *__restrict__ Y, int64_t ldy) {
    constexpr int T = 64 * NW;
    constexpr int XPT = (MG * 64 * CPL + T - 1) / T;  // activation chunks per thread
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // M x K/2
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row_bytes = K / 2;
    const int nch = row_bytes / 16;
    // a wavefront past N still takes part in the activation copy and its barrier
    const int n0 = (blockIdx.x * NW + wave) * G;
    const int rows = max(0, min(G, N - n0));

    const __amdgpu_buffer_rsrc_t ra = gemv_rows_rsrc(A, 0, M, row_bytes);
    v4i xt[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * T;  // chunk c of the M x nch activation chunks
        xt[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, c < M * nch ? (uint32_t)c * 16u : kGemvOob, 0, 0);
    }
    v4i w[G][CPL];
    gemv_load_rows<G, CPL>(gemv_rows_rsrc(B, n0, rows, row_bytes), lane, nch, rows, row_bytes, w);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int c = tid + i * T;
        if (c < M * nch) *reinterpret_cast<v4i *>(xs + c * 16) = xt[i];
    }
    __syncthreads();
    v4i x[MG][CPL];
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            x[m][j] = m < M && c < nch ? *reinterpret_cast<const v4i *>(xs + m * row_bytes + c * 16)
                                       : v4i{0, 0, 0, 0};
        }

    int acc[G][MG];
    gemv_accumulate<G, MG, CPL>(w, x, acc);
    float sx[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) sx[m] = m < M ? sa[m] : 0.0f;
    gemv_store<G, MG>(acc, lane, M, n0, rows, sx, sb, bias, Y, ldy);
}

template <int NW, int MG, int G, int CPL>
hipError_t launch_cfg(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                      int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy, hipStream_t stream) {
    const dim3 grid((unsigned)((n + G * NW - 1) / (G * NW))), block(64 * NW);
    const size_t lds = (size_t)m * (size_t)(k / 2);
    gemv_w4a4_kernel<NW, MG, G, CPL><<<grid, block, lds, stream>>>(a, b, sa, sb, bias, (int)m, (int)n, (int)k, y, ldy);
    return hipGetLastError();
}

template <int NW, int MG, int G>
hipError_t launch_g(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                    int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy, hipStream_t stream) {
    switch ((k / 32 + 63) / 64) {  // 16-byte chunks of a row per lane
    case 1: return launch_cfg<NW, MG, G, 1>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    case 2: return launch_cfg<NW, MG, G, 2>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    case 3: return launch_cfg<NW, MG, G, 3>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    case 4: return launch_cfg<NW, MG, G, 4>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    default: return launch_cfg<NW, MG, G, 8>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    }
}

// Weight rows per wavefront, from a sweep of 1, 2 and 4 rows and 4, 8 and 16
// wavefronts per workgroup over N = 4096-16384 and K = 1024-8192 (32 weight
// copies in turn): four wavefronts, of two rows where N > 8192, else one.
template <int MG>
hipError_t launch_mg(const int8_t *a, const int8_t *b, const float *sa, const float *sb, const float *bias,
                     int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy, hipStream_t stream) {
    if (n > 8192) return launch_g<kGemvWaves, MG, 2>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
    return launch_g<kGemvWaves, MG, 1>(a, b, sa, sb, bias, m, n, k, y, ldy, stream);
}

}  // namespace

bool gemv_w4a4_fits(int64_t m, int64_t k) { return m >= 1 && m <= 2 && k >= 256 && k % 128 == 0 && k <= 16384; }

hipError_t launch_gemv_w4a4(const int8_t *x_q, const float *x_scales, const int8_t *w_packed, const float *w_scales,
                            const float *bias, int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy,
                            hipStream_t stream) {
    if (m <= 1) return launch_mg<1>(x_q, w_packed, x_scales, w_scales, bias, m, n, k, y, ldy, stream);
    return launch_mg<2>(x_q, w_packed, x_scales, w_scales, bias, m, n, k, y, ldy, stream);
}

}  // namespace ck4
