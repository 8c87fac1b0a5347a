// LoRA down-projection of the dynamic LoRA side path, in the rotated basis.
//
// What it computes ("Comfy-INT4-HIPtest" README, LoRA modes: "Dynamic"
// keeps the LoRA matrices apart and adds their product at run time;
// "ComfyUI-INT4-Fast", Features: the LoRA down projection is rotated with the
// same Hadamard transform as the weights so that it stays coherent with the
// rotated activation):
//   r      = x * blockdiag(H_b, ..., H_b) * fp32(1/sqrt(b))   (the fp32 rotation
//            of the quantiser, bit for bit)
//   t[m,j] = bf16(alpha * sum_k bf16(r[m,k]) * a_rot[j,k])    (fp32 accumulation)
// with a_rot = bf16(rotation of the unrotated down projection A). Because the
// rotation is orthonormal, r a_rot^T equals x A^T up to rounding.
//
// One workgroup owns a 16-row tile of x; its 8 wavefronts split K in chunks of
// whole Hadamard blocks. A wavefront rotates its rows' chunk in VGPRs with the
// quantiser's butterflies, stores the bf16 values in its own LDS region (16-byte
// units XOR-swizzled by row so that a fragment read touches distinct banks),
// and multiplies them against a_rot with v_mfma_f32_16x16x32_bf16. The 8
// partial sums are added in a fixed order through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"
#include "fwht.h"

namespace ck4 {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// LPB: lanes per Hadamard block (rot_block / 16); CL: lanes per row-chunk
// (at least 8, so a chunk is at least 128 elements); RANK: LoRA rank.
template <int LPB, int CL, int RANK>
__global__ __launch_bounds__(64 * kWaves) void lora_down_kernel(const uint16_t *__restrict__ x, int M, int K,
                                                                int64_t ldx, float c,
                                                                const uint16_t *__restrict__ a_rot, float alpha,
                                                                uint16_t *__restrict__ t) {
    constexpr int CH = 16 * CL;    // elements of a row per chunk
    constexpr int RP = 64 / CL;    // rows per rotation pass
    constexpr int NF = RANK / 16;  // output fragments of 16 rank columns
    constexpr int ROWB = CH * 2;   // LDS bytes per staged row
    constexpr int UNITS = ROWB / 16;
    constexpr int STAGE_B = kWaves * 16 * ROWB;
    constexpr int RED_B = (kWaves - 1) * NF * 64 * 16;
    static_assert(UNITS >= 8, "a staged row holds at least eight 16-byte units");
    __shared__ __attribute__((aligned(16))) uint8_t lds[STAGE_B > RED_B ? STAGE_B : RED_B];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m0 = blockIdx.x * 16;
    uint8_t *my = lds + wave * 16 * ROWB;
    const int nchunks = K / CH;
    const int per = (nchunks + kWaves - 1) / kWaves;
    const int c_begin = wave * per;
    const int c_end = min(nchunks, c_begin + per);
    // the sign each lane carries out of the cross-lane butterflies, folded into 1/sqrt(b)
    const float c_lane = (__popc(lane & (LPB - 1)) & 1) ? -c : c;
    const int lin = lane % CL;  // lane within its row's chunk
    const int rsub = lane / CL;  // row within a rotation pass
    auto unit_off = [](int u, int row) { return row * ROWB + ((u ^ (row & 7)) * 16); };

    v4f acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (int ci = c_begin; ci < c_end; ++ci) {
#pragma unroll
        for (int p = 0; p < 16 / RP; ++p) {
            const int rl = p * RP + rsub;
            const int m = m0 + rl;
            float v[kElems];
            if (m < M) {
                load_chunk(x + (int64_t)m * ldx + (int64_t)ci * CH + lin * kElems, v);
            } else {
#pragma unroll
                for (int i = 0; i < kElems; ++i) v[i] = 0.0f;
            }
            fwht_in_lane(v);
            fwht_cross_lane<LPB>(v, lane);
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = bf16_bits(v[2 * i] * c_lane) | (bf16_bits(v[2 * i + 1] * c_lane) << 16);
            *reinterpret_cast<uint4 *>(my + unit_off(2 * lin, rl)) = make_uint4(w[0], w[1], w[2], w[3]);
            *reinterpret_cast<uint4 *>(my + unit_off(2 * lin + 1, rl)) = make_uint4(w[4], w[5], w[6], w[7]);
        }
        // the wavefront reads back what it wrote (LDS operations of one
        // wavefront complete in order)
#pragma unroll
        for (int kk = 0; kk < CH / 32; ++kk) {
            // second operand: staged row (l & 15), the 8 k at 8 (l >> 4) of this 32-k slice
            const v8bf b = *reinterpret_cast<const v8bf *>(my + unit_off(kk * 4 + (lane >> 4), lane & 15));
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                // first operand: a_rot row 16 f + (l & 15), the same 8 k
                const v8bf a = *reinterpret_cast<const v8bf *>(
                    a_rot + (int64_t)(16 * f + (lane & 15)) * K + (int64_t)ci * CH + kk * 32 + 8 * (lane >> 4));
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[f], 0, 0, 0);
            }
        }
    }

    __syncthreads();  // the staging area becomes the reduction buffer
    v4f *red = reinterpret_cast<v4f *>(lds);
    if (wave > 0) {
#pragma unroll
        for (int f = 0; f < NF; ++f) red[((wave - 1) * NF + f) * 64 + lane] = acc[f];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll 1
    for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] += red[(w * NF + f) * 64 + lane];

    // lane holds t[m0 + (l & 15)][16 f + 4 (l >> 4) + r]
    const int m = m0 + (lane & 15);
    if (m >= M) return;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const uint32_t lo = bf16_bits(acc[f][0] * alpha) | (bf16_bits(acc[f][1] * alpha) << 16);
        const uint32_t hi = bf16_bits(acc[f][2] * alpha) | (bf16_bits(acc[f][3] * alpha) << 16);
        *reinterpret_cast<uint2 *>(t + (int64_t)m * RANK + 16 * f + 4 * (lane >> 4)) = make_uint2(lo, hi);
    }
}

template <int LPB, int RANK>
hipError_t launch_down(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, float c, const uint16_t *a_rot,
                       float alpha, uint16_t *t, hipStream_t stream) {
    constexpr int CL = LPB < 8 ? 8 : LPB;
    const dim3 grid((unsigned)((m + 15) / 16)), block(64 * kWaves);
    lora_down_kernel<LPB, CL, RANK><<<grid, block, 0, stream>>>(x, (int)m, (int)k, ldx, c, a_rot, alpha, t);
    return hipGetLastError();
}

template <int RANK>
hipError_t launch_down_rank(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                            const uint16_t *a_rot, float alpha, uint16_t *t, hipStream_t stream) {
    const float c = (float)(1.0 / __builtin_sqrt((double)rot_block));
    switch (rot_block / 16) {
    case 1: return launch_down<1, RANK>(x, m, k, ldx, c, a_rot, alpha, t, stream);
    case 2: return launch_down<2, RANK>(x, m, k, ldx, c, a_rot, alpha, t, stream);
    case 4: return launch_down<4, RANK>(x, m, k, ldx, c, a_rot, alpha, t, stream);
    case 8: return launch_down<8, RANK>(x, m, k, ldx, c, a_rot, alpha, t, stream);
    default: return launch_down<16, RANK>(x, m, k, ldx, c, a_rot, alpha, t, stream);
    }
}

}  // namespace

hipError_t launch_lora_down(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, const uint16_t *a_rot,
                            int64_t rank, float alpha, uint16_t *t, hipStream_t stream) {
    if (rank == 32) return launch_down_rank<32>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
    if (rank == 64) return launch_down_rank<64>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
    if (rank == 128) return launch_down_rank<128>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
    return launch_down_rank<256>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
}

}  // namespace ck4
