// Block Walsh-Hadamard butterflies on lane-held chunks, shared by the
// quantiser and the LoRA down-projection so that both produce the same fp32
// rotation ("[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with fused CUDA
// kernels", Description: the rotation stage of the activation kernel).
//
// A lane holds a chunk of 16 contiguous elements. Butterflies with stride
// 1..8 stay inside the chunk; stride 16 m pairs the lane with lane ^ m. Each
// cross-lane stage is u' = fma(u_partner, k, u) with k = -1 in the upper lane,
// so a lane carries a known sign (-1)^popcount(lane & (LPB - 1)) that the
// caller folds into the final multiply by 1/sqrt(b): the values are then
// bitwise those of the plain radix-2 butterflies with ascending stride.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck4 {
namespace {

constexpr int kElems = 16;  // contiguous elements per chunk

__device__ __forceinline__ void load_chunk(const uint16_t *p, float v[kElems]) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    uint4 a = q[0], b = q[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void load_chunk(const float *p, float v[kElems]) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 t = q[i];
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
}

// Butterflies with stride 1, 2, 4, 8 inside the chunk (ascending).
__device__ __forceinline__ void fwht_in_lane(float v[kElems]) {
#pragma unroll
    for (int h = 1; h < kElems; h <<= 1) {
#pragma unroll
        for (int i = 0; i < kElems; ++i) {
            if (i & h) continue;
            float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
}

// The value held by lane L ^ mask. The exchange goes through the LDS
// crossbar (ds_swizzle, ds_bpermute) rather than a DPP move, so it costs no
// VALU instruction: the kernel is bound by VALU issue.
template <int MASK>
__device__ __forceinline__ float partner(float x) {
    const int xi = __float_as_int(x);
    int r;
    if constexpr (MASK <= 16) {
        r = __builtin_amdgcn_ds_swizzle(xi, 0x1F | (MASK << 10));  // bitmask mode, xor MASK
    } else {
        r = __builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ MASK) << 2), xi);
    }
    return __int_as_float(r);
}

template <int MASK>
__device__ __forceinline__ void cross_stage(float v[kElems], int lane) {
    const float k = (lane & MASK) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < kElems; ++i) v[i] = __builtin_fmaf(partner<MASK>(v[i]), k, v[i]);
}

// All cross-lane stages for a block of LPB lanes (ascending mask).
template <int LPB>
__device__ __forceinline__ void fwht_cross_lane(float v[kElems], int lane) {
    if constexpr (LPB > 1) cross_stage<1>(v, lane);
    if constexpr (LPB > 2) cross_stage<2>(v, lane);
    if constexpr (LPB > 4) cross_stage<4>(v, lane);
    if constexpr (LPB > 8) cross_stage<8>(v, lane);
    if constexpr (LPB > 16) cross_stage<16>(v, lane);
    if constexpr (LPB > 32) cross_stage<32>(v, lane);
}

}  // namespace
}  // namespace ck4
