// LoRA up projection added to the fp32 values of an int8- or FP6-MFMA output
// tile, before its bf16 rounding (dynamic LoRA, "Comfy-INT4-HIPtest" README,
// LoRA modes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"

namespace ck4 {

typedef float lora_v4f __attribute__((ext_vector_type(4)));
typedef __bf16 lora_v8bf __attribute__((ext_vector_type(8)));

// y[i][j] += the LoRA term of output fragment (i, j): 16 columns from
// nbase + 16 i by 16 rows from mbase + 16 j (both multiples of 16), in the
// int8 accumulator layout (lane l: row l & 15, columns 4 (l >> 4) .. + 3).
// t and b are in MFMA fragment order (16-row x 32-column tiles of 512
// values in operand register order, tile (r / 16, c / 32) at
// ((r / 16) * (rank / 32) + c / 32) * 512), so each operand register is one
// contiguous 1 KB wavefront load: lane l reads the 16 bytes at 16 l. Each
// 32-wide slice of the rank is one v_mfma_f32_16x16x32_bf16 per fragment,
// first operand a tile of b, second a tile of t. Row blocks past the last
// one read the last one; their results are never stored. The whole
// wavefront runs it.
template <int FN, int FM>
__device__ __forceinline__ void lora_up(lora_v4f (&y)[FN][FM], const LoraUp lo, int nbase, int mbase, int N, int M,
                                        int lane) {
    const int tq = lo.rank / 32;
    const int nb_last = (N + 15) / 16 - 1, mb_last = (M + 15) / 16 - 1;
    const uint16_t *bp[FN];
    const uint16_t *tp[FM];
#pragma unroll
    for (int i = 0; i < FN; ++i) bp[i] = lo.b + (int64_t)min(nbase / 16 + i, nb_last) * tq * 512 + lane * 8;
#pragma unroll
    for (int j = 0; j < FM; ++j) tp[j] = lo.t + (int64_t)min(mbase / 16 + j, mb_last) * tq * 512 + lane * 8;
    // slices in pairs, the second slice's loads issued before the first
    // slice's MFMAs (loads retire in order, so those MFMAs do not wait for them)
    auto load = [&](lora_v8bf (&bf)[FN], lora_v8bf (&tf)[FM], int kk) {
#pragma unroll
        for (int i = 0; i < FN; ++i) bf[i] = *reinterpret_cast<const lora_v8bf *>(bp[i] + kk * 512);
#pragma unroll
        for (int j = 0; j < FM; ++j) tf[j] = *reinterpret_cast<const lora_v8bf *>(tp[j] + kk * 512);
    };
    auto madd = [&](const lora_v8bf (&bf)[FN], const lora_v8bf (&tf)[FM]) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) y[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[i], tf[j], y[i][j], 0, 0, 0);
    };
    for (int kk = 0; kk < tq; kk += 2) {
        lora_v8bf b0[FN], t0[FM], b1[FN], t1[FM];
        load(b0, t0, kk);
        if (kk + 1 < tq) load(b1, t1, kk + 1);
        madd(b0, t0);
        if (kk + 1 < tq) madd(b1, t1);
    }
}

}  // namespace ck4
