// LoRA down-projection of the dynamic LoRA side path, in the rotated basis.
//
// What it computes ("Comfy-INT4-HIPtest" README, LoRA modes: the Dynamic mode
// keeps the LoRA factors apart and adds their product at run time;
// "ComfyUI-INT4-Fast", Features: the LoRA down projection is rotated with the
// same Hadamard blocks as the weights, so that it matches the rotated
// activation):
//   r      = x * blockdiag(H_b, ..., H_b), accumulated in fp32, times fp32(1/sqrt(b))
//   t[m,j] = bf16(alpha * sum_k bf16(r[m,k]) * a_rot[j,k])    (fp32 accumulation)
// with a_rot = bf16(rotation of the unrotated down projection A). Because the
// rotation is orthonormal, r a_rot^T equals x A^T up to rounding.
//
// Everything runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16), with
// no LDS staging: the Hadamard block is a dense +-1 contraction, so a 16-row
// tile of x is rotated by MFMAs against +-1 fragments held in registers, and
// the rotated fragments leave the MFMA already in the operand layout of the
// LoRA product. Layouts (lane l, i = l & 15, g = l >> 4):
//  * an operand register holds 8 values of one row (first operand) or one
//    column (second operand), i, at k = 8 g + s of a 32-wide k slice; a
//    result holds rows 4 g + r, r < 4, of column i;
//  * rotation: first operand H[16 f + i][32 kk + 8 g + s], second operand the
//    16 bytes of x row i at 32 kk + 8 g; result fragment f holds the rotated
//    values o = 16 f + 4 g + r of row i;
//  * LoRA product, output pair p (fragments 2 p, 2 p + 1): second operand
//    slots s = the rotated values o = 32 p + 16 (s >> 2) + 4 g + (s & 3) of
//    row i, first operand the same 8 k of a_rot row j. Every o of the pair
//    appears once over (g, s), and both operands put the same k in the same
//    (g, s), which is all an MFMA needs.
// MFMA fragment order. a_rot, t and the up projection live in HBM as 16-row
// x 32-column tiles of 512 values in exactly that register order: element
// (i, c) of a tile at (16 ((c >> 2) & 3) + i) * 8 + 4 (c >> 4) + (c & 3),
// tile (r / 16, c / 32) at ((r / 16) * (cols / 32) + c / 32) * 512. One
// operand register of a wavefront is then one contiguous 1 KB load or store
// (lane l at 16 l bytes). Loading the same operands row-wise instead puts
// four different rows in every group of four lanes, which costs the address
// unit four times the cycles per load.
// H[o][k] = (-1)^popcount(o & k) inside a block. With o = 16 f + i and
// k = 32 kk + 8 g + s, the sign splits into a per-lane pattern over s (bits
// 0-3 of o and k), a per-lane flip (-1)^(f0 (g >> 1)) (bit 4) and a sign that
// depends only on f and kk (bits 5 and up), so four registers (P, -P, Q, -Q)
// hold every fragment of every block size from 32 up; 16-blocks use P masked
// to one half of the slice.
//
// A workgroup owns RT 16-row tiles (two when there are more than 256 tiles
// and rank and block are at most 128, else one); its 8 wavefronts split K in
// chunks of max(128, b) elements. Each wavefront prefetches the next chunks
// of x (and, at rank 32, of a_rot) while it multiplies the current one. The
// partial sums meet in a fixed-order tree through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck4_kernels.h"

namespace ck4 {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ v8bf as_v8bf(v4u u) { return __builtin_bit_cast(v8bf, u); }

__device__ __forceinline__ v4f mfma(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// G: Hadamard block; RANK: LoRA rank; RT: 16-row tiles per workgroup.
template <int G, int RANK, int RT>
__global__ __launch_bounds__(64 * kWaves) void lora_down_kernel(const uint16_t *__restrict__ x, int M, int K,
                                                                int64_t ldx, float c,
                                                                const uint16_t *__restrict__ a_rot, float alpha,
                                                                uint16_t *__restrict__ t) {
    constexpr int CH = G > 128 ? G : 128;  // k per chunk
    constexpr int KS = CH / 32;            // 32-wide k slices per chunk
    constexpr int NP = CH / 32;            // output fragment pairs per chunk
    constexpr int NF = RANK / 16;          // t fragments per row tile
    static_assert(G >= 16 && G <= 256 && (G & (G - 1)) == 0, "block size");
    __shared__ v4f red[kWaves / 2][RT][NF][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int g = lane >> 4;
    const int m0 = blockIdx.x * 16 * RT;
    const int nchunks = K / CH;
    const int per = (nchunks + kWaves - 1) / kWaves;
    const int c_begin = wave * per;
    const int c_end = min(nchunks, c_begin + per);

    // +-1 fragments: P[s] = (-1)^(popcount(i & s & 7) + ((i >> 3) & g & 1)),
    // Q = P (-1)^(g >> 1); bf16 1.0 = 0x3F80, sign bit 0x8000.
    uint32_t pw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t h = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int s = 2 * w + half;
            const uint32_t neg = (__popc(i & s & 7) + ((i >> 3) & g & 1)) & 1;
            h |= (0x3F80u | (neg << 15)) << (16 * half);
        }
        pw[w] = h;
    }
    const uint32_t qflip = (g >> 1) ? 0x80008000u : 0u;
    const v8bf P = as_v8bf(v4u{pw[0], pw[1], pw[2], pw[3]});
    const v8bf NP_ = as_v8bf(v4u{pw[0] ^ 0x80008000u, pw[1] ^ 0x80008000u, pw[2] ^ 0x80008000u, pw[3] ^ 0x80008000u});
    const v8bf Q = as_v8bf(v4u{pw[0] ^ qflip, pw[1] ^ qflip, pw[2] ^ qflip, pw[3] ^ qflip});
    const v8bf NQ = as_v8bf(v4u{pw[0] ^ qflip ^ 0x80008000u, pw[1] ^ qflip ^ 0x80008000u, pw[2] ^ qflip ^ 0x80008000u,
                                pw[3] ^ qflip ^ 0x80008000u});
    // 16-blocks: the slice's first 16 k (g < 2) or last 16 k (g >= 2)
    const v8bf Z0 = (g >> 1) ? as_v8bf(v4u{0, 0, 0, 0}) : P;
    const v8bf Z1 = (g >> 1) ? P : as_v8bf(v4u{0, 0, 0, 0});

    // rotation fragment for output fragment f and k slice kk of one chunk
    auto hfrag = [&](int f, int kk) -> v8bf {
        if constexpr (G == 16) {
            return (f & 1) ? Z1 : Z0;  // f == 2 kk + (f & 1)
        } else {
            const int fl = f % (G / 16);   // f within its block
            const int kl = kk % (G / 32);  // kk within its block
            const bool neg = __builtin_popcount((fl >> 1) & kl) & 1;
            return (fl & 1) ? (neg ? NQ : Q) : (neg ? NP_ : P);
        }
    };
    // the first k slice that feeds output fragment f, and how many do
    auto kk_first = [](int f) { return G == 16 ? f >> 1 : (f / (G / 16)) * (G / 32); };
    constexpr int KK_PER_F = G == 16 ? 1 : G / 32;

    const uint16_t *xrow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) xrow[rt] = x + (int64_t)min(m0 + 16 * rt + i, M - 1) * ldx + 8 * g;
    // a_rot in fragment order through a buffer descriptor: 16 lane bytes in
    // the VGPR offset, the tile in a scalar
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a_rot), (short)0, RANK * K * 2, 0x00020000);
    const uint32_t a_voff = (uint32_t)lane * 16u;
    const int kq = K / 32;  // tiles per 16 rows of a_rot

    v4f tacc[RT][NF];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int fr = 0; fr < NF; ++fr) tacc[rt][fr] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // One chunk's operands: its x fragments and its down-projection
    // fragments. Two chunks are in flight ahead of the MFMAs, each loaded as
    // a whole (x and a_rot together): memory loads retire in order, so a
    // fragment load issued after a later chunk's prefetch would make the
    // MFMAs wait for that prefetch too. Ranks whose fragments do not fit
    // twice in registers load them per output pair, one chunk ahead.
    constexpr bool PIPE = NP * NF <= 8;
    constexpr int NA = PIPE ? NP : 1;
    auto load_x = [&](v8bf (&dst)[RT][KS], int ci) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                dst[rt][kk] = *reinterpret_cast<const v8bf *>(xrow[rt] + (int64_t)ci * CH + 32 * kk);
    };
    auto load_af = [&](v8bf (&dst)[NF], int ci, int p) {
#pragma unroll
        for (int fr = 0; fr < NF; ++fr) {
            const uint32_t so = (uint32_t)(fr * kq + ci * (CH / 32) + p) * 1024u;
            dst[fr] = as_v8bf(__builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff, so, 0)));
        }
    };
    auto load_chunk = [&](v8bf (&xd)[RT][KS], v8bf (&ad)[NA][NF], int ci) {
        if constexpr (PIPE) {
#pragma unroll
            for (int p = 0; p < NP; ++p) load_af(ad[p], ci, p);
        }
        load_x(xd, ci);
    };
    auto compute = [&](const v8bf (&xf)[RT][KS], const v8bf (&ad)[NA][NF], int ci) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            v8bf af[NF];
            if constexpr (PIPE) {
#pragma unroll
                for (int fr = 0; fr < NF; ++fr) af[fr] = ad[p][fr];
            } else {
                load_af(af, ci, p);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                v4f r2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int f = 2 * p + h;
                    const int k0 = kk_first(f);
                    r2[h] = mfma(hfrag(f, k0), xf[rt][k0], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                    for (int q = 1; q < KK_PER_F; ++q) r2[h] = mfma(hfrag(f, k0 + q), xf[rt][k0 + q], r2[h]);
                }
                const v8bf xr = as_v8bf(v4u{bf16_bits(r2[0][0] * c) | (bf16_bits(r2[0][1] * c) << 16),
                                            bf16_bits(r2[0][2] * c) | (bf16_bits(r2[0][3] * c) << 16),
                                            bf16_bits(r2[1][0] * c) | (bf16_bits(r2[1][1] * c) << 16),
                                            bf16_bits(r2[1][2] * c) | (bf16_bits(r2[1][3] * c) << 16)});
#pragma unroll
                for (int fr = 0; fr < NF; ++fr) tacc[rt][fr] = mfma(af[fr], xr, tacc[rt][fr]);
            }
        }
    };

    if constexpr (PIPE) {
        v8bf x0[RT][KS], x1[RT][KS], a0[NA][NF], a1[NA][NF];
        if (c_begin < c_end) load_chunk(x0, a0, c_begin);
        if (c_begin + 1 < c_end) load_chunk(x1, a1, c_begin + 1);
        for (int ci = c_begin; ci < c_end; ci += 2) {
            compute(x0, a0, ci);
            if (ci + 2 < c_end) load_chunk(x0, a0, ci + 2);
            if (ci + 1 < c_end) {
                compute(x1, a1, ci + 1);
                if (ci + 3 < c_end) load_chunk(x1, a1, ci + 3);
            }
        }
    } else {
        v8bf xf[RT][KS], xn[RT][KS], none[NA][NF];
        if (c_begin < c_end) load_x(xn, c_begin);
        for (int ci = c_begin; ci < c_end; ++ci) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) xf[rt][kk] = xn[rt][kk];
            if (ci + 1 < c_end) load_x(xn, ci + 1);
            compute(xf, none, ci);
        }
    }

    // fixed-order tree: (w, w + 4), then (w, w + 2), then (0, 1); every
    // wavefront reaches every barrier
#pragma unroll
    for (int half = kWaves / 2; half >= 1; half /= 2) {
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int fr = 0; fr < NF; ++fr) red[wave - half][rt][fr][lane] = tacc[rt][fr];
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int fr = 0; fr < NF; ++fr) tacc[rt][fr] += red[wave][rt][fr][lane];
        }
        __syncthreads();
    }
    if (wave != 0) return;

    // Lane holds t[m0 + 16 rt + i][16 fr + 4 g + r]. In fragment order the
    // pair (2 q, 2 q + 1) of one lane is the 16 bytes at lane * 16 of tile
    // (row block, q): one contiguous 1 KB store per pair. Row blocks past the
    // last one that holds a row < M are not stored; rows >= M inside the last
    // block hold the clamped row's values.
    const int row_blocks = (M + 15) / 16;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rb = m0 / 16 + rt;
        if (rb >= row_blocks) continue;
#pragma unroll
        for (int q = 0; q < NF / 2; ++q) {
            const v4f a0 = tacc[rt][2 * q], a1 = tacc[rt][2 * q + 1];
            const uint4 o = make_uint4(bf16_bits(a0[0] * alpha) | (bf16_bits(a0[1] * alpha) << 16),
                                       bf16_bits(a0[2] * alpha) | (bf16_bits(a0[3] * alpha) << 16),
                                       bf16_bits(a1[0] * alpha) | (bf16_bits(a1[1] * alpha) << 16),
                                       bf16_bits(a1[2] * alpha) | (bf16_bits(a1[3] * alpha) << 16));
            *reinterpret_cast<uint4 *>(t + ((int64_t)rb * (NF / 2) + q) * 512 + lane * 8) = o;
        }
    }
}

// Up projection b (bf16 [n, rank], row stride ldb) to fragment order, rows
// padded with zeros to a multiple of 16. One thread per 16-byte unit u of
// the output: tile u / 64, lane l = u % 64 (row 16 (tile / (rank / 32)) +
// (l & 15), columns 32 (tile % (rank / 32)) + 4 (l >> 4) + {0..3, 16..19}).
__global__ __launch_bounds__(256) void lora_pack_kernel(const uint16_t *__restrict__ b, int n, int rank, int64_t ldb,
                                                        int64_t units, uint16_t *__restrict__ out) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const int l = (int)(u & 63);
    const int64_t tile = u >> 6;
    const int tq = rank / 32;
    const int64_t row = (tile / tq) * 16 + (l & 15);
    const int col = (int)(tile % tq) * 32 + 4 * (l >> 4);
    uint2 lo = make_uint2(0, 0), hi = make_uint2(0, 0);
    if (row < n) {
        const uint16_t *src = b + row * ldb + col;
        lo = make_uint2((uint32_t)src[0] | ((uint32_t)src[1] << 16), (uint32_t)src[2] | ((uint32_t)src[3] << 16));
        hi = make_uint2((uint32_t)src[16] | ((uint32_t)src[17] << 16), (uint32_t)src[18] | ((uint32_t)src[19] << 16));
    }
    *reinterpret_cast<uint4 *>(out + u * 8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

template <int G, int RANK>
hipError_t launch_down(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, const uint16_t *a_rot, float alpha,
                       uint16_t *t, hipStream_t stream) {
    // two 16-row tiles per workgroup (half the re-reads of a_rot) once one
    // tile per workgroup would take more than one workgroup per CU
    constexpr bool CAN_RT2 = RANK <= 128 && G <= 128;
    const float c = (float)(1.0 / __builtin_sqrt((double)G));
    const dim3 block(64 * kWaves);
    if (CAN_RT2 && (m + 15) / 16 > 256) {
        const dim3 grid((unsigned)((m + 31) / 32));
        lora_down_kernel<G, RANK, CAN_RT2 ? 2 : 1><<<grid, block, 0, stream>>>(x, (int)m, (int)k, ldx, c, a_rot,
                                                                                alpha, t);
    } else {
        const dim3 grid((unsigned)((m + 15) / 16));
        lora_down_kernel<G, RANK, 1><<<grid, block, 0, stream>>>(x, (int)m, (int)k, ldx, c, a_rot, alpha, t);
    }
    return hipGetLastError();
}

template <int RANK>
hipError_t launch_down_rank(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                            const uint16_t *a_rot, float alpha, uint16_t *t, hipStream_t stream) {
    switch (rot_block) {
    case 16: return launch_down<16, RANK>(x, m, k, ldx, a_rot, alpha, t, stream);
    case 32: return launch_down<32, RANK>(x, m, k, ldx, a_rot, alpha, t, stream);
    case 64: return launch_down<64, RANK>(x, m, k, ldx, a_rot, alpha, t, stream);
    case 128: return launch_down<128, RANK>(x, m, k, ldx, a_rot, alpha, t, stream);
    default: return launch_down<256, RANK>(x, m, k, ldx, a_rot, alpha, t, stream);
    }
}

}  // namespace

hipError_t launch_lora_pack(const uint16_t *b, int64_t n, int64_t rank, int64_t ldb, uint16_t *out,
                            hipStream_t stream) {
    const int64_t units = (n + 15) / 16 * (rank / 32) * 64;
    lora_pack_kernel<<<dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream>>>(b, (int)n, (int)rank, ldb, units,
                                                                                       out);
    return hipGetLastError();
}

hipError_t launch_lora_down(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, const uint16_t *a_rot,
                            int64_t rank, float alpha, uint16_t *t, hipStream_t stream) {
    if (rank == 32) return launch_down_rank<32>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
    if (rank == 64) return launch_down_rank<64>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
    if (rank == 128) return launch_down_rank<128>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
    return launch_down_rank<256>(x, m, k, ldx, rot_block, a_rot, alpha, t, stream);
}

}  // namespace ck4
