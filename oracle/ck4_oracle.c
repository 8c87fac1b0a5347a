/*
 * CPU oracle for the W4A4 ConvRot linear layer -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, step-by-step statement of what the layer
 * computes. Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product library never does, and the two
 * share no code, header, table or constant.
 *
 * Sources (web pages, cited by title and section):
 *  [PR63]  "[PR #63] int4_tensorwise: W4A4 layout (+ConvRot) with fused CUDA
 *          kernels" (comfy-kitchen), section "Description".
 *  [PR97]  "[PR #97] [MERGED] HIP port of #90: grouped W4A8 over the INT8
 *          GEMM" (comfy-kitchen), sections "What this adds", "Chunk sizing",
 *          "Testing".
 *  [HIPT]  "Comfy-INT4-HIPtest" README, section "What it provides".
 *  [FAST]  "ComfyUI-INT4-Fast" (comfy.icu listing), section "Features".
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes):
 *  - Hadamard: Sylvester order H_1 = [1], H_2n = [[H, H], [H, -H]], no random
 *    signs, applied independently to each contiguous block of g elements
 *    along K. Butterfly stages run with ascending stride h = 1, 2, ..., g/2;
 *    a radix-4 step is two consecutive radix-2 stages, smaller stride first,
 *    which gives bit-identical fp32 results. The rotation is orthonormal: the
 *    block result is multiplied by c_g = (float)(1/sqrt(g)) once, after the
 *    last stage.
 *  - Arithmetic of everything that decides an integer code is fp32 (the
 *    kernel's precision; the pages fix none): rotation, absmax, scale, the
 *    quotient. Scale s = absmax / 7 (fp32 divide), code q = rint(r / s)
 *    (fp32 divide, round half to even), clamped to [-7, 7]. An all-zero
 *    row (or group) has s = 0 and q = 0.
 *  - Packing: byte j = (q[2j] & 15) | (q[2j+1] & 15) << 4, even k in the low
 *    nibble [PR63].
 *  - Epilogue: y = bf16_rne(acc * s_x[m] * s_w[n] + bias[n]) evaluated in
 *    fp64 and rounded once to bf16.
 *  - Grouped W4A8 decode: s_row = (max_g s_g * 7) / 127, w8 = clamp(rint(q *
 *    (s_g / s_row)), -127, 127), all fp32; an all-zero row gives s_row = 0,
 *    w8 = 0.
 *  - Codebook ([PR97] "What this adds", "On #96"; the pages give no values
 *    and no mapping): the 4-bit code u (0..15, as stored) stands for cb[u]
 *    times the group scale, cmax = max |cb[u]|. Preparation: s = absmax /
 *    cmax, t = v / s (t = 0 when s = 0), u = the index of the smallest fp32
 *    |t - cb[u]|, the lowest index on ties. Decode: s_row = (max_g s_g *
 *    cmax) / 127, w8 = clamp(rint(cb[u] * (s_g / s_row)), -127, 127).
 *  - Dynamic LoRA ([HIPT] "LoRA modes", [FAST] "Features"): stated in the
 *    Python layer of the oracle (oracle/__init__.py), in fp64 over the bf16
 *    operands, with this file's rotation and bf16 rounding.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 * No FMA contraction and no reassociation, so every fp32 operation below is
 * the single IEEE operation it reads as.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int ck4o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void ck4o_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* Hadamard rotation ([PR63] Description: the rotation stage of the fused
 * activation kernel; [HIPT] What it provides; [FAST] Features).           */

/* The normalisation constant of a g-point orthonormal Hadamard transform,
 * rounded once to fp32. */
float ck4o_hadamard_scale_f32(int g) { return (float)(1.0 / sqrt((double)g)); }

/* In-place unnormalised fast Walsh-Hadamard transform of one block of g
 * fp32 values (g a power of two), radix-2 butterflies, ascending stride. */
void ck4o_fwht_f32(float *v, int g) {
    for (int h = 1; h < g; h *= 2) {
        for (int i = 0; i < g; i++) {
            if (i & h) continue;
            float a = v[i];
            float b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
}

/* The same transform in fp64 (used by checks of the rotation itself). */
void ck4o_fwht_f64(double *v, int g) {
    for (int h = 1; h < g; h *= 2) {
        for (int i = 0; i < g; i++) {
            if (i & h) continue;
            double a = v[i];
            double b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
}

/* r[row, :] = blockdiag(H_g, ..., H_g) * c_g applied to x[row, :] in fp32.
 * x is fp32 [m, ldx]; r is fp32 [m, k]. */
void ck4o_rotate_rows_f32(const float *x, int64_t m, int64_t k, int64_t ldx, int g, float *r) {
    const float c = ck4o_hadamard_scale_f32(g);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; row++) {
        float *out = r + row * k;
        memcpy(out, x + row * ldx, (size_t)k * sizeof(float));
        for (int64_t b0 = 0; b0 < k; b0 += g) {
            ck4o_fwht_f32(out + b0, g);
            for (int i = 0; i < g; i++) out[b0 + i] = out[b0 + i] * c;
        }
    }
}

/* Same, but the input is bf16 (uint16 bit patterns), widened exactly. */
void ck4o_rotate_rows_bf16(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int g, float *r) {
    const float c = ck4o_hadamard_scale_f32(g);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; row++) {
        float *out = r + row * k;
        for (int64_t j = 0; j < k; j++) {
            uint32_t u = ((uint32_t)x[row * ldx + j]) << 16;
            float f;
            memcpy(&f, &u, 4);
            out[j] = f;
        }
        for (int64_t b0 = 0; b0 < k; b0 += g) {
            ck4o_fwht_f32(out + b0, g);
            for (int i = 0; i < g; i++) out[b0 + i] = out[b0 + i] * c;
        }
    }
}

/* fp64 rotation with the exact normalisation 1/sqrt(g) (used by checks). */
void ck4o_rotate_rows_f64(const double *x, int64_t m, int64_t k, int g, double *r) {
    const double c = 1.0 / sqrt((double)g);
    for (int64_t row = 0; row < m; row++) {
        double *out = r + row * k;
        memcpy(out, x + row * k, (size_t)k * sizeof(double));
        for (int64_t b0 = 0; b0 < k; b0 += g) {
            ck4o_fwht_f64(out + b0, g);
            for (int i = 0; i < g; i++) out[b0 + i] *= c;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Symmetric absmax quantisation ([PR63]: rowwise int4 quantize; the int32
 * bound 49*K = 7*7*K fixes the code range to [-7, 7]). qmax = 7 for int4,
 * 127 for the int8 activations of the grouped W4A8 path ([PR97] "What this
 * adds": the decoded weight feeds the rowwise int8 GEMM).
 *
 * group == 0: one scale per row over all k (scales [m]).
 * group  > 0: one scale per contiguous group of `group` elements (scales
 *             [m, k/group]).
 * q is int8 [m, k], one code per element (unpacked). */
void ck4o_quantize_rows(const float *r, int64_t m, int64_t k, int group, int qmax, int8_t *q,
                        float *scales) {
    const int64_t gs = group > 0 ? group : k;
    const int64_t ng = k / gs;
    const float fq = (float)qmax;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; row++) {
        for (int64_t gi = 0; gi < ng; gi++) {
            const float *v = r + row * k + gi * gs;
            int8_t *out = q + row * k + gi * gs;
            float amax = 0.0f;
            for (int64_t j = 0; j < gs; j++) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            float s = amax / fq;
            scales[row * ng + gi] = s;
            for (int64_t j = 0; j < gs; j++) {
                if (s == 0.0f) {
                    out[j] = 0;
                    continue;
                }
                float t = rintf(v[j] / s);
                if (t > fq) t = fq;
                if (t < -fq) t = -fq;
                out[j] = (int8_t)t;
            }
        }
    }
}

/* Stochastic-rounding quantisation ([HIPT] LoRA modes, "Stochastic": LoRA
 * patches are baked into the weight with stochastic instead of nearest
 * rounding, so small updates survive in expectation). Reading: the scale and
 * the all-zero case are those of ck4o_quantize_rows; each element draws one
 * u in [0, 1) (supplied by the caller, u[row * ldu + col]) and
 *   t = RN(RN(v / s) + u)   (fp32),   q = clamp(floor(t), -qmax, qmax),
 * so q is floor(v/s) or floor(v/s) + 1 with E[q] = v/s up to fp32 rounding. */
void ck4o_quantize_rows_sr(const float *r, const float *u, int64_t ldu, int64_t m, int64_t k, int group, int qmax,
                           int8_t *q, float *scales) {
    const int64_t gs = group > 0 ? group : k;
    const int64_t ng = k / gs;
    const float fq = (float)qmax;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; row++) {
        for (int64_t gi = 0; gi < ng; gi++) {
            const float *v = r + row * k + gi * gs;
            const float *uv = u + row * ldu + gi * gs;
            int8_t *out = q + row * k + gi * gs;
            float amax = 0.0f;
            for (int64_t j = 0; j < gs; j++) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            float s = amax / fq;
            scales[row * ng + gi] = s;
            for (int64_t j = 0; j < gs; j++) {
                if (s == 0.0f) {
                    out[j] = 0;
                    continue;
                }
                float x = v[j] / s;
                float t = floorf(x + uv[j]);
                if (t > fq) t = fq;
                if (t < -fq) t = -fq;
                out[j] = (int8_t)t;
            }
        }
    }
}

/* FP8 E4M3 group scales ([PR97] What this adds: fp32 or e4m3 group scales).
 * The OCP E4M3 format: sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN; normals (1 + m/8) 2^(e-7), e = 1..15,
 * largest 448; subnormals (m/8) 2^-6. Reading for encoding (the pages name
 * only the format): round to nearest, ties to even, computed in double;
 * magnitudes at or above 448 saturate to 448. */
float ck4o_e4m3_decode(uint8_t b) {
    const int e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)((b & 0x80) ? -v : v);
}

uint8_t ck4o_e4m3_encode(float xf) {
    const double x = fabs((double)xf);
    const uint8_t sign = signbit(xf) ? 0x80 : 0x00;
    if (!(x < 448.0)) return sign | 0x7E;
    if (x < ldexp(1.0, -6)) {                 /* subnormal: a multiple of 2^-9 */
        const double m = nearbyint(x * 512.0); /* ties to even; 8 is the least normal */
        return sign | (uint8_t)m;
    }
    int ex;
    frexp(x, &ex);                 /* x = f 2^ex, f in [0.5, 1) */
    int e = ex - 1;                /* x = F 2^e, F in [1, 2) */
    double mm = nearbyint((ldexp(x, -e) - 1.0) * 8.0);
    if (mm == 8.0) {
        mm = 0.0;
        e += 1;
    }
    const int be = e + 7;
    if (be > 15 || (be == 15 && mm == 7.0)) return sign | 0x7E;
    return sign | (uint8_t)((be << 3) | (int)mm);
}

/* ------------------------------------------------------------------------- */
/* Packing of signed int4 pairs into bytes, the even element in the low nibble
 * ([PR63] Description: the weight layout is [N, K/2] bytes of code pairs);
 * unpacking is its exact inverse. */

void ck4o_pack_int4(const int8_t *q, int64_t count, int8_t *packed) {
    for (int64_t j = 0; j < count / 2; j++) {
        uint8_t lo = (uint8_t)q[2 * j] & 0x0F;
        uint8_t hi = (uint8_t)q[2 * j + 1] & 0x0F;
        packed[j] = (int8_t)(uint8_t)(lo | (hi << 4));
    }
}

static int8_t sext4(unsigned nib) { return (int8_t)(nib >= 8 ? (int)nib - 16 : (int)nib); }

void ck4o_unpack_int4(const int8_t *packed, int64_t count, int8_t *q) {
    for (int64_t j = 0; j < count / 2; j++) {
        uint8_t b = (uint8_t)packed[j];
        q[2 * j] = sext4(b & 0x0F);
        q[2 * j + 1] = sext4(b >> 4);
    }
}

/* ------------------------------------------------------------------------- */
/* Composed steps. */

/* Weight prep ([PR63] quantize_int4_convrot_weight): rotate each row of W in
 * fp32, quantise (per row when group == 0, per K-group otherwise), pack.
 * w fp32 [n, ldw]; packed int8 [n, k/2]; scales fp32 [n] or [n, k/group]. */
void ck4o_quantize_weight_convrot(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                  int8_t *packed, float *scales) {
    float *r = (float *)malloc((size_t)(n * k) * sizeof(float));
    int8_t *q = (int8_t *)malloc((size_t)(n * k));
    ck4o_rotate_rows_f32(w, n, k, ldw, g, r);
    ck4o_quantize_rows(r, n, k, group, 7, q, scales);
    ck4o_pack_int4(q, n * k, packed);
    free(q);
    free(r);
}

/* The weight preparation above with stochastic rounding (u fp32 [n, ldu]). */
void ck4o_quantize_weight_convrot_sr(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                     const float *u, int64_t ldu, int8_t *packed, float *scales) {
    float *r = (float *)malloc((size_t)(n * k) * sizeof(float));
    int8_t *q = (int8_t *)malloc((size_t)(n * k));
    ck4o_rotate_rows_f32(w, n, k, ldw, g, r);
    ck4o_quantize_rows_sr(r, u, ldu, n, k, group, 7, q, scales);
    ck4o_pack_int4(q, n * k, packed);
    free(q);
    free(r);
}

/* Grouped weight quantisation with e4m3 group scales: the fp32 group scale
 * absmax / 7 is rounded to e4m3, and the codes are taken against the value
 * that byte decodes to, clamp(rint(v / s8), -7, 7) (a scale that decodes to
 * 0 gives codes 0). */
void ck4o_quantize_weight_convrot_e4m3(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                       int8_t *packed, uint8_t *scales8) {
    float *r = (float *)malloc((size_t)(n * k) * sizeof(float));
    int8_t *q = (int8_t *)malloc((size_t)(n * k));
    ck4o_rotate_rows_f32(w, n, k, ldw, g, r);
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; row++) {
        for (int64_t gi = 0; gi < ng; gi++) {
            const float *v = r + row * k + gi * group;
            int8_t *out = q + row * k + gi * group;
            float amax = 0.0f;
            for (int64_t j = 0; j < group; j++) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            const uint8_t b = ck4o_e4m3_encode(amax / 7.0f);
            scales8[row * ng + gi] = b;
            const float s = ck4o_e4m3_decode(b);
            for (int64_t j = 0; j < group; j++) {
                if (s == 0.0f) {
                    out[j] = 0;
                    continue;
                }
                float t = rintf(v[j] / s);
                if (t > 7.0f) t = 7.0f;
                if (t < -7.0f) t = -7.0f;
                out[j] = (int8_t)t;
            }
        }
    }
    ck4o_pack_int4(q, n * k, packed);
    free(q);
    free(r);
}

/* Activation path ([PR63] Description: activations are rotated and quantised
 * to int4 at run time, inside the kernel): bf16 x [m, ldx] -> rotate ->
 * per-row quantise.
 * bits == 4: out is packed int8 [m, k/2], codes in [-7, 7].
 * bits == 8: out is int8 [m, k], codes in [-127, 127]. scales fp32 [m]. */
void ck4o_rotate_quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int g, int bits,
                              int8_t *out, float *scales) {
    float *r = (float *)malloc((size_t)(m * k) * sizeof(float));
    ck4o_rotate_rows_bf16(x, m, k, ldx, g, r);
    if (bits == 4) {
        int8_t *q = (int8_t *)malloc((size_t)(m * k));
        ck4o_quantize_rows(r, m, k, 0, 7, q, scales);
        ck4o_pack_int4(q, m * k, out);
        free(q);
    } else {
        ck4o_quantize_rows(r, m, k, 0, 127, out, scales);
    }
    free(r);
}

/* Integer GEMM ([PR63]: s4.s4 with int32 accumulation, |acc| <= 49*K):
 * acc[i, j] = sum_k a[i, k] * b[j, k]. Operands are packed int4 (bits == 4,
 * [rows, k/2]) or int8 codes (bits == 8, [rows, k]); both are K-major. */
void ck4o_gemm_acc(const int8_t *a, const int8_t *b, int64_t m, int64_t n, int64_t k, int bits,
                   int32_t *acc) {
    int8_t *au = (int8_t *)malloc((size_t)(m * k));
    int8_t *bu = (int8_t *)malloc((size_t)(n * k));
    if (bits == 4) {
        ck4o_unpack_int4(a, m * k, au);
        ck4o_unpack_int4(b, n * k, bu);
    } else {
        memcpy(au, a, (size_t)(m * k));
        memcpy(bu, b, (size_t)(n * k));
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++) {
        for (int64_t j = 0; j < n; j++) {
            const int8_t *ar = au + i * k;
            const int8_t *br = bu + j * k;
            int32_t s = 0;
            for (int64_t t = 0; t < k; t++) s += (int32_t)ar[t] * (int32_t)br[t];
            acc[i * n + j] = s;
        }
    }
    free(bu);
    free(au);
}

/* Round an fp64 value to the nearest bf16 (ties to even), directly from
 * fp64 so there is one rounding. Values beyond the bf16 range saturate to
 * +-inf; bf16 subnormals are rounded on the subnormal grid. */
uint16_t ck4o_f64_to_bf16(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    if (isnan(v)) return 0x7FC0;
    int e;
    double mant = frexp(fabs(v), &e); /* |v| = mant * 2^e, mant in [0.5, 1) */
    /* bf16 keeps 8 significant bits; the smallest normal exponent is -126,
     * so below that the grid spacing stays 2^-133. */
    int keep = 8;
    if (e - 1 < -126) keep = 8 - (-126 - (e - 1));
    double scaled = ldexp(mant, keep);
    double rounded = nearbyint(scaled); /* round half to even */
    double y = ldexp(rounded, e - keep);
    float f = (float)y; /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) u = (u & 0x80000000u) | 0x7F800000u;
    uint16_t out = (uint16_t)(u >> 16);
    if (signbit(v)) out |= 0x8000;
    return out;
}

/* Element-wise single rounding of fp64 values to bf16 bits. */
void ck4o_f64_to_bf16_array(const double *v, int64_t count, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) out[i] = ck4o_f64_to_bf16(v[i]);
}

/* Rank-one epilogue ([PR63] Description: the row and column scales do not
 * depend on k, so they are applied once after the integer sum): y[i, j] = bf16(acc[i, j] * sx[i] * sw[j] (+ bias[j])), evaluated in
 * fp64. y is bf16 bits with row stride ldy. bias may be NULL. */
void ck4o_epilogue_bf16(const int32_t *acc, const float *sx, const float *sw, const float *bias,
                        int64_t m, int64_t n, int64_t ldy, uint16_t *y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; i++) {
        for (int64_t j = 0; j < n; j++) {
            double v = (double)acc[i * n + j] * (double)sx[i] * (double)sw[j];
            if (bias) v += (double)bias[j];
            y[i * ldy + j] = ck4o_f64_to_bf16(v);
        }
    }
}

/* Full W4A4 linear: bf16 x [m, k] against a prepared weight. */
void ck4o_linear_w4a4(const uint16_t *x, const int8_t *w_packed, const float *w_scales, const float *bias,
                      int64_t m, int64_t n, int64_t k, int g, uint16_t *y) {
    int8_t *xq = (int8_t *)malloc((size_t)(m * k / 2));
    float *sx = (float *)malloc((size_t)m * sizeof(float));
    int32_t *acc = (int32_t *)malloc((size_t)(m * n) * sizeof(int32_t));
    ck4o_rotate_quantize_act(x, m, k, k, g, 4, xq, sx);
    ck4o_gemm_acc(xq, w_packed, m, n, k, 4, acc);
    ck4o_epilogue_bf16(acc, sx, w_scales, bias, m, n, n, y);
    free(acc);
    free(sx);
    free(xq);
}

/* ------------------------------------------------------------------------- */
/* Grouped W4A8 ([PR97] "What this adds"): int4 codes with fp32 scales per
 * group of `group` elements along K are decoded to int8 codes with a single
 * fp32 scale per output row, so the rowwise int8 GEMM's rank-one epilogue
 * still applies. Rows [n0, n0 + nc) of the weight are decoded (the chunked
 * path of [PR97] "Chunk sizing"); w8 is int8 [nc, k], row_scales fp32 [nc]. */
void ck4o_decode_w4a8(const int8_t *w_packed, const float *group_scales, int64_t n, int64_t k, int group,
                      int64_t n0, int64_t nc, int8_t *w8, float *row_scales) {
    (void)n;
    const int64_t ng = k / group;
    for (int64_t i = 0; i < nc; i++) {
        const int64_t row = n0 + i;
        const float *sg = group_scales + row * ng;
        float smax = 0.0f;
        for (int64_t gi = 0; gi < ng; gi++)
            if (sg[gi] > smax) smax = sg[gi];
        float srow = (smax * 7.0f) / 127.0f;
        row_scales[i] = srow;
        for (int64_t gi = 0; gi < ng; gi++) {
            float mult = srow == 0.0f ? 0.0f : sg[gi] / srow;
            for (int64_t j = 0; j < group; j++) {
                int64_t kk = gi * group + j;
                uint8_t byte = (uint8_t)w_packed[row * (k / 2) + kk / 2];
                int8_t qv = sext4((kk & 1) ? (byte >> 4) : (byte & 0x0F));
                float t = rintf((float)qv * mult);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
                w8[i * k + kk] = (int8_t)t;
            }
        }
    }
}

/* ---- Codebook variant of the grouped W4A8 weight ([PR97] "What this adds":
 * an optional codebook for the decode; "On #96": a frozen codebook lookup
 * table). cb holds 16 fp32 entries; cmax = max |cb[u]| (assumed > 0). */

static float codebook_cmax(const float *cb) {
    float c = 0.0f;
    for (int u = 0; u < 16; u++)
        if (fabsf(cb[u]) > c) c = fabsf(cb[u]);
    return c;
}

/* Index of the entry nearest to t by the fp32 distance |t - cb[u]|, the
 * lowest index among equal distances. */
static int codebook_nearest(float t, const float *cb) {
    int best = 0;
    float bd = fabsf(t - cb[0]);
    for (int u = 1; u < 16; u++) {
        float d = fabsf(t - cb[u]);
        if (d < bd) {
            bd = d;
            best = u;
        }
    }
    return best;
}

/* Rotate the rows in fp32, then for each group of `group` elements along K:
 * s = absmax / cmax (with e4m3 != 0 rounded to e4m3: the byte is stored and
 * its decoded value used), t = v / s (0 when s = 0), code = nearest entry.
 * packed int8 [n, k/2] holds the indices, even k in the low nibble; scales
 * is fp32 [n, k/group] or, with e4m3, uint8 [n, k/group]. */
void ck4o_quantize_weight_convrot_codebook(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                           const float *cb, int e4m3, int8_t *packed, void *scales) {
    float *r = (float *)malloc((size_t)(n * k) * sizeof(float));
    int8_t *u = (int8_t *)malloc((size_t)(n * k));
    ck4o_rotate_rows_f32(w, n, k, ldw, g, r);
    const float cmax = codebook_cmax(cb);
    const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < n; row++) {
        for (int64_t gi = 0; gi < ng; gi++) {
            const float *v = r + row * k + gi * group;
            int8_t *out = u + row * k + gi * group;
            float amax = 0.0f;
            for (int64_t j = 0; j < group; j++) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            float s = amax / cmax;
            if (e4m3) {
                const uint8_t b = ck4o_e4m3_encode(s);
                ((uint8_t *)scales)[row * ng + gi] = b;
                s = ck4o_e4m3_decode(b);
            } else {
                ((float *)scales)[row * ng + gi] = s;
            }
            for (int64_t j = 0; j < group; j++) {
                const float t = s == 0.0f ? 0.0f : v[j] / s;
                out[j] = (int8_t)codebook_nearest(t, cb);
            }
        }
    }
    ck4o_pack_int4(u, n * k, packed);
    free(u);
    free(r);
}

/* Decode of rows [n0, n0 + nc) of a codebook weight with fp32 group scales:
 * s_row = (max_g s_g * cmax) / 127, w8 = clamp(rint(cb[u] * (s_g / s_row)),
 * -127, 127), all fp32; an all-zero row gives s_row = 0 and w8 = 0. */
void ck4o_decode_w4a8_codebook(const int8_t *w_packed, const float *group_scales, const float *cb, int64_t n,
                               int64_t k, int group, int64_t n0, int64_t nc, int8_t *w8, float *row_scales) {
    (void)n;
    const float cmax = codebook_cmax(cb);
    const int64_t ng = k / group;
    for (int64_t i = 0; i < nc; i++) {
        const int64_t row = n0 + i;
        const float *sg = group_scales + row * ng;
        float smax = 0.0f;
        for (int64_t gi = 0; gi < ng; gi++)
            if (sg[gi] > smax) smax = sg[gi];
        const float srow = (smax * cmax) / 127.0f;
        row_scales[i] = srow;
        for (int64_t gi = 0; gi < ng; gi++) {
            const float mult = srow == 0.0f ? 0.0f : sg[gi] / srow;
            for (int64_t j = 0; j < group; j++) {
                const int64_t kk = gi * group + j;
                const uint8_t byte = (uint8_t)w_packed[row * (k / 2) + kk / 2];
                const unsigned code = (kk & 1) ? (byte >> 4) : (byte & 0x0F);
                float t = rintf(cb[code] * mult);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
                w8[i * k + kk] = (int8_t)t;
            }
        }
    }
}
