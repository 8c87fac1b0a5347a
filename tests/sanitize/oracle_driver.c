/* Driver of every function of oracle/ck4_oracle.c on small inputs, built
 * with the address and undefined-behaviour sanitizers (tests/test_sanitizers.py).
 *
 * Every buffer is a heap allocation of exactly the size the function's
 * contract states (strided inputs with their full stride), so a read or write
 * past it is reported; the inputs include a zero row, large and tiny values
 * (E4M3 saturation and subnormal scales) and the odd row counts and group
 * sizes the oracle accepts. Results are not checked here (the pins do that). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ck4o_num_threads(void);
void ck4o_set_num_threads(int n);
float ck4o_hadamard_scale_f32(int g);
void ck4o_fwht_f32(float *v, int g);
void ck4o_fwht_f64(double *v, int g);
void ck4o_rotate_rows_f32(const float *x, int64_t m, int64_t k, int64_t ldx, int g, float *r);
void ck4o_rotate_rows_bf16(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int g, float *r);
void ck4o_rotate_rows_f64(const double *x, int64_t m, int64_t k, int g, double *r);
void ck4o_quantize_rows(const float *r, int64_t m, int64_t k, int group, int qmax, int8_t *q, float *scales);
void ck4o_quantize_rows_sr(const float *r, const float *u, int64_t ldu, int64_t m, int64_t k, int group, int qmax,
                           int8_t *q, float *scales);
float ck4o_e4m3_decode(uint8_t b);
uint8_t ck4o_e4m3_encode(float x);
void ck4o_pack_int4(const int8_t *q, int64_t count, int8_t *packed);
void ck4o_unpack_int4(const int8_t *packed, int64_t count, int8_t *q);
void ck4o_quantize_weight_convrot(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                  int8_t *packed, float *scales);
void ck4o_quantize_weight_convrot_sr(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                     const float *u, int64_t ldu, int8_t *packed, float *scales);
void ck4o_quantize_weight_convrot_e4m3(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                       int8_t *packed, uint8_t *scales8);
void ck4o_rotate_quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int g, int bits, int8_t *out,
                              float *scales);
void ck4o_gemm_acc(const int8_t *a, const int8_t *b, int64_t m, int64_t n, int64_t k, int bits, int32_t *acc);
uint16_t ck4o_f64_to_bf16(double v);
void ck4o_f64_to_bf16_array(const double *v, int64_t count, uint16_t *out);
void ck4o_epilogue_bf16(const int32_t *acc, const float *sx, const float *sw, const float *bias, int64_t m,
                        int64_t n, int64_t ldy, uint16_t *y);
void ck4o_linear_w4a4(const uint16_t *x, const int8_t *w_packed, const float *w_scales, const float *bias,
                      int64_t m, int64_t n, int64_t k, int g, uint16_t *y);
void ck4o_decode_w4a8(const int8_t *w_packed, const float *group_scales, int64_t n, int64_t k, int group,
                      int64_t n0, int64_t nc, int8_t *w8, float *row_scales);
void ck4o_quantize_weight_convrot_codebook(const float *w, int64_t n, int64_t k, int64_t ldw, int g, int group,
                                           const float *cb, int e4m3, int8_t *packed, void *scales);
void ck4o_decode_w4a8_codebook(const int8_t *w_packed, const float *group_scales, const float *cb, int64_t n,
                               int64_t k, int group, int64_t n0, int64_t nc, int8_t *w8, float *row_scales);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* splitmix64 -> [0, 1) */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (double)((z ^ (z >> 31)) >> 11) * 0x1p-53;
}
static float normal(void) { return (float)(sqrt(-2.0 * log(1.0 - uniform())) * cos(6.283185307179586 * uniform())); }

static void *xalloc(size_t bytes) {
    void *p = malloc(bytes ? bytes : 1);
    if (!p) abort();
    return p;
}

static float *weights(int64_t n, int64_t ld) {
    float *w = xalloc((size_t)(n * ld) * sizeof(float));
    for (int64_t i = 0; i < n * ld; i++) w[i] = 0.02f * normal();
    for (int64_t j = 0; j < ld; j++) w[j] = 0.0f;                      /* row 0: all zero */
    if (n > 2) {
        for (int64_t j = 0; j < ld; j++) w[ld + j] *= 3e4f;            /* row 1: scales above 448 */
        for (int64_t j = 0; j < ld; j++) w[2 * ld + j] *= 1e-6f;       /* row 2: subnormal E4M3 scales */
    }
    return w;
}

static uint16_t *activations(int64_t m, int64_t ld) {
    uint16_t *x = xalloc((size_t)(m * ld) * sizeof(uint16_t));
    for (int64_t i = 0; i < m * ld; i++) {
        float f = normal() * ((i % 97) == 3 ? 20.0f : 1.0f);
        uint32_t u;
        memcpy(&u, &f, 4);
        x[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
    for (int64_t j = 0; j < ld; j++) x[j] = 0; /* row 0: all zero */
    return x;
}

int main(void) {
    ck4o_set_num_threads(2);
    if (ck4o_num_threads() < 1) return 1;
    (void)ck4o_hadamard_scale_f32(128);

    for (int g = 2; g <= 256; g *= 2) {
        float *v = xalloc(g * sizeof(float));
        double *d = xalloc(g * sizeof(double));
        for (int i = 0; i < g; i++) v[i] = (float)(d[i] = normal());
        ck4o_fwht_f32(v, g);
        ck4o_fwht_f64(d, g);
        free(v);
        free(d);
    }

    const int64_t m = 5, n = 7, k = 512, ldx = 520, ldw = 516;
    const int g = 128;
    float cb[16];
    for (int u = 0; u < 16; u++) cb[u] = (float)(u - 8) / 8.0f + 0.01f * (float)u;

    /* rotations */
    {
        float *w = weights(n, ldw);
        uint16_t *x = activations(m, ldx);
        float *r = xalloc((size_t)(m * k) * sizeof(float));
        float *rw = xalloc((size_t)(n * k) * sizeof(float));
        double *xd = xalloc((size_t)(m * k) * sizeof(double));
        double *rd = xalloc((size_t)(m * k) * sizeof(double));
        for (int64_t i = 0; i < m * k; i++) xd[i] = normal();
        for (int rb = 16; rb <= 512; rb *= 2) {
            ck4o_rotate_rows_bf16(x, m, k, ldx, rb, r);
            ck4o_rotate_rows_f32(w, n, k, ldw, rb, rw);
            ck4o_rotate_rows_f64(xd, m, k, rb, rd);
        }
        /* quantisers on the rotation, all group sizes, both code ranges */
        int8_t *q = xalloc((size_t)(n * k));
        float *u = xalloc((size_t)(n * (k + 4)) * sizeof(float));
        for (int64_t i = 0; i < n * (k + 4); i++) u[i] = (float)uniform();
        for (int grp = 0; grp <= 512; grp = grp ? grp * 2 : 4) {
            const int64_t ns = grp ? n * (k / grp) : n;
            float *s = xalloc((size_t)ns * sizeof(float));
            ck4o_quantize_rows(rw, n, k, grp, 7, q, s);
            ck4o_quantize_rows(rw, n, k, grp, 127, q, s);
            ck4o_quantize_rows_sr(rw, u, k + 4, n, k, grp, 7, q, s);
            free(s);
        }
        free(u);
        free(q);
        free(rd);
        free(xd);
        free(rw);
        free(r);
        free(x);
        free(w);
    }

    /* E4M3 and bf16 conversions over their whole ranges */
    for (int b = 0; b < 256; b++) (void)ck4o_e4m3_decode((uint8_t)b);
    for (int i = 0; i < 4000; i++) (void)ck4o_e4m3_encode((float)ldexp(normal(), (int)(uniform() * 40) - 20));
    (void)ck4o_e4m3_encode(1e30f);
    (void)ck4o_e4m3_encode(-0.0f);
    {
        const int64_t c = 64;
        double *v = xalloc(c * sizeof(double));
        uint16_t *o = xalloc(c * sizeof(uint16_t));
        for (int64_t i = 0; i < c; i++) v[i] = ldexp(normal(), (int)(uniform() * 300) - 150);
        v[0] = 0.0;
        v[1] = -0.0;
        v[2] = 1e300;
        v[3] = 1e-300;
        ck4o_f64_to_bf16_array(v, c, o);
        free(o);
        free(v);
    }

    /* pack / unpack of every nibble pair */
    {
        int8_t q[512], p[256], back[512];
        for (int i = 0; i < 512; i++) q[i] = (int8_t)((i % 16) - 8);
        ck4o_pack_int4(q, 512, p);
        ck4o_unpack_int4(p, 512, back);
    }

    /* weight preparation: per row, grouped, stochastic, E4M3, codebook */
    {
        float *w = weights(n, ldw);
        float *u = xalloc((size_t)(n * ldw) * sizeof(float));
        for (int64_t i = 0; i < n * ldw; i++) u[i] = (float)uniform();
        int8_t *wp = xalloc((size_t)(n * k / 2));
        for (int grp = 0; grp <= 512; grp = grp ? grp * 2 : 4) {
            const int64_t ns = grp ? n * (k / grp) : n;
            float *s = xalloc((size_t)ns * sizeof(float));
            ck4o_quantize_weight_convrot(w, n, k, ldw, g, grp, wp, s);
            ck4o_quantize_weight_convrot_sr(w, n, k, ldw, g, grp, u, ldw, wp, s);
            if (grp) {
                uint8_t *s8 = xalloc((size_t)ns);
                ck4o_quantize_weight_convrot_e4m3(w, n, k, ldw, g, grp, wp, s8);
                ck4o_quantize_weight_convrot_codebook(w, n, k, ldw, g, grp, cb, 1, wp, s8);
                ck4o_quantize_weight_convrot_codebook(w, n, k, ldw, g, grp, cb, 0, wp, s);
                /* decode rows [2, n) and the whole weight */
                int8_t *w8 = xalloc((size_t)(n * k));
                float *rs = xalloc((size_t)n * sizeof(float));
                ck4o_decode_w4a8_codebook(wp, s, cb, n, k, grp, 2, n - 2, w8, rs);
                ck4o_quantize_weight_convrot(w, n, k, ldw, g, grp, wp, s);
                ck4o_decode_w4a8(wp, s, n, k, grp, 0, n, w8, rs);
                ck4o_decode_w4a8(wp, s, n, k, grp, n - 1, 1, w8, rs);
                free(rs);
                free(w8);
                free(s8);
            }
            free(s);
        }
        free(wp);
        free(u);
        free(w);
    }

    /* activations, GEMM, epilogue, the whole layer */
    {
        uint16_t *x = activations(m, ldx);
        float *w = weights(n, k);
        int8_t *xq4 = xalloc((size_t)(m * k / 2));
        int8_t *xq8 = xalloc((size_t)(m * k));
        float *sx = xalloc((size_t)m * sizeof(float));
        int8_t *wp = xalloc((size_t)(n * k / 2));
        float *ws = xalloc((size_t)n * sizeof(float));
        int32_t *acc = xalloc((size_t)(m * n) * sizeof(int32_t));
        float *bias = xalloc((size_t)n * sizeof(float));
        const int64_t ldy = n + 3;
        uint16_t *y = xalloc((size_t)(m * ldy) * sizeof(uint16_t));
        for (int64_t j = 0; j < n; j++) bias[j] = normal();
        ck4o_rotate_quantize_act(x, m, k, ldx, g, 4, xq4, sx);
        ck4o_rotate_quantize_act(x, m, k, ldx, g, 8, xq8, sx);
        ck4o_quantize_weight_convrot(w, n, k, k, g, 0, wp, ws);
        ck4o_gemm_acc(xq4, wp, m, n, k, 4, acc);
        ck4o_epilogue_bf16(acc, sx, ws, bias, m, n, ldy, y);
        ck4o_epilogue_bf16(acc, sx, ws, NULL, m, n, ldy, y);
        int8_t *w8 = xalloc((size_t)(n * k));
        ck4o_unpack_int4(wp, n * k, w8);
        ck4o_gemm_acc(xq8, w8, m, n, k, 8, acc);
        free(w8);
        uint16_t *xc = activations(m, k);
        uint16_t *y2 = xalloc((size_t)(m * n) * sizeof(uint16_t));
        ck4o_linear_w4a4(xc, wp, ws, bias, m, n, k, g, y2);
        ck4o_linear_w4a4(xc, wp, ws, NULL, m, n, k, g, y2);
        free(y2);
        free(xc);
        free(y);
        free(bias);
        free(acc);
        free(ws);
        free(wp);
        free(sx);
        free(xq8);
        free(xq4);
        free(w);
        free(x);
    }
    /* the accumulator bound: all +7 codes at the largest k the library takes */
    {
        const int64_t kk = 131072;
        int8_t *a = xalloc((size_t)(kk / 2)), *b = xalloc((size_t)(kk / 2));
        memset(a, 0x77, (size_t)(kk / 2));
        memset(b, 0x99, (size_t)(kk / 2));
        int32_t acc1;
        ck4o_gemm_acc(a, b, 1, 1, kk, 4, &acc1);
        if (acc1 != -49 * kk) return 2;
        free(b);
        free(a);
    }
    printf("oracle driver ok\n");
    return 0;
}
