// Host-only driver of the C ABI's argument validation, built with the
// address and undefined-behaviour sanitizers (tests/test_sanitizers.py).
//
// The HIP runtime calls the validation layer makes and the kernel launchers
// are replaced by stand-ins: the device query reports no device, a gfx950 or
// another GPU (argv[1] = none | gfx950 | other), and each launcher only counts
// its calls. Every entry point is called with valid arguments and with each
// kind of invalid one (null, misaligned, short strides, unsupported shapes,
// and sizes at the int64 limits, where an unchecked product would overflow).
// A rejected call must return its documented status and launch nothing; a
// valid call must launch exactly the expected kernels when the device is a
// gfx950 and nothing otherwise.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "ck4.h"
#include "ck4_kernels.h"
#include "gemv.h"

static int g_mode = 0;  // 0: no device, 1: gfx950, 2: another GPU
static int g_launches = 0;

hipError_t hipGetDevice(int *d) {
    if (g_mode == 0) return hipErrorNoDevice;
    *d = 0;
    return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t *p, int) {
    std::memset(p, 0, sizeof *p);
    std::strcpy(p->gcnArchName, g_mode == 1 ? "gfx950:sramecc+:xnack-" : "gfx942:sramecc+:xnack-");
    p->l2CacheSize = 4 << 20;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t) { return "stand-in"; }

namespace ck4 {
hipError_t launch_rotate_quant(const void *, int, int64_t, int64_t, int64_t, int, int, int, void *, int64_t, float *,
                               hipStream_t, WeightOpts) { return ++g_launches, hipSuccess; }
hipError_t launch_gemm(bool, const int8_t *, const int8_t *, const float *, const float *, const float *, int64_t,
                       int64_t, int64_t, bool, void *, int64_t, hipStream_t, LoraUp) { return ++g_launches, hipSuccess; }
hipError_t launch_gemm_fp6(const uint8_t *, const uint8_t *, const float *, const float *, const float *, int64_t,
                           int64_t, int64_t, bool, void *, int64_t, hipStream_t, LoraUp, bool) {
    return ++g_launches, hipSuccess;
}
hipError_t launch_lora_pack(const uint16_t *, int64_t, int64_t, int64_t, uint16_t *, hipStream_t) {
    return ++g_launches, hipSuccess;
}
hipError_t launch_lora_down(const uint16_t *, int64_t, int64_t, int64_t, int, const uint16_t *, int64_t, float,
                            uint16_t *, hipStream_t) { return ++g_launches, hipSuccess; }
hipError_t launch_w4a8_decode(const int8_t *, const void *, bool, int64_t, int, int64_t, int64_t, int8_t *, float *,
                              hipStream_t, const Codebook &) { return ++g_launches, hipSuccess; }
hipError_t launch_w4a8_fused(const int8_t *, const float *, const int8_t *, const void *, bool, int64_t, int64_t,
                             int64_t, int, uint16_t *, int64_t, hipStream_t, const Codebook &) {
    return ++g_launches, hipSuccess;
}
// the fused decode-time layer's shape rule, reduced to what these calls need:
// m <= 2 with 128-blocks takes the one-launch kernel, anything else the
// quantiser followed by the GEMM (two launches)
bool skinny_layer_fits(int64_t m, int64_t, int64_t k, int rot_block) { return m >= 1 && m <= 2 && rot_block == 128 && k <= 8192; }
hipError_t launch_skinny_layer(const uint16_t *, int64_t, const int8_t *, const float *, const float *, int64_t,
                               int64_t, int64_t, int8_t *, float *, uint16_t *, int64_t, hipStream_t) {
    return ++g_launches, hipSuccess;
}
bool gemv_w4a4_fits(int64_t m, int64_t k) { return m >= 1 && m <= 2 && k >= 256 && k % 128 == 0 && k <= 16384; }
hipError_t launch_gemv_w4a4(const int8_t *, const float *, const int8_t *, const float *, const float *, int64_t,
                            int64_t, int64_t, uint16_t *, int64_t, hipStream_t) {
    return ++g_launches, hipSuccess;
}
bool w4a8_gemv_fits(int64_t m, int64_t n, int64_t, int, bool codebook) { return !codebook && m <= 2 && n <= 8192; }
hipError_t launch_w4a8_gemv(const int8_t *, const float *, const int8_t *, const void *, bool, int64_t, int64_t,
                            int64_t, int, uint16_t *, int64_t, hipStream_t) {
    return ++g_launches, hipSuccess;
}
bool w4a8_layer_fits(int64_t m, int64_t n, int64_t k, int rot_block, int group, bool codebook, bool) {
    return !codebook && m == 1 && n <= 8192 && rot_block == 128 && group >= 32 && k <= 8192;
}
hipError_t launch_w4a8_layer(const uint16_t *, int64_t, const int8_t *, const void *, bool, int64_t, int64_t,
                             int64_t, int, int8_t *, float *, uint16_t *, int64_t, hipStream_t) {
    return ++g_launches, hipSuccess;
}
alignas(256) static unsigned char g_fake_scratch[256];
hipError_t noalloc_scratch(int, void **ptr) {
    *ptr = g_fake_scratch;
    return hipSuccess;
}
}  // namespace ck4

static int g_fails = 0;
static int g_checked = 0;

// ok_launches: launches of a valid call on a gfx950; on another device or
// none the same call must fail with CK4_ERR_DEVICE and launch nothing.
#define VALID(call, ok_launches)                                                                       \
    do {                                                                                               \
        const int before = g_launches;                                                                 \
        const ck4_status s = (call);                                                                   \
        const int want_s = g_mode == 1 ? CK4_OK : CK4_ERR_DEVICE;                                      \
        const int want_l = g_mode == 1 ? (ok_launches) : 0;                                           \
        ++g_checked;                                                                                   \
        if (s != want_s || g_launches - before != want_l) {                                            \
            std::fprintf(stderr, "line %d: %s -> status %d (want %d), %d launches (want %d): %s\n",     \
                         __LINE__, #call, (int)s, want_s, g_launches - before, want_l, ck4_last_error()); \
            ++g_fails;                                                                                 \
        }                                                                                              \
    } while (0)

#define REFUSED(call, status)                                                                          \
    do {                                                                                               \
        const int before = g_launches;                                                                 \
        const ck4_status s = (call);                                                                   \
        ++g_checked;                                                                                   \
        if (s != (status) || g_launches != before || std::strlen(ck4_last_error()) == 0) {             \
            std::fprintf(stderr, "line %d: %s -> status %d (want %d), %d launches: %s\n", __LINE__,     \
                         #call, (int)s, (int)(status), g_launches - before, ck4_last_error());          \
            ++g_fails;                                                                                 \
        }                                                                                              \
    } while (0)

// A refusal whose status may be INVALID or UNSUPPORTED (sizes out of range).
#define REJECTED(call)                                                                                 \
    do {                                                                                               \
        const int before = g_launches;                                                                 \
        const ck4_status s = (call);                                                                   \
        ++g_checked;                                                                                   \
        if (s == CK4_OK || g_launches != before) {                                                     \
            std::fprintf(stderr, "line %d: %s -> status %d, %d launches\n", __LINE__, #call, (int)s,   \
                         g_launches - before);                                                         \
            ++g_fails;                                                                                 \
        }                                                                                              \
    } while (0)

alignas(256) static unsigned char g_buf[4096];

int main(int argc, char **argv) {
    const std::string mode = argc > 1 ? argv[1] : "none";
    g_mode = mode == "gfx950" ? 1 : mode == "other" ? 2 : 0;
    void *P = g_buf;                 // 256-byte aligned stand-in device pointer, never dereferenced
    void *ODD = g_buf + 4;           // misaligned
    float *F = (float *)P;
    int8_t *I8 = (int8_t *)P;
    uint8_t *U8 = (uint8_t *)P;
    uint16_t *U16 = (uint16_t *)P;
    int32_t *I32 = (int32_t *)P;
    const int64_t BIG = INT64_MAX, NEG = INT64_MIN;
    float cb[16];
    for (int u = 0; u < 16; ++u) cb[u] = (float)(u - 8) / 8.0f;
    float cb_nan[16];
    std::memcpy(cb_nan, cb, sizeof cb);
    cb_nan[5] = __builtin_nanf("");
    float cb_zero[16] = {};

    // ---- weight preparation
    VALID(ck4_quantize_weight_convrot(F, 64, 256, 256, 128, 0, I8, F, nullptr), 1);
    VALID(ck4_quantize_weight_convrot(F, 64, 256, 260, 128, 128, I8, F, nullptr), 1);
    REFUSED(ck4_quantize_weight_convrot(nullptr, 64, 256, 256, 128, 0, I8, F, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot(F, 0, 256, 256, 128, 0, I8, F, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot(F, 64, 256, 200, 128, 0, I8, F, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot(F, 64, 256, 258, 128, 0, I8, F, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot((float *)ODD, 64, 256, 256, 128, 0, I8, F, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot(F, 64, 256, 256, 96, 0, I8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_quantize_weight_convrot(F, 64, 384, 384, 256, 0, I8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_quantize_weight_convrot(F, 64, 32768, 32768, 128, 0, I8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_quantize_weight_convrot(F, 64, 256, 256, 128, 3, I8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_quantize_weight_convrot(F, 64, 256, 256, 128, 2048, I8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_quantize_weight_convrot(F, BIG, 256, 256, 128, 0, I8, F, nullptr));
    REJECTED(ck4_quantize_weight_convrot(F, NEG, 256, 256, 128, 0, I8, F, nullptr));
    REJECTED(ck4_quantize_weight_convrot(F, 64, BIG, BIG, 128, 0, I8, F, nullptr));
    REJECTED(ck4_quantize_weight_convrot(F, 64, 256, BIG, 128, 0, I8, F, nullptr));
    REJECTED(ck4_quantize_weight_convrot(F, 64, 256, NEG, 128, 0, I8, F, nullptr));
    VALID(ck4_quantize_weight_convrot_sr(F, 64, 256, 256, 128, 0, F, 256, I8, F, nullptr), 1);
    REFUSED(ck4_quantize_weight_convrot_sr(F, 64, 256, 256, 128, 0, nullptr, 256, I8, F, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot_sr(F, 64, 256, 256, 128, 0, F, 100, I8, F, nullptr), CK4_ERR_INVALID);
    REJECTED(ck4_quantize_weight_convrot_sr(F, 64, 256, 256, 128, 0, F, BIG, I8, F, nullptr));
    VALID(ck4_quantize_weight_convrot_e4m3(F, 64, 256, 256, 128, 64, I8, U8, nullptr), 1);
    REFUSED(ck4_quantize_weight_convrot_e4m3(F, 64, 256, 256, 128, 0, I8, U8, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_quantize_weight_convrot_e4m3(F, 64, 256, BIG, 128, 64, I8, U8, nullptr));
    VALID(ck4_quantize_weight_convrot_codebook(F, 64, 256, 256, 128, 64, cb, 0, I8, F, nullptr), 1);
    VALID(ck4_quantize_weight_convrot_codebook(F, 64, 256, 256, 128, 4, cb, 1, I8, U8, nullptr), 1);
    REFUSED(ck4_quantize_weight_convrot_codebook(F, 64, 256, 256, 128, 64, nullptr, 0, I8, F, nullptr),
            CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot_codebook(F, 64, 256, 256, 128, 64, cb_nan, 0, I8, F, nullptr),
            CK4_ERR_INVALID);
    REFUSED(ck4_quantize_weight_convrot_codebook(F, 64, 256, 256, 128, 64, cb_zero, 0, I8, F, nullptr),
            CK4_ERR_INVALID);
    VALID(ck4_quantize_weight_convrot_int8(F, 64, 256, 256, 128, I8, F, nullptr), 1);
    REFUSED(ck4_quantize_weight_convrot_int8(F, 64, 256, 256, 128, (int8_t *)ODD, F, nullptr), CK4_ERR_INVALID);
    REJECTED(ck4_quantize_weight_convrot_int8(F, BIG, BIG, BIG, 128, I8, F, nullptr));

    // ---- activation quantisers and the fp32 rotation
    VALID(ck4_rotate_quantize_act(U16, 8, 256, 256, 128, 4, I8, F, nullptr), 1);
    VALID(ck4_rotate_quantize_act(U16, 8, 256, 264, 128, 8, I8, F, nullptr), 1);
    REFUSED(ck4_rotate_quantize_act(U16, 8, 256, 256, 128, 5, I8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_rotate_quantize_act(U16, 8, 256, 260, 128, 4, I8, F, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_rotate_quantize_act(U16, 8, 256, 256, 128, 8, (int8_t *)(g_buf + 8), F, nullptr), CK4_ERR_INVALID);
    REJECTED(ck4_rotate_quantize_act(U16, BIG, 256, 256, 128, 4, I8, F, nullptr));
    REJECTED(ck4_rotate_quantize_act(U16, 8, 256, BIG, 128, 4, I8, F, nullptr));
    REJECTED(ck4_rotate_quantize_act(U16, 8, NEG, 256, 128, 4, I8, F, nullptr));
    VALID(ck4_rotate_act_f32(U16, 8, 256, 256, 64, F, nullptr), 1);
    REJECTED(ck4_rotate_act_f32(U16, 8, 256, BIG, 64, F, nullptr));

    // ---- GEMMs on packed int4 and int8
    VALID(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, 256, U16, 8, nullptr), 1);
    VALID(ck4_linear_w4a4(I8, F, I8, F, F, 100, 200, 1024, U16, 204, nullptr), 1);
    REFUSED(ck4_linear_w4a4(I8, nullptr, I8, F, nullptr, 8, 8, 256, U16, 8, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, 256, U16, 6, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, 256, (uint16_t *)ODD, 8, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, 192, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, 128, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    VALID(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, 384, U16, 8, nullptr), 1);
    VALID(ck4_linear_w4a4(I8, F, I8, F, F, 3, 5000, 640, U16, 5000, nullptr), 1);   // the matrix-vector kernel
    VALID(ck4_linear_w4a4(I8, F, I8, F, F, 1, 5000, 16384, U16, 5000, nullptr), 1);  // k past it: the GEMM
    REFUSED(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, 262144, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_linear_w4a4(I8, F, I8, F, nullptr, BIG, 8, 256, U16, 8, nullptr));

    // the whole layer from bf16: one launch for m <= 2 (128-blocks), else two
    VALID(ck4_linear_w4a4_bf16(U16, 1, 3072, 3072, 128, I8, F, F, 12288, I8, F, U16, 12288, nullptr), 1);
    VALID(ck4_linear_w4a4_bf16(U16, 2, 384, 392, 128, I8, F, nullptr, 5, I8, F, U16, 8, nullptr), 1);
    VALID(ck4_linear_w4a4_bf16(U16, 4, 384, 392, 128, I8, F, nullptr, 5, I8, F, U16, 8, nullptr), 2);
    VALID(ck4_linear_w4a4_bf16(U16, 64, 3072, 3072, 128, I8, F, nullptr, 300, I8, F, U16, 300, nullptr), 2);
    VALID(ck4_linear_w4a4_bf16(U16, 2, 1024, 1024, 64, I8, F, nullptr, 300, I8, F, U16, 300, nullptr), 2);
    REFUSED(ck4_linear_w4a4_bf16(nullptr, 1, 256, 256, 128, I8, F, F, 8, I8, F, U16, 8, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 256, 256, 128, I8, F, F, 8, nullptr, F, U16, 8, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 256, 256, 128, I8, F, F, 8, (int8_t *)ODD, F, U16, 8, nullptr),
            CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 256, 200, 128, I8, F, F, 8, I8, F, U16, 8, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 256, 260, 128, I8, F, F, 8, I8, F, U16, 8, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 128, 128, 128, I8, F, F, 8, I8, F, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 320, 320, 64, I8, F, F, 8, I8, F, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 256, 256, 100, I8, F, F, 8, I8, F, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_linear_w4a4_bf16(U16, 1, 32768, 32768, 128, I8, F, F, 8, I8, F, U16, 8, nullptr),
            CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_linear_w4a4_bf16(U16, BIG, 256, 256, 128, I8, F, F, 8, I8, F, U16, 8, nullptr));
    REJECTED(ck4_linear_w4a4_bf16(U16, 1, 256, BIG, 128, I8, F, F, 8, I8, F, U16, 8, nullptr));
    REJECTED(ck4_linear_w4a4_bf16(U16, 1, 256, 256, 128, I8, F, F, NEG, I8, F, U16, 8, nullptr));
    // the grouped W4A8 layer from bf16: one launch for m = 1 (128-blocks, groups >= 32), else the
    // quantiser and the W4A8 linear (fused for m <= 64: two launches)
    VALID(ck4_linear_w4a8_grouped_bf16(U16, 1, 3072, 3072, 128, I8, F, 0, 5120, 128, I8, F, U16, 5120, nullptr, 0,
                                       nullptr), 1);
    VALID(ck4_linear_w4a8_grouped_bf16(U16, 1, 3072, 3072, 128, I8, F, 0, 12288, 128, I8, F, U16, 12288, nullptr, 0,
                                       nullptr), 2);
    VALID(ck4_linear_w4a8_grouped_bf16(U16, 1, 384, 392, 128, I8, F, 1, 5, 128, I8, F, U16, 8, nullptr, 0, nullptr),
          1);
    VALID(ck4_linear_w4a8_grouped_bf16(U16, 2, 384, 392, 128, I8, F, 1, 5, 128, I8, F, U16, 8, nullptr, 0, nullptr),
          2);
    VALID(ck4_linear_w4a8_grouped_bf16(U16, 4, 384, 392, 128, I8, F, 0, 5, 128, I8, F, U16, 8, nullptr, 0, nullptr),
          2);
    VALID(ck4_linear_w4a8_grouped_bf16(U16, 1, 384, 384, 128, I8, F, 0, 5, 16, I8, F, U16, 8, nullptr, 0, nullptr),
          2);
    REFUSED(ck4_linear_w4a8_grouped_bf16(nullptr, 1, 256, 256, 128, I8, F, 0, 8, 128, I8, F, U16, 8, nullptr, 0,
                                         nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a8_grouped_bf16(U16, 1, 256, 256, 128, I8, F, 0, 8, 128, (int8_t *)ODD, F, U16, 8, nullptr,
                                         0, nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a8_grouped_bf16(U16, 1, 256, 200, 128, I8, F, 0, 8, 128, I8, F, U16, 8, nullptr, 0,
                                         nullptr), CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a8_grouped_bf16(U16, 1, 256, 256, 128, I8, F, 0, 8, 96, I8, F, U16, 8, nullptr, 0,
                                         nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_linear_w4a8_grouped_bf16(U16, 1, 128, 128, 128, I8, F, 0, 8, 128, I8, F, U16, 8, nullptr, 0,
                                         nullptr), CK4_ERR_UNSUPPORTED);
    REFUSED(ck4_linear_w4a8_grouped_bf16(U16, 1, 32768, 32768, 128, I8, F, 0, 8, 128, I8, F, U16, 8, nullptr, 0,
                                         nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_linear_w4a8_grouped_bf16(U16, BIG, 256, 256, 128, I8, F, 0, 8, 128, I8, F, U16, 8, nullptr, 0,
                                          nullptr));
    REJECTED(ck4_linear_w4a8_grouped_bf16(U16, 1, 256, 256, 128, I8, F, 0, NEG, 128, I8, F, U16, 8, nullptr, 0,
                                          nullptr));
    REJECTED(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, BIG, 256, U16, BIG, nullptr));
    REJECTED(ck4_linear_w4a4(I8, F, I8, F, nullptr, 8, 8, BIG, U16, 8, nullptr));
    REJECTED(ck4_linear_w4a4(I8, F, I8, F, nullptr, NEG, NEG, NEG, U16, NEG, nullptr));
    VALID(ck4_gemm_w4a4_acc_i32(I8, I8, 8, 8, 256, I32, 8, nullptr), 1);
    REFUSED(ck4_gemm_w4a4_acc_i32(I8, I8, 8, 8, 256, (int32_t *)(g_buf + 8), 8, nullptr), CK4_ERR_INVALID);
    VALID(ck4_linear_w8a8(I8, F, I8, F, nullptr, 8, 8, 128, U16, 8, nullptr), 1);
    REFUSED(ck4_linear_w8a8(I8, F, I8, F, nullptr, 8, 8, 64, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);

    // ---- the FP6 operand path
    if (ck4_fp6_bytes(17, 256) != 32 * 2 * 96 || ck4_fp6_bytes(16, 200) != 0 || ck4_fp6_bytes(0, 128) != 0 ||
        ck4_fp6_bytes(BIG, 128) != 0 || ck4_fp6_bytes(16, BIG) != 0 || ck4_fp6_bytes(NEG, NEG) != 0) {
        std::fprintf(stderr, "ck4_fp6_bytes edge values wrong\n");
        ++g_fails;
    }
    VALID(ck4_rotate_quantize_act_fp6(U16, 8, 256, 256, 128, U8, F, nullptr), 1);
    REFUSED(ck4_rotate_quantize_act_fp6(U16, 8, 192, 192, 64, U8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_rotate_quantize_act_fp6(U16, BIG, 256, BIG, 128, U8, F, nullptr));
    VALID(ck4_quantize_weight_convrot_fp6(F, 8, 256, 256, 128, U8, F, nullptr), 1);
    VALID(ck4_linear_w4a4_fp6(U8, F, U8, F, nullptr, 8, 8, 128, U16, 8, nullptr), 1);
    REFUSED(ck4_linear_w4a4_fp6(U8, F, U8, F, nullptr, 8, 8, 192, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_linear_w4a4_fp6(U8, F, U8, F, nullptr, BIG, BIG, BIG, U16, BIG, nullptr));
    VALID(ck4_gemm_w4a4_fp6_acc_i32(U8, U8, 8, 8, 128, I32, 8, nullptr), 1);
    if (ck4_fp6c_bytes(17, 256) != 32 * 2 * 64 || ck4_fp6c_bytes(16, 200) != 0 || ck4_fp6c_bytes(0, 128) != 0 ||
        ck4_fp6c_bytes(BIG, 128) != 0 || ck4_fp6c_bytes(16, BIG) != 0 || ck4_fp6c_bytes(NEG, NEG) != 0) {
        std::fprintf(stderr, "ck4_fp6c_bytes edge values wrong\n");
        ++g_fails;
    }
    VALID(ck4_rotate_quantize_act_fp6c(U16, 8, 256, 256, 128, U8, F, nullptr), 1);
    REFUSED(ck4_rotate_quantize_act_fp6c(U16, 8, 192, 192, 64, U8, F, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_rotate_quantize_act_fp6c(U16, BIG, 256, BIG, 128, U8, F, nullptr));
    VALID(ck4_quantize_weight_convrot_fp6c(F, 8, 256, 256, 128, U8, F, nullptr), 1);
    VALID(ck4_linear_w4a4_fp6c(U8, F, U8, F, nullptr, 8, 8, 128, U16, 8, nullptr), 1);
    REFUSED(ck4_linear_w4a4_fp6c(U8, F, U8, F, nullptr, 8, 8, 192, U16, 8, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_linear_w4a4_fp6c(U8, F, U8, F, nullptr, BIG, BIG, BIG, U16, BIG, nullptr));
    VALID(ck4_gemm_w4a4_fp6c_acc_i32(U8, U8, 8, 8, 128, I32, 8, nullptr), 1);
    int tm = 0, tn = 0;
    if (ck4_gemm_fp6_tile(4608, 3072, 3072, &tm, &tn) != CK4_OK || tm != 288 || tn != 192 ||
        ck4_gemm_fp6_tile(16, 8, 128, &tm, &tn) != CK4_OK || tm != 96 || tn != 128) {
        std::fprintf(stderr, "ck4_gemm_fp6_tile wrong\n");
        ++g_fails;
    }
    REJECTED(ck4_gemm_fp6_tile(BIG, BIG, 128, &tm, &tn));
    REJECTED(ck4_gemm_fp6_tile(8, 8, BIG, &tm, &tn));
    REJECTED(ck4_gemm_fp6_tile(8, 8, 128, nullptr, &tn));

    // ---- grouped W4A8: decode and linear (fused, chunked, single pass)
    VALID(ck4_dequant_w4a8_grouped(I8, F, 64, 256, 128, 0, 64, I8, F, nullptr), 1);
    VALID(ck4_dequant_w4a8_grouped(I8, F, 64, 256, 4, 16, 48, I8, F, nullptr), 1);
    REFUSED(ck4_dequant_w4a8_grouped(I8, F, 64, 256, 128, 16, 64, I8, F, nullptr), CK4_ERR_INVALID);
    REJECTED(ck4_dequant_w4a8_grouped(I8, F, 64, 256, 128, BIG, 64, I8, F, nullptr));
    REJECTED(ck4_dequant_w4a8_grouped(I8, F, 64, 256, 128, 1, BIG, I8, F, nullptr));
    REJECTED(ck4_dequant_w4a8_grouped(I8, F, BIG, BIG, 128, 0, BIG, I8, F, nullptr));
    REJECTED(ck4_dequant_w4a8_grouped(I8, F, 64, 256, 128, NEG, 64, I8, F, nullptr));
    VALID(ck4_dequant_w4a8_grouped_e4m3(I8, U8, 64, 256, 64, 0, 64, I8, F, nullptr), 1);
    VALID(ck4_dequant_w4a8_codebook(I8, U8, 1, cb, 64, 256, 64, 0, 64, I8, F, nullptr), 1);
    REFUSED(ck4_dequant_w4a8_codebook(I8, U8, 1, cb_nan, 64, 256, 64, 0, 64, I8, F, nullptr), CK4_ERR_INVALID);
    const size_t ws = ck4_w4a8_workspace_bytes(8, 1000, 1024, 256);
    if (ws < (size_t)256 * 1024 || ck4_w4a8_workspace_bytes(8, 1000, 1024, 0) != 0 ||
        ck4_w4a8_workspace_bytes(BIG, BIG, BIG, -1) != 0 || ck4_w4a8_workspace_bytes(8, BIG, BIG, BIG) != 0 ||
        ck4_w4a8_workspace_bytes(NEG, 8, 8, NEG) != 0) {
        std::fprintf(stderr, "ck4_w4a8_workspace_bytes edge values wrong\n");
        ++g_fails;
    }
    VALID(ck4_linear_w4a8_grouped(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, 0, nullptr, 0, nullptr), 1);
    VALID(ck4_linear_w4a8_grouped(I8, F, I8, F, 1, 1000, 1024, 128, U16, 1008, 0, nullptr, 0, nullptr), 1);
    VALID(ck4_linear_w4a8_grouped(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, 256, P, ws, nullptr), 8);
    VALID(ck4_linear_w4a8_grouped(I8, F, I8, F, 100, 1000, 1024, 128, U16, 1008, 0, P, BIG, nullptr), 2);
    REFUSED(ck4_linear_w4a8_grouped(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, 256, P, 100, nullptr),
            g_mode == 1 ? CK4_ERR_INVALID : CK4_ERR_DEVICE);
    REFUSED(ck4_linear_w4a8_grouped(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, 250, P, ws, nullptr),
            CK4_ERR_INVALID);
    REFUSED(ck4_linear_w4a8_grouped(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, 256, nullptr, 0, nullptr),
            CK4_ERR_INVALID);
    REJECTED(ck4_linear_w4a8_grouped(I8, F, I8, F, 8, BIG, 1024, 128, U16, BIG, -1, P, BIG, nullptr));
    REJECTED(ck4_linear_w4a8_grouped(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, BIG, P, BIG, nullptr));
    VALID(ck4_linear_w4a8_grouped_e4m3(I8, F, I8, U8, 8, 1000, 1024, 64, U16, 1008, 0, nullptr, 0, nullptr), 1);
    VALID(ck4_linear_w4a8_codebook(I8, F, I8, F, 0, cb, 8, 1000, 1024, 64, U16, 1008, 0, nullptr, 0, nullptr), 1);
    VALID(ck4_linear_w4a8_grouped_noalloc(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, 256, nullptr), 8);
    VALID(ck4_linear_w4a8_grouped_noalloc(I8, F, I8, F, 8, 1000, 1024, 128, U16, 1008, 0, nullptr), 1);
    REFUSED(ck4_linear_w4a8_grouped_noalloc(I8, F, I8, F, 8, 12288, 8192, 128, U16, 12288, -1, nullptr),
            CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_linear_w4a8_grouped_noalloc(I8, F, I8, F, 8, BIG, BIG, 128, U16, BIG, -1, nullptr));
    REJECTED(ck4_linear_w4a8_grouped_noalloc(I8, F, I8, F, NEG, 8, 1024, 128, U16, 8, 0, nullptr));

    // ---- dynamic LoRA
    VALID(ck4_lora_prepare_down(F, 32, 256, 256, 128, U16, nullptr), 1);
    REFUSED(ck4_lora_prepare_down(F, 48, 256, 256, 128, U16, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_lora_prepare_down(F, 32, 256, BIG, 128, U16, nullptr));
    VALID(ck4_lora_prepare_up(U16, 100, 64, 64, U16, nullptr), 1);
    REJECTED(ck4_lora_prepare_up(U16, BIG, 64, BIG, U16, nullptr));
    REJECTED(ck4_lora_prepare_up(U16, 100, 64, NEG, U16, nullptr));
    VALID(ck4_lora_down(U16, 100, 1024, 1024, 128, U16, 64, 0.5f, U16, nullptr), 1);
    REFUSED(ck4_lora_down(U16, 100, 1024, 1024, 512, U16, 64, 0.5f, U16, nullptr), CK4_ERR_UNSUPPORTED);
    REJECTED(ck4_lora_down(U16, BIG, 1024, BIG, 128, U16, 64, 0.5f, U16, nullptr));
    VALID(ck4_linear_w4a4_lora(I8, F, I8, F, nullptr, U16, U16, 128, 100, 200, 1024, U16, 200, nullptr), 1);
    REFUSED(ck4_linear_w4a4_lora(I8, F, I8, F, nullptr, U16, U16, 100, 100, 200, 1024, U16, 200, nullptr),
            CK4_ERR_UNSUPPORTED);
    VALID(ck4_linear_w4a4_fp6_lora(U8, F, U8, F, nullptr, U16, U16, 32, 100, 200, 1024, U16, 200, nullptr), 1);
    VALID(ck4_linear_w4a4_fp6c_lora(U8, F, U8, F, nullptr, U16, U16, 32, 100, 200, 1024, U16, 200, nullptr), 1);

    std::printf("%s: %d calls checked, %d failures\n", mode.c_str(), g_checked, g_fails);
    return g_fails == 0 ? 0 : 1;
}
