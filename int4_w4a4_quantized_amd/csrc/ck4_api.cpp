// C ABI of the ck4 library: argument validation, launch selection, errors.
// Every entry point validates everything before it touches the device, so a
// rejected call launches nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/ck4.h"
#include "ck4_kernels.h"
#include "gemv.h"

#define CK4_VERSION_STRING "ck4 0.1.0 gfx950"

static_assert(CK4_NOALLOC_SCRATCH_BYTES == ck4::kNoallocScratchBytes, "ck4.h and the kernels disagree");

namespace {

thread_local std::string g_last_error;

ck4_status fail(ck4_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

ck4_status ok() {
    g_last_error.clear();
    return CK4_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// A host codebook of 16 fp32 entries -> the kernels' by-value copy.
ck4_status make_codebook(const char *fn, const float *codebook, ck4::Codebook *cb) {
    if (!codebook) return fail(CK4_ERR_INVALID, "%s: null codebook", fn);
    float cmax = 0.0f;
    for (int u = 0; u < 16; ++u) {
        if (!std::isfinite(codebook[u])) return fail(CK4_ERR_INVALID, "%s: codebook[%d] is not finite", fn, u);
        cb->v[u] = codebook[u];
        cmax = std::fabs(codebook[u]) > cmax ? std::fabs(codebook[u]) : cmax;
    }
    if (!(cmax >= 0x1p-64f && cmax <= 0x1p64f))
        return fail(CK4_ERR_INVALID, "%s: max |codebook| = %g is outside [2^-64, 2^64]", fn, (double)cmax);
    cb->cmax = cmax;
    cb->on = true;
    return CK4_OK;
}

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];
int64_t g_l2_bytes[kMaxDevices];

// The kernels are built for gfx950 only; refuse any other device.
ck4_status check_device(const char *fn, int *dev_out = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(CK4_ERR_DEVICE, "%s: no current HIP device", fn);
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            g_dev_ok[dev] = 0;
            return;
        }
        g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
        g_l2_bytes[dev] = prop.l2CacheSize;
    });
    if (!g_dev_ok[dev]) return fail(CK4_ERR_DEVICE, "%s: current device is not gfx950", fn);
    if (dev_out) *dev_out = dev;
    return CK4_OK;
}

ck4_status launched(const char *fn, hipError_t e) {
    if (e != hipSuccess) return fail(CK4_ERR_DEVICE, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

constexpr int64_t kMaxActK = 16384;     // rotate/quantise kernels hold a row in VGPRs
constexpr int64_t kMaxGemmK = 131072;   // 256 * 49 * K < 2^31 for the widened int4 products
constexpr int64_t kMaxRows = 0x7FFFFFFF;
constexpr int64_t kMaxStride = int64_t(1) << 40;  // elements; row * stride stays far inside int64

// A row stride in elements that is at least `width`, a multiple of `mult`
// (so rows stay aligned) and not absurdly large; checked without forming any
// product of caller values.
ck4_status check_stride(const char *fn, const char *name, int64_t ld, int64_t width, int64_t mult) {
    if (ld < width) return fail(CK4_ERR_INVALID, "%s: %s=%lld < %lld", fn, name, (long long)ld, (long long)width);
    if (ld % mult != 0)
        return fail(CK4_ERR_INVALID, "%s: %s=%lld is not a multiple of %lld", fn, name, (long long)ld, (long long)mult);
    if (ld > kMaxStride) return fail(CK4_ERR_UNSUPPORTED, "%s: %s=%lld too large", fn, name, (long long)ld);
    return CK4_OK;
}

ck4_status check_rot(const char *fn, int64_t k, int rot_block) {
    if (!pow2(rot_block) || rot_block < 16 || rot_block > 1024)
        return fail(CK4_ERR_UNSUPPORTED, "%s: rot_block=%d (need a power of two in [16, 1024])", fn, rot_block);
    if (k % rot_block != 0)
        return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of rot_block=%d", fn, (long long)k,
                    rot_block);
    if (k > kMaxActK) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld > %lld", fn, (long long)k, (long long)kMaxActK);
    return CK4_OK;
}

ck4_status check_gemm_common(const char *fn, int64_t m, int64_t n, int64_t k, int64_t ldy, const void *y,
                             size_t y_align) {
    if (m <= 0 || n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: m, n, k must be positive", fn);
    if (m > kMaxRows || n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: m or n too large", fn);
    if (ck4_status s = check_stride(fn, "ldy", ldy, n, 4)) return s;
    if (!aligned(y, y_align)) return fail(CK4_ERR_INVALID, "%s: output pointer not %zu-byte aligned", fn, y_align);
    if (k > kMaxGemmK) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld > %lld", fn, (long long)k, (long long)kMaxGemmK);
    return CK4_OK;
}

}  // namespace

extern "C" {

const char *ck4_version(void) { return CK4_VERSION_STRING; }

const char *ck4_status_string(ck4_status s) {
    switch (s) {
    case CK4_OK: return "ok";
    case CK4_ERR_INVALID: return "invalid argument";
    case CK4_ERR_UNSUPPORTED: return "unsupported shape or option";
    case CK4_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char *ck4_last_error(void) { return g_last_error.c_str(); }

ck4_status ck4_quantize_weight_convrot(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block, int group,
                                       int8_t *w_packed, float *w_scales, void *stream) {
    const char *fn = "ck4_quantize_weight_convrot";
    if (!w || !w_packed || !w_scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: n and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldw", ldw, k, 4)) return s;
    if (!aligned(w, 16)) return fail(CK4_ERR_INVALID, "%s: w not 16-byte aligned", fn);
    if (!aligned(w_packed, 8) || !aligned(w_scales, 4)) return fail(CK4_ERR_INVALID, "%s: outputs misaligned", fn);
    if (n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: n too large", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (group != 0 && (!pow2(group) || group < 4 || group > 1024 || k % group != 0))
        return fail(CK4_ERR_UNSUPPORTED, "%s: group=%d (need 0 or a power of two in [4, 1024] dividing k)", fn,
                    group);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(w, 1, n, k, ldw, rot_block, 0, group, w_packed, k / 2, w_scales,
                                                  static_cast<hipStream_t>(stream)));
}

ck4_status ck4_quantize_weight_convrot_sr(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                          int group, const float *u, int64_t ldu, int8_t *w_packed, float *w_scales,
                                          void *stream) {
    const char *fn = "ck4_quantize_weight_convrot_sr";
    if (!w || !u || !w_packed || !w_scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: n and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldw", ldw, k, 4)) return s;
    if (ck4_status s = check_stride(fn, "ldu", ldu, k, 4)) return s;
    if (!aligned(w, 16) || !aligned(u, 16)) return fail(CK4_ERR_INVALID, "%s: w or u not 16-byte aligned", fn);
    if (!aligned(w_packed, 8) || !aligned(w_scales, 4)) return fail(CK4_ERR_INVALID, "%s: outputs misaligned", fn);
    if (n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: n too large", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (group != 0 && (!pow2(group) || group < 4 || group > 1024 || k % group != 0))
        return fail(CK4_ERR_UNSUPPORTED, "%s: group=%d (need 0 or a power of two in [4, 1024] dividing k)", fn,
                    group);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(w, 1, n, k, ldw, rot_block, 0, group, w_packed, k / 2, w_scales,
                                                  static_cast<hipStream_t>(stream), ck4::WeightOpts{u, ldu, false}));
}

ck4_status ck4_quantize_weight_convrot_e4m3(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                            int group, int8_t *w_packed, uint8_t *group_scales, void *stream) {
    const char *fn = "ck4_quantize_weight_convrot_e4m3";
    if (!w || !w_packed || !group_scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: n and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldw", ldw, k, 4)) return s;
    if (!aligned(w, 16)) return fail(CK4_ERR_INVALID, "%s: w not 16-byte aligned", fn);
    if (!aligned(w_packed, 8)) return fail(CK4_ERR_INVALID, "%s: w_packed misaligned", fn);
    if (n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: n too large", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (!pow2(group) || group < 4 || group > 1024 || k % group != 0)
        return fail(CK4_ERR_UNSUPPORTED, "%s: group=%d (need a power of two in [4, 1024] dividing k)", fn, group);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(w, 1, n, k, ldw, rot_block, 0, group, w_packed, k / 2,
                                                  reinterpret_cast<float *>(group_scales),
                                                  static_cast<hipStream_t>(stream), ck4::WeightOpts{nullptr, 0, true}));
}

ck4_status ck4_quantize_weight_convrot_codebook(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                                int group, const float *codebook, int scale_e4m3, int8_t *w_packed,
                                                void *group_scales, void *stream) {
    const char *fn = "ck4_quantize_weight_convrot_codebook";
    if (!w || !w_packed || !group_scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    ck4::WeightOpts wo{nullptr, 0, scale_e4m3 != 0};
    if (ck4_status s = make_codebook(fn, codebook, &wo.cb)) return s;
    if (n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: n and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldw", ldw, k, 4)) return s;
    if (!aligned(w, 16)) return fail(CK4_ERR_INVALID, "%s: w not 16-byte aligned", fn);
    if (!aligned(w_packed, 8) || (!scale_e4m3 && !aligned(group_scales, 4)))
        return fail(CK4_ERR_INVALID, "%s: outputs misaligned", fn);
    if (n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: n too large", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (!pow2(group) || group < 4 || group > 1024 || k % group != 0)
        return fail(CK4_ERR_UNSUPPORTED, "%s: group=%d (need a power of two in [4, 1024] dividing k)", fn, group);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(w, 1, n, k, ldw, rot_block, 0, group, w_packed, k / 2,
                                                  static_cast<float *>(group_scales),
                                                  static_cast<hipStream_t>(stream), wo));
}

ck4_status ck4_quantize_weight_convrot_int8(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                            int8_t *w_q8, float *w_scales, void *stream) {
    const char *fn = "ck4_quantize_weight_convrot_int8";
    if (!w || !w_q8 || !w_scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: n and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldw", ldw, k, 4)) return s;
    if (!aligned(w, 16)) return fail(CK4_ERR_INVALID, "%s: w not 16-byte aligned", fn);
    if (!aligned(w_q8, 16) || !aligned(w_scales, 4)) return fail(CK4_ERR_INVALID, "%s: outputs misaligned", fn);
    if (n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: n too large", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(w, 1, n, k, ldw, rot_block, 1, 0, w_q8, k, w_scales,
                                                  static_cast<hipStream_t>(stream)));
}

ck4_status ck4_rotate_quantize_act(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, int bits,
                                   int8_t *x_q, float *x_scales, void *stream) {
    const char *fn = "ck4_rotate_quantize_act";
    if (!x || !x_q || !x_scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (m <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: m and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldx", ldx, k, 8)) return s;
    if (bits != 4 && bits != 8) return fail(CK4_ERR_UNSUPPORTED, "%s: bits=%d (need 4 or 8)", fn, bits);
    if (!aligned(x, 16)) return fail(CK4_ERR_INVALID, "%s: x not 16-byte aligned", fn);
    if (!aligned(x_q, bits == 4 ? 8 : 16) || !aligned(x_scales, 4))
        return fail(CK4_ERR_INVALID, "%s: outputs misaligned", fn);
    if (m > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: m too large", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(x, 0, m, k, ldx, rot_block, bits == 4 ? 0 : 1, 0, x_q,
                                                  bits == 4 ? k / 2 : k, x_scales, static_cast<hipStream_t>(stream)));
}

ck4_status ck4_rotate_act_f32(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, float *r,
                              void *stream) {
    const char *fn = "ck4_rotate_act_f32";
    if (!x || !r) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (m <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: m and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldx", ldx, k, 8)) return s;
    if (!aligned(x, 16)) return fail(CK4_ERR_INVALID, "%s: x not 16-byte aligned", fn);
    if (!aligned(r, 16)) return fail(CK4_ERR_INVALID, "%s: r not 16-byte aligned", fn);
    if (m > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: m too large", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(x, 0, m, k, ldx, rot_block, 2, 0, r, k, nullptr,
                                                  static_cast<hipStream_t>(stream)));
}

static ck4_status gemm_entry(const char *fn, bool s4, const int8_t *a, const float *sa, const int8_t *b,
                             const float *sb, const float *bias, int64_t m, int64_t n, int64_t k, bool out_i32,
                             void *y, int64_t ldy, void *stream, ck4::LoraUp lora = ck4::LoraUp{}) {
    if (!a || !b || !y || (!out_i32 && (!sa || !sb))) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (ck4_status s = check_gemm_common(fn, m, n, k, ldy, y, out_i32 ? 16 : 8)) return s;
    if (!aligned(a, 16) || !aligned(b, 16)) return fail(CK4_ERR_INVALID, "%s: operands not 16-byte aligned", fn);
    if (k % 128 != 0) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of 128", fn, (long long)k);
    // packed int4 rows are walked in 128-byte windows, which a row of k = 128
    // (64 bytes) cannot hold
    if (s4 && k < 256) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld < 256 for packed int4", fn, (long long)k);
    if (ck4_status s = check_device(fn)) return s;
    // one or two activation rows: the matrix-vector kernel (same bits)
    if (s4 && !out_i32 && (lora.t == nullptr || lora.rank == 0) && ck4::gemv_w4a4_fits(m, k))
        return launched(fn, ck4::launch_gemv_w4a4(a, sa, b, sb, bias, m, n, k, static_cast<uint16_t *>(y), ldy,
                                                  static_cast<hipStream_t>(stream)));
    return launched(fn, ck4::launch_gemm(s4, a, b, sa, sb, bias, m, n, k, out_i32, y, ldy,
                                         static_cast<hipStream_t>(stream), lora));
}

ck4_status ck4_linear_w4a4(const int8_t *x_q, const float *x_scales, const int8_t *w_packed, const float *w_scales,
                           const float *bias, int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy,
                           void *stream) {
    return gemm_entry("ck4_linear_w4a4", true, x_q, x_scales, w_packed, w_scales, bias, m, n, k, false, y, ldy,
                      stream);
}

ck4_status ck4_linear_w4a4_bf16(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                const int8_t *w_packed, const float *w_scales, const float *bias, int64_t n,
                                int8_t *x_q, float *x_scales, uint16_t *y, int64_t ldy, void *stream) {
    const char *fn = "ck4_linear_w4a4_bf16";
    if (!x || !w_packed || !w_scales || !x_q || !x_scales || !y) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (ck4_status s = check_gemm_common(fn, m, n, k, ldy, y, 8)) return s;
    if (ck4_status s = check_stride(fn, "ldx", ldx, k, 8)) return s;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(x_q, 16) || !aligned(x_scales, 4))
        return fail(CK4_ERR_INVALID, "%s: x, w_packed or x_q not 16-byte aligned, or x_scales misaligned", fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (k % 128 != 0 || k < 256)
        return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld (need a multiple of 128, at least 256)", fn, (long long)k);
    if (ck4_status s = check_device(fn)) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (ck4::skinny_layer_fits(m, n, k, rot_block))
        return launched(fn, ck4::launch_skinny_layer(x, ldx, w_packed, w_scales, bias, m, n, k, x_q, x_scales, y, ldy,
                                                     st));
    if (ck4_status s = launched(fn, ck4::launch_rotate_quant(x, 0, m, k, ldx, rot_block, 0, 0, x_q, k / 2, x_scales,
                                                             st)))
        return s;
    return launched(fn, ck4::launch_gemm(true, x_q, w_packed, x_scales, w_scales, bias, m, n, k, false, y, ldy, st,
                                         ck4::LoraUp{}));
}

ck4_status ck4_gemm_w4a4_acc_i32(const int8_t *x_q, const int8_t *w_packed, int64_t m, int64_t n, int64_t k,
                                 int32_t *acc, int64_t ldacc, void *stream) {
    return gemm_entry("ck4_gemm_w4a4_acc_i32", true, x_q, nullptr, w_packed, nullptr, nullptr, m, n, k, true, acc,
                      ldacc, stream);
}

ck4_status ck4_linear_w8a8(const int8_t *x_q8, const float *x_scales, const int8_t *w8, const float *w_scales,
                           const float *bias, int64_t m, int64_t n, int64_t k, uint16_t *y, int64_t ldy,
                           void *stream) {
    return gemm_entry("ck4_linear_w8a8", false, x_q8, x_scales, w8, w_scales, bias, m, n, k, false, y, ldy,
                      stream);
}

size_t ck4_fp6_bytes(int64_t rows, int64_t k) {
    if (rows <= 0 || rows > kMaxRows || k <= 0 || k > kMaxGemmK || k % 128 != 0) return 0;
    return (size_t)((rows + 15) / 16 * 16) * (size_t)(k / 128) * 96;
}

size_t ck4_fp6c_bytes(int64_t rows, int64_t k) {
    if (rows <= 0 || rows > kMaxRows || k <= 0 || k > kMaxGemmK || k % 128 != 0) return 0;
    return (size_t)((rows + 15) / 16 * 16) * (size_t)(k / 128) * 64;
}

static ck4_status quantize_fp6(const char *fn, const void *x, int in_kind, int64_t rows, int64_t k, int64_t ldx,
                               int rot_block, uint8_t *q6, float *scales, void *stream, int out_kind = 4) {
    const size_t esz = in_kind == 0 ? 2 : 4;
    if (!x || !q6 || !scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (rows <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: rows and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldx", ldx, k, (int64_t)(16 / esz))) return s;
    if (!aligned(x, 16)) return fail(CK4_ERR_INVALID, "%s: input not 16-byte aligned", fn);
    if (!aligned(q6, 16) || !aligned(scales, 4)) return fail(CK4_ERR_INVALID, "%s: outputs misaligned", fn);
    if (rows > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: too many rows", fn);
    if (k % 128 != 0) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of 128", fn, (long long)k);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(x, in_kind, rows, k, ldx, rot_block, out_kind, 0, q6, 0, scales,
                                                  static_cast<hipStream_t>(stream)));
}

ck4_status ck4_rotate_quantize_act_fp6(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                       uint8_t *x_q6, float *x_scales, void *stream) {
    return quantize_fp6("ck4_rotate_quantize_act_fp6", x, 0, m, k, ldx, rot_block, x_q6, x_scales, stream);
}

ck4_status ck4_quantize_weight_convrot_fp6(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                           uint8_t *w_q6, float *w_scales, void *stream) {
    return quantize_fp6("ck4_quantize_weight_convrot_fp6", w, 1, n, k, ldw, rot_block, w_q6, w_scales, stream);
}

ck4_status ck4_rotate_quantize_act_fp6c(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                        uint8_t *x_q6c, float *x_scales, void *stream) {
    return quantize_fp6("ck4_rotate_quantize_act_fp6c", x, 0, m, k, ldx, rot_block, x_q6c, x_scales, stream, 5);
}

ck4_status ck4_quantize_weight_convrot_fp6c(const float *w, int64_t n, int64_t k, int64_t ldw, int rot_block,
                                            uint8_t *w_q6c, float *w_scales, void *stream) {
    return quantize_fp6("ck4_quantize_weight_convrot_fp6c", w, 1, n, k, ldw, rot_block, w_q6c, w_scales, stream, 5);
}

static ck4_status gemm_fp6_entry(const char *fn, const uint8_t *a, const float *sa, const uint8_t *b,
                                 const float *sb, const float *bias, int64_t m, int64_t n, int64_t k, bool out_i32,
                                 void *y, int64_t ldy, void *stream, ck4::LoraUp lora = ck4::LoraUp{},
                                 bool compact = false) {
    if (!a || !b || !y || (!out_i32 && (!sa || !sb))) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (ck4_status s = check_gemm_common(fn, m, n, k, ldy, y, out_i32 ? 16 : 8)) return s;
    if (!aligned(a, 16) || !aligned(b, 16)) return fail(CK4_ERR_INVALID, "%s: operands not 16-byte aligned", fn);
    if (k % 128 != 0) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of 128", fn, (long long)k);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_gemm_fp6(a, b, sa, sb, bias, m, n, k, out_i32, y, ldy,
                                             static_cast<hipStream_t>(stream), lora, compact));
}

ck4_status ck4_linear_w4a4_fp6(const uint8_t *x_q6, const float *x_scales, const uint8_t *w_q6,
                               const float *w_scales, const float *bias, int64_t m, int64_t n, int64_t k,
                               uint16_t *y, int64_t ldy, void *stream) {
    return gemm_fp6_entry("ck4_linear_w4a4_fp6", x_q6, x_scales, w_q6, w_scales, bias, m, n, k, false, y, ldy,
                          stream);
}

ck4_status ck4_gemm_w4a4_fp6_acc_i32(const uint8_t *x_q6, const uint8_t *w_q6, int64_t m, int64_t n, int64_t k,
                                     int32_t *acc, int64_t ldacc, void *stream) {
    return gemm_fp6_entry("ck4_gemm_w4a4_fp6_acc_i32", x_q6, nullptr, w_q6, nullptr, nullptr, m, n, k, true, acc,
                          ldacc, stream);
}

ck4_status ck4_linear_w4a4_fp6c(const uint8_t *x_q6c, const float *x_scales, const uint8_t *w_q6c,
                                const float *w_scales, const float *bias, int64_t m, int64_t n, int64_t k,
                                uint16_t *y, int64_t ldy, void *stream) {
    return gemm_fp6_entry("ck4_linear_w4a4_fp6c", x_q6c, x_scales, w_q6c, w_scales, bias, m, n, k, false, y, ldy,
                          stream, ck4::LoraUp{}, true);
}

ck4_status ck4_gemm_w4a4_fp6c_acc_i32(const uint8_t *x_q6c, const uint8_t *w_q6c, int64_t m, int64_t n, int64_t k,
                                      int32_t *acc, int64_t ldacc, void *stream) {
    return gemm_fp6_entry("ck4_gemm_w4a4_fp6c_acc_i32", x_q6c, nullptr, w_q6c, nullptr, nullptr, m, n, k, true, acc,
                          ldacc, stream, ck4::LoraUp{}, true);
}

ck4_status ck4_gemm_fp6_tile(int64_t m, int64_t n, int64_t k, int *tile_m, int *tile_n) {
    const char *fn = "ck4_gemm_fp6_tile";
    if (!tile_m || !tile_n) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (m <= 0 || n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: m, n, k must be positive", fn);
    if (m > kMaxRows || n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: m or n too large", fn);
    if (k % 128 != 0) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of 128", fn, (long long)k);
    if (k > kMaxGemmK) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld > %lld", fn, (long long)k, (long long)kMaxGemmK);
    const bool large = ck4::gemm_fp6_large_tile(m, n);
    *tile_m = large ? 288 : 96;
    *tile_n = large ? 192 : 128;
    return ok();
}

}  // extern "C"

namespace {

ck4_status dequant_w4a8(const char *fn, const int8_t *w_packed, const void *group_scales, bool e4m3, int64_t n,
                        int64_t k, int group, int64_t n0, int64_t nc, int8_t *w8, float *row_scales, void *stream,
                        const ck4::Codebook &cb = ck4::Codebook{}) {
    if (!w_packed || !group_scales || !w8 || !row_scales) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (n <= 0 || k <= 0 || nc <= 0) return fail(CK4_ERR_INVALID, "%s: n, k, nc must be positive", fn);
    if (n0 < 0 || n0 >= n || nc > n - n0) return fail(CK4_ERR_INVALID, "%s: rows [n0, n0+nc) outside [0, n)", fn);
    if (n > kMaxRows || k > kMaxGemmK) return fail(CK4_ERR_UNSUPPORTED, "%s: n or k too large", fn);
    if (!pow2(group) || group < 4 || group > 1024 || k % group != 0)
        return fail(CK4_ERR_UNSUPPORTED, "%s: group=%d (need a power of two in [4, 1024] dividing k)", fn, group);
    if (!aligned(w_packed, 16) || !aligned(w8, 16) || (k / 2) % 8 != 0)
        return fail(CK4_ERR_INVALID, "%s: w_packed / w8 not 16-byte aligned", fn);
    if (nc > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: nc too large", fn);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_w4a8_decode(w_packed, group_scales, e4m3, k, group, n0, nc, w8, row_scales,
                                                static_cast<hipStream_t>(stream), cb));
}

}  // namespace

extern "C" {

ck4_status ck4_dequant_w4a8_grouped(const int8_t *w_packed, const float *group_scales, int64_t n, int64_t k,
                                    int group, int64_t n0, int64_t nc, int8_t *w8, float *row_scales,
                                    void *stream) {
    return dequant_w4a8("ck4_dequant_w4a8_grouped", w_packed, group_scales, false, n, k, group, n0, nc, w8,
                        row_scales, stream);
}

ck4_status ck4_dequant_w4a8_grouped_e4m3(const int8_t *w_packed, const uint8_t *group_scales, int64_t n, int64_t k,
                                         int group, int64_t n0, int64_t nc, int8_t *w8, float *row_scales,
                                         void *stream) {
    return dequant_w4a8("ck4_dequant_w4a8_grouped_e4m3", w_packed, group_scales, true, n, k, group, n0, nc, w8,
                        row_scales, stream);
}

ck4_status ck4_dequant_w4a8_codebook(const int8_t *w_packed, const void *group_scales, int scale_e4m3,
                                     const float *codebook, int64_t n, int64_t k, int group, int64_t n0, int64_t nc,
                                     int8_t *w8, float *row_scales, void *stream) {
    const char *fn = "ck4_dequant_w4a8_codebook";
    ck4::Codebook cb;
    if (ck4_status s = make_codebook(fn, codebook, &cb)) return s;
    return dequant_w4a8(fn, w_packed, group_scales, scale_e4m3 != 0, n, k, group, n0, nc, w8, row_scales, stream,
                        cb);
}

// Column chunk of the decode + int8 GEMM path; 0 means the fused kernel.
static int64_t w4a8_chunk(int64_t m, int64_t n, int64_t k, int64_t chunk_cols, int64_t l2_bytes) {
    if (chunk_cols < 0) return n;
    if (chunk_cols > 0) return chunk_cols < n ? chunk_cols : n;
    const char *e_rows = std::getenv("CK4_W4A8_CHUNK_MAX_ROWS");
    const int64_t max_rows = e_rows ? std::atoll(e_rows) : 64;
    if (m > max_rows) return n;
    const char *e_cols = std::getenv("CK4_W4A8_CHUNK_COLS");
    int64_t c = e_cols ? std::atoll(e_cols) : 0;
    if (c <= 0) {
        // skinny rows: decode in registers inside the GEMM (no round trip)
        if (m <= 64 && k >= 256) return 0;
        c = (l2_bytes / k) / 128 * 128;
        if (c < 1024) c = 1024;
        if (c > 4096) c = 4096;
    }
    if (c >= n) return n;
    c = (c + 15) / 16 * 16;
    return c < n ? c : n;
}

static int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

size_t ck4_w4a8_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t chunk_cols) {
    if (m <= 0 || n <= 0 || k <= 0 || m > kMaxRows || n > kMaxRows || k > kMaxGemmK) return 0;
    int dev = 0;
    int64_t l2 = 4 << 20;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices && check_device("ws", &dev) == CK4_OK)
        l2 = g_l2_bytes[dev];
    const int64_t c = w4a8_chunk(m, n, k, chunk_cols, l2);
    if (c == 0) return 0;
    return (size_t)(align_up(c * k, 256) + align_up(c * 4, 256));
}

}  // extern "C"

namespace {

ck4_status linear_w4a8(const char *fn, const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                       const void *group_scales, bool e4m3, int64_t m, int64_t n, int64_t k, int group, uint16_t *y,
                       int64_t ldy, int64_t chunk_cols, void *workspace, size_t ws_bytes, void *stream,
                       const ck4::Codebook &cb = ck4::Codebook{}) {
    if (!x_q8 || !x_scales || !w_packed || !group_scales || !y)
        return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (ck4_status s = check_gemm_common(fn, m, n, k, ldy, y, 8)) return s;
    if (!aligned(x_q8, 16) || !aligned(w_packed, 16) || (workspace && !aligned(workspace, 16)))
        return fail(CK4_ERR_INVALID, "%s: operands not 16-byte aligned", fn);
    if (k % 128 != 0) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of 128", fn, (long long)k);
    if (!pow2(group) || group < 4 || group > 1024 || k % group != 0)
        return fail(CK4_ERR_UNSUPPORTED, "%s: group=%d (need a power of two in [4, 1024] dividing k)", fn, group);
    if (chunk_cols > 0 && chunk_cols % 16 != 0)
        return fail(CK4_ERR_INVALID, "%s: chunk_cols=%lld is not a multiple of 16", fn, (long long)chunk_cols);
    if (chunk_cols != 0 && !workspace)
        return fail(CK4_ERR_INVALID, "%s: the decode paths (chunk_cols != 0) need a workspace", fn);
    int dev = 0;
    if (ck4_status s = check_device(fn, &dev)) return s;
    const int64_t c = w4a8_chunk(m, n, k, chunk_cols, g_l2_bytes[dev]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (c == 0 && ck4::w4a8_gemv_fits(m, n, k, group, cb.on))
        return launched(fn, ck4::launch_w4a8_gemv(x_q8, x_scales, w_packed, group_scales, e4m3, m, n, k, group, y,
                                                  ldy, st));
    if (c == 0) return launched(fn, ck4::launch_w4a8_fused(x_q8, x_scales, w_packed, group_scales, e4m3, m, n, k,
                                                           group, y, ldy, st, cb));
    const size_t need = (size_t)(align_up(c * k, 256) + align_up(c * 4, 256));
    if (!workspace || ws_bytes < need)
        return fail(CK4_ERR_INVALID, "%s: workspace %zu bytes < %zu needed", fn, workspace ? ws_bytes : 0, need);
    int8_t *w8 = static_cast<int8_t *>(workspace);
    float *srow = reinterpret_cast<float *>(static_cast<char *>(workspace) + align_up(c * k, 256));
    for (int64_t n0 = 0; n0 < n; n0 += c) {
        const int64_t nc = (n - n0) < c ? (n - n0) : c;
        hipError_t e = ck4::launch_w4a8_decode(w_packed, group_scales, e4m3, k, group, n0, nc, w8, srow, st, cb);
        if (e != hipSuccess) return launched(fn, e);
        e = ck4::launch_gemm(false, x_q8, w8, x_scales, srow, nullptr, m, nc, k, false, y + n0, ldy, st);
        if (e != hipSuccess) return launched(fn, e);
    }
    return ok();
}

}  // namespace

extern "C" {

ck4_status ck4_linear_w4a8_grouped(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                   const float *group_scales, int64_t m, int64_t n, int64_t k, int group,
                                   uint16_t *y, int64_t ldy, int64_t chunk_cols, void *workspace, size_t ws_bytes,
                                   void *stream) {
    return linear_w4a8("ck4_linear_w4a8_grouped", x_q8, x_scales, w_packed, group_scales, false, m, n, k, group, y,
                       ldy, chunk_cols, workspace, ws_bytes, stream);
}

ck4_status ck4_linear_w4a8_grouped_bf16(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block,
                                        const int8_t *w_packed, const void *group_scales, int scale_e4m3, int64_t n,
                                        int group, int8_t *x_q8, float *x_scales, uint16_t *y, int64_t ldy,
                                        void *workspace, size_t ws_bytes, void *stream) {
    const char *fn = "ck4_linear_w4a8_grouped_bf16";
    if (!x || !w_packed || !group_scales || !x_q8 || !x_scales || !y)
        return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (ck4_status s = check_gemm_common(fn, m, n, k, ldy, y, 8)) return s;
    if (ck4_status s = check_stride(fn, "ldx", ldx, k, 8)) return s;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(x_q8, 16) || !aligned(x_scales, 4) ||
        (workspace && !aligned(workspace, 16)))
        return fail(CK4_ERR_INVALID, "%s: x, w_packed, x_q8 or workspace not 16-byte aligned, or x_scales misaligned",
                    fn);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (k % 128 != 0 || k < 256)
        return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld (need a multiple of 128, at least 256)", fn, (long long)k);
    if (!pow2(group) || group < 4 || group > 1024 || k % group != 0)
        return fail(CK4_ERR_UNSUPPORTED, "%s: group=%d (need a power of two in [4, 1024] dividing k)", fn, group);
    if (ck4_status s = check_device(fn)) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (ck4::w4a8_layer_fits(m, n, k, rot_block, group, false, scale_e4m3 != 0))
        return launched(fn, ck4::launch_w4a8_layer(x, ldx, w_packed, group_scales, scale_e4m3 != 0, m, n, k, group,
                                                   x_q8, x_scales, y, ldy, st));
    if (ck4_status s = launched(fn, ck4::launch_rotate_quant(x, 0, m, k, ldx, rot_block, 1, 0, x_q8, k, x_scales, st)))
        return s;
    return linear_w4a8(fn, x_q8, x_scales, w_packed, group_scales, scale_e4m3 != 0, m, n, k, group, y, ldy, 0,
                       workspace, ws_bytes, stream);
}

ck4_status ck4_linear_w4a8_grouped_noalloc(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                           const float *group_scales, int64_t m, int64_t n, int64_t k, int group,
                                           uint16_t *y, int64_t ldy, int64_t chunk_cols, void *stream) {
    const char *fn = "ck4_linear_w4a8_grouped_noalloc";
    if (m <= 0 || n <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: m, n, k must be positive", fn);
    if (m > kMaxRows || n > kMaxRows || k > kMaxGemmK)
        return fail(CK4_ERR_UNSUPPORTED, "%s: m, n or k too large", fn);
    if (chunk_cols < 0 && (size_t)(align_up(n * k, 256) + align_up(n * 4, 256)) > ck4::kNoallocScratchBytes)
        return fail(CK4_ERR_UNSUPPORTED, "%s: the single-pass decode of n=%lld x k=%lld needs more than the %zu-byte "
                    "fixed buffer; pass a chunk width", fn, (long long)n, (long long)k, ck4::kNoallocScratchBytes);
    int dev = 0;
    if (ck4_status s = check_device(fn, &dev)) return s;
    const size_t need = ck4_w4a8_workspace_bytes(m, n, k, chunk_cols);
    if (need > ck4::kNoallocScratchBytes)
        return fail(CK4_ERR_UNSUPPORTED, "%s: the decode needs %zu bytes, more than the %zu-byte fixed buffer; pass a "
                    "smaller chunk width", fn, need, ck4::kNoallocScratchBytes);
    void *scratch = nullptr;
    if (need > 0) {
        const hipError_t e = ck4::noalloc_scratch(dev, &scratch);
        if (e != hipSuccess || !scratch)
            return fail(CK4_ERR_DEVICE, "%s: no address for the fixed buffer: %s", fn, hipGetErrorString(e));
    }
    return linear_w4a8(fn, x_q8, x_scales, w_packed, group_scales, false, m, n, k, group, y, ldy, chunk_cols, scratch,
                       need > 0 ? ck4::kNoallocScratchBytes : 0, stream);
}

ck4_status ck4_linear_w4a8_grouped_e4m3(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                        const uint8_t *group_scales, int64_t m, int64_t n, int64_t k, int group,
                                        uint16_t *y, int64_t ldy, int64_t chunk_cols, void *workspace,
                                        size_t ws_bytes, void *stream) {
    return linear_w4a8("ck4_linear_w4a8_grouped_e4m3", x_q8, x_scales, w_packed, group_scales, true, m, n, k, group,
                       y, ldy, chunk_cols, workspace, ws_bytes, stream);
}

ck4_status ck4_linear_w4a8_codebook(const int8_t *x_q8, const float *x_scales, const int8_t *w_packed,
                                    const void *group_scales, int scale_e4m3, const float *codebook, int64_t m,
                                    int64_t n, int64_t k, int group, uint16_t *y, int64_t ldy, int64_t chunk_cols,
                                    void *workspace, size_t ws_bytes, void *stream) {
    const char *fn = "ck4_linear_w4a8_codebook";
    ck4::Codebook cb;
    if (ck4_status s = make_codebook(fn, codebook, &cb)) return s;
    return linear_w4a8(fn, x_q8, x_scales, w_packed, group_scales, scale_e4m3 != 0, m, n, k, group, y, ldy,
                       chunk_cols, workspace, ws_bytes, stream, cb);
}

}  // extern "C"

namespace {

bool lora_rank_ok(int64_t rank) { return rank == 32 || rank == 64 || rank == 128 || rank == 256; }

}  // namespace

extern "C" {

ck4_status ck4_lora_prepare_down(const float *a, int64_t rank, int64_t k, int64_t lda, int rot_block,
                                 uint16_t *a_pack, void *stream) {
    const char *fn = "ck4_lora_prepare_down";
    if (!a || !a_pack) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (rank <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: rank and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "lda", lda, k, 4)) return s;
    if (!aligned(a, 16)) return fail(CK4_ERR_INVALID, "%s: a not 16-byte aligned", fn);
    if (!aligned(a_pack, 16)) return fail(CK4_ERR_INVALID, "%s: a_pack not 16-byte aligned", fn);
    if (!lora_rank_ok(rank))
        return fail(CK4_ERR_UNSUPPORTED, "%s: rank=%lld (need 32, 64, 128 or 256)", fn, (long long)rank);
    if (rot_block > 256) return fail(CK4_ERR_UNSUPPORTED, "%s: rot_block=%d > 256", fn, rot_block);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    if (k % 32 != 0) return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of 32", fn, (long long)k);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_rotate_quant(a, 1, rank, k, lda, rot_block, 3, 0, a_pack, k, nullptr,
                                                  static_cast<hipStream_t>(stream)));
}

ck4_status ck4_lora_prepare_up(const uint16_t *b, int64_t n, int64_t rank, int64_t ldb, uint16_t *b_pack,
                               void *stream) {
    const char *fn = "ck4_lora_prepare_up";
    if (!b || !b_pack) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (n <= 0) return fail(CK4_ERR_INVALID, "%s: n must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldb", ldb, rank, 4)) return s;
    if (!aligned(b, 8)) return fail(CK4_ERR_INVALID, "%s: b not 8-byte aligned", fn);
    if (!aligned(b_pack, 16)) return fail(CK4_ERR_INVALID, "%s: b_pack not 16-byte aligned", fn);
    if (!lora_rank_ok(rank))
        return fail(CK4_ERR_UNSUPPORTED, "%s: rank=%lld (need 32, 64, 128 or 256)", fn, (long long)rank);
    if (n > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: n too large", fn);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_lora_pack(b, n, rank, ldb, b_pack, static_cast<hipStream_t>(stream)));
}

ck4_status ck4_lora_down(const uint16_t *x, int64_t m, int64_t k, int64_t ldx, int rot_block, const uint16_t *a_pack,
                         int64_t rank, float alpha, uint16_t *t_pack, void *stream) {
    const uint16_t *a_rot = a_pack;
    uint16_t *t = t_pack;
    const char *fn = "ck4_lora_down";
    if (!x || !a_rot || !t) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (m <= 0 || k <= 0) return fail(CK4_ERR_INVALID, "%s: m and k must be positive", fn);
    if (ck4_status s = check_stride(fn, "ldx", ldx, k, 8)) return s;
    if (!aligned(x, 16)) return fail(CK4_ERR_INVALID, "%s: x not 16-byte aligned", fn);
    if (!aligned(a_rot, 16) || !aligned(t, 16)) return fail(CK4_ERR_INVALID, "%s: a_pack or t_pack misaligned", fn);
    if (m > kMaxRows) return fail(CK4_ERR_UNSUPPORTED, "%s: m too large", fn);
    if (!lora_rank_ok(rank))
        return fail(CK4_ERR_UNSUPPORTED, "%s: rank=%lld (need 32, 64, 128 or 256)", fn, (long long)rank);
    if (rot_block > 256) return fail(CK4_ERR_UNSUPPORTED, "%s: rot_block=%d > 256", fn, rot_block);
    if (ck4_status s = check_rot(fn, k, rot_block)) return s;
    const int64_t chunk = rot_block < 128 ? 128 : rot_block;
    if (k % chunk != 0)
        return fail(CK4_ERR_UNSUPPORTED, "%s: k=%lld is not a multiple of %lld", fn, (long long)k, (long long)chunk);
    if (ck4_status s = check_device(fn)) return s;
    return launched(fn, ck4::launch_lora_down(x, m, k, ldx, rot_block, a_rot, rank, alpha, t,
                                               static_cast<hipStream_t>(stream)));
}

ck4_status ck4_linear_w4a4_lora(const int8_t *x_q, const float *x_scales, const int8_t *w_packed,
                                const float *w_scales, const float *bias, const uint16_t *t_pack,
                                const uint16_t *b_pack, int64_t rank, int64_t m, int64_t n, int64_t k, uint16_t *y,
                                int64_t ldy, void *stream) {
    const char *fn = "ck4_linear_w4a4_lora";
    const uint16_t *t = t_pack, *b_up = b_pack;
    if (!t || !b_up) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (!aligned(t, 16) || !aligned(b_up, 16)) return fail(CK4_ERR_INVALID, "%s: t_pack or b_pack misaligned", fn);
    if (!lora_rank_ok(rank))
        return fail(CK4_ERR_UNSUPPORTED, "%s: rank=%lld (need 32, 64, 128 or 256)", fn, (long long)rank);
    return gemm_entry(fn, true, x_q, x_scales, w_packed, w_scales, bias, m, n, k, false, y, ldy, stream,
                      ck4::LoraUp{t, b_up, (int)rank});
}


static ck4_status fp6_lora_entry(const char *fn, const uint8_t *x_q6, const float *x_scales, const uint8_t *w_q6,
                                 const float *w_scales, const float *bias, const uint16_t *t_pack,
                                 const uint16_t *b_pack, int64_t rank, int64_t m, int64_t n, int64_t k, uint16_t *y,
                                 int64_t ldy, void *stream, bool compact) {
    if (!t_pack || !b_pack) return fail(CK4_ERR_INVALID, "%s: null pointer", fn);
    if (!aligned(t_pack, 16) || !aligned(b_pack, 16))
        return fail(CK4_ERR_INVALID, "%s: t_pack or b_pack misaligned", fn);
    if (!lora_rank_ok(rank))
        return fail(CK4_ERR_UNSUPPORTED, "%s: rank=%lld (need 32, 64, 128 or 256)", fn, (long long)rank);
    return gemm_fp6_entry(fn, x_q6, x_scales, w_q6, w_scales, bias, m, n, k, false, y, ldy, stream,
                          ck4::LoraUp{t_pack, b_pack, (int)rank}, compact);
}

ck4_status ck4_linear_w4a4_fp6_lora(const uint8_t *x_q6, const float *x_scales, const uint8_t *w_q6,
                                    const float *w_scales, const float *bias, const uint16_t *t_pack,
                                    const uint16_t *b_pack, int64_t rank, int64_t m, int64_t n, int64_t k,
                                    uint16_t *y, int64_t ldy, void *stream) {
    return fp6_lora_entry("ck4_linear_w4a4_fp6_lora", x_q6, x_scales, w_q6, w_scales, bias, t_pack, b_pack, rank,
                          m, n, k, y, ldy, stream, false);
}

ck4_status ck4_linear_w4a4_fp6c_lora(const uint8_t *x_q6c, const float *x_scales, const uint8_t *w_q6c,
                                     const float *w_scales, const float *bias, const uint16_t *t_pack,
                                     const uint16_t *b_pack, int64_t rank, int64_t m, int64_t n, int64_t k,
                                     uint16_t *y, int64_t ldy, void *stream) {
    return fp6_lora_entry("ck4_linear_w4a4_fp6c_lora", x_q6c, x_scales, w_q6c, w_scales, bias, t_pack, b_pack,
                          rank, m, n, k, y, ldy, stream, true);
}

}  // extern "C"
