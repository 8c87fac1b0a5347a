// Streaming-read probe of the benchmark (libck4_bench.so, not part of the
// ck4 ABI): how fast a plain kernel can read a buffer of a given size on
// this part. The skinny-M layers are weight-streaming, so their HBM figure is
// reported both against the 8 TB/s peak and against what this kernel reaches
// on buffers of the same size.
//
// Each thread reads four 16-byte words, all issued before any is used, and
// folds them with XOR; a word is written only if the fold hits a value the
// caller passes and the data never produces, so the loads cannot be removed
// and the kernel writes (almost) nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                              uint32_t key, uint32_t *__restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kPerThread) + threadIdx.x;
    uint4 v[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        v[i] = j < n16 ? p[j] : make_uint4(0, 0, 0, 0);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == key) sink[blockIdx.x & 255] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, > 0) from the 16-byte aligned device
// buffer p on `stream`; sink is device memory of at least 1 KB. Returns 0, or
// -1 for invalid arguments, or the HIP error code of the launch.
int ck4_bench_stream_read(const void *p, int64_t bytes, uint32_t key, void *sink, void *stream) {
    if (!p || !sink || bytes <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15) != 0) return -1;
    const int64_t n16 = bytes / 16;
    const int64_t per_block = (int64_t)kThreads * kPerThread;
    const int64_t blocks = (n16 + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return -1;
    stream_read_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4 *>(p), n16, key, static_cast<uint32_t *>(sink));
    return (int)hipGetLastError();
}

}  // extern "C"
