// Measurement helpers exported next to the operators: a streaming copy of
// known size (the practical HBM ceiling, and the calibration kernel for the
// hardware byte counters) and an empty kernel (the launch floor).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rowred.h"

namespace {

typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 1;  // float4 packs per thread

// Thread t of group g copies packs (g * kCopyUnroll + u) * kCopyBlock + t of
// n / 4 whole packs; group 0's threads also copy the n % 4 trailing floats.
// One non-temporal 16-byte load and store per thread: the fastest plain copy
// measured on MI355X (6.63 TB/s over 1 GiB moved; 6.0-6.3 TB/s with 2, 4 or 8
// packs per thread or 512- and 1024-thread groups, 5.7 TB/s without the
// non-temporal hints; a 1 GiB read-only stream reaches 7.0 TB/s, a
// write-only one 6.0 TB/s).
__global__ void __launch_bounds__(kCopyBlock) copy_kernel(const float *__restrict__ src,
                                                          float *__restrict__ dst, int64_t n) {
    const int64_t packs = n / 4;
    const int64_t first = (int64_t)blockIdx.x * kCopyUnroll * kCopyBlock + threadIdx.x;
    f32x4u v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t p = first + (int64_t)u * kCopyBlock;
        if (p < packs) v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4u *>(src + 4 * p));
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t p = first + (int64_t)u * kCopyBlock;
        if (p < packs) __builtin_nontemporal_store(v[u], reinterpret_cast<f32x4u *>(dst + 4 * p));
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) dst[4 * packs + threadIdx.x] = src[4 * packs + threadIdx.x];
}

__global__ void __launch_bounds__(64) empty_kernel() {}

}  // namespace

extern "C" {

int rr_copy_f32(const float *src, float *dst, int64_t n, void *stream) {
    if (n < 0) return RR_ERR_INVALID_ARGUMENT;
    if (n == 0) return RR_OK;
    if (src == nullptr || dst == nullptr || (reinterpret_cast<uintptr_t>(src) & 3u) ||
        (reinterpret_cast<uintptr_t>(dst) & 3u))
        return RR_ERR_INVALID_ARGUMENT;
    const int64_t packs = n / 4;
    int64_t groups = (packs + (int64_t)kCopyBlock * kCopyUnroll - 1) / ((int64_t)kCopyBlock * kCopyUnroll);
    if (groups == 0) groups = 1;
    if (groups > 0x7fffffff) return RR_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)groups), dim3(kCopyBlock), 0,
                       reinterpret_cast<hipStream_t>(stream), src, dst, n);
    return hipGetLastError() == hipSuccess ? RR_OK : RR_ERR_LAUNCH;
}

int rr_empty_kernel(void *stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? RR_OK : RR_ERR_LAUNCH;
}

}  // extern "C"
