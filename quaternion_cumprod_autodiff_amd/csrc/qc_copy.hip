// qc_copy.hip -- a plain streaming device copy for gfx950, the practical
// bandwidth ceiling that the scan kernels are measured against (include/qc_bench.h).
//
// Each block copies 16 KiB per iteration: 256 threads x 4 vectors of 16 bytes,
// the four loads of a thread issued before its stores, so a wave has 4 KiB of
// reads in flight and every load or store instruction of a wave covers 1 KiB
// contiguous.  Loads and stores are non-temporal (the data is touched once).
// The grid is a fixed number of blocks per compute unit walking the buffer in
// block-sized strides.
#include "qc_bench.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kPerBlock = int64_t(kThreads) * kUnroll;   // vectors per block iteration

__global__ void __launch_bounds__(kThreads) stream_copy_kernel(const f32x4* __restrict__ src,
                                                               f32x4* __restrict__ dst, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * kPerBlock;
    for (int64_t base = int64_t(blockIdx.x) * kPerBlock + threadIdx.x; base < n; base += stride) {
        f32x4 v[kUnroll];
        if (base + (kUnroll - 1) * kThreads < n) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + base + u * kThreads);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + base + u * kThreads);
        } else {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (base + u * kThreads < n) v[u] = __builtin_nontemporal_load(src + base + u * kThreads);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (base + u * kThreads < n) __builtin_nontemporal_store(v[u], dst + base + u * kThreads);
        }
    }
}

}  // namespace

extern "C" int qc_stream_copy(const void* src, void* dst, size_t nbytes, int32_t blocks_per_cu, void* stream) {
    if (nbytes == 0) return 0;
    if (!src || !dst) return -1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | nbytes) % 16 != 0) return -3;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + nbytes && d0 < s0 + nbytes) return -5;
    if (blocks_per_cu < 1 || blocks_per_cu > 64) return -8;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -7;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -7;
    const int64_t n = int64_t(nbytes / 16);
    int64_t blocks = int64_t(cus) * blocks_per_cu;
    const int64_t needed = (n + kPerBlock - 1) / kPerBlock;
    if (blocks > needed) blocks = needed;
    const f32x4* s = static_cast<const f32x4*>(src);
    f32x4* d = static_cast<f32x4*>(dst);
    int64_t nn = n;
    void* params[] = {&s, &d, &nn};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&stream_copy_kernel), dim3(unsigned(blocks)),
                                         dim3(kThreads), params, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? 0 : -7;
}
