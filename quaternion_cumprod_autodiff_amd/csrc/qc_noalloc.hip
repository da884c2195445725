// qc_noalloc.hip -- quat_cumprod_bwd_noalloc: the backward of the quaternion
// scan for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Its workspace is a fixed
// device array of this library instead of a caller's buffer.
//
// The array lives once per GPU, for the life of the process.  On the first
// call on a device (with that device current) its device address is taken
// with hipGetSymbolAddress and kept per device; host code only ever uses that
// address.  The same call zeroes the array's header (status word and launch
// counter) with the library's fill kernel.  Carry slots need no clearing:
// every slot is validated by a hash of its value and the launch's epoch, so
// contents left by earlier calls are never accepted.  Every call ends with a
// one-thread kernel that hands the status bits of the call to the caller's
// `status` word (when given) and clears them, so each call starts clean.
#include "quat_cumprod.h"
#include "qc_internal.hpp"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void take_status_kernel(uint32_t* hdr, int32_t* out) {
    if (threadIdx.x == 0) {
        const uint32_t bits = __hip_atomic_exchange(&hdr[qc::kHdrStatus], 0u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (out != nullptr) out[0] = int32_t(bits);
    }
}

// Device address of this device's copy of `scratch` (set up on first use).
int scratch_for_current_device(hipStream_t st, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return qc::record_hip_error(e);
    if (dev < 0 || dev >= kMaxDevices) return QC_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return qc::record_hip_error(e);
        if (p == nullptr) return QC_ERR_HIP;
        e = qc::launch_zero_words(static_cast<uint32_t*>(p), size_t(qc::kHdrWords), st);
        if (e != hipSuccess) return qc::record_hip_error(e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QC_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

extern "C" int quat_cumprod_bwd_noalloc(const void* q, const void* init, const void* d_cum, const void* ckpt,
                                        size_t ckpt_bytes, void* d_q, void* d_init,
                                        int64_t b, int64_t s, int64_t h, int64_t j, int32_t dtype,
                                        int32_t* status, void* stream) {
    // Arguments that need no device: shape, dtype, the fixed maximum.
    const size_t need = quat_cumprod_workspace_bytes(b, s, h, j, dtype);
    if (need == 0 || (!d_q && !d_init))   // invalid shape or dtype, or nothing wanted: same code as the
        return quat_cumprod_bwd(q, init, d_cum, ckpt, ckpt_bytes, d_q, d_init, b, s, h, j, dtype,
                                nullptr, 0, stream);   // allocating form, which fails or returns before any HIP call
    if (need > kScratchBytes) return QC_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(status) % 4 != 0) return QC_ERR_ALIGN;
    if (status != nullptr) {
        const size_t io = dtype == QC_DTYPE_F32 ? 16 : 8;
        const size_t big = size_t(b) * size_t(s) * size_t(h) * size_t(j) * io, small = size_t(b) * size_t(h) * size_t(j) * io;
        const size_t ck = quat_cumprod_ckpt_bytes(b, s, h, j, dtype);
        if (overlaps(status, 4, q, big) || overlaps(status, 4, init, small) || overlaps(status, 4, d_cum, big) ||
            overlaps(status, 4, ckpt, ck) || overlaps(status, 4, d_q, big) || overlaps(status, 4, d_init, small))
            return QC_ERR_ALIAS;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    int rc = scratch_for_current_device(st, &ws);
    if (rc != QC_OK) return rc;
    rc = quat_cumprod_bwd(q, init, d_cum, ckpt, ckpt_bytes, d_q, d_init, b, s, h, j, dtype, ws, kScratchBytes,
                          stream);
    if (rc != QC_OK) return rc;
    uint32_t* hdr = static_cast<uint32_t*>(ws);
    int32_t* out = status;
    void* params[] = {&hdr, &out};
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(&take_status_kernel), dim3(1), dim3(64), params, 0, st);
    return e == hipSuccess ? QC_OK : qc::record_hip_error(e);
}
