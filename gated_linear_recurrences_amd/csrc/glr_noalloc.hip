// gdelta_chunk_fwd for callers that cannot allocate device memory: the workspace its kernels
// pass data through (the per-chunk factor T_U and cumulative log-gates, or the WY factors at
// the smaller chunks) is a fixed array of this file instead of a caller-owned buffer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "glr.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per device, alive until the process ends; shared by every call on that device.
// Host code never passes this name to a kernel: it stands for a host-side shadow, not a
// device address. The device address comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;

// The device address of `scratch` on the current device, looked up once per device.
la_status current_scratch(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        char msg[160];
        std::snprintf(msg, sizeof(msg), "hipGetDevice failed: %s", hipGetErrorString(err));
        return static_cast<la_status>(glr::report_error(LA_ERR_HIP, msg));
    }
    if (dev < 0 || dev >= kMaxDevices)
        return static_cast<la_status>(glr::report_error(LA_ERR_UNSUPPORTED, "device index above 63"));
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess || p == nullptr) {
                char msg[160];
                std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(err));
                return static_cast<la_status>(glr::report_error(LA_ERR_HIP, msg));
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LA_OK;
}

}  // namespace

extern "C" la_status gdelta_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                              const float* beta, const float* s0, void* o, float* s_out,
                                              int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                                              void* stream) {
    // every argument is checked before the array is looked up, so a rejected call touches no device
    const glr::ChunkArgs a{q, k, v, log_alpha, beta, s0, o, s_out, B, H, T, dk, dv, chunk, nullptr};
    la_status st = static_cast<la_status>(glr::check_chunk_call(glr::kGDelta, a, dtype));
    if (st != LA_OK) return st;
    size_t need = 0;
    st = la_chunk_workspace_size(LA_GDELTA, B, H, T, dk, dv, chunk, dtype, &need);
    if (st != LA_OK) return st;
    if (need > kScratchBytes) {
        char msg[160];
        std::snprintf(msg, sizeof(msg), "workspace of %zu bytes exceeds the fixed %zu bytes of the no-allocation entry point",
                      need, kScratchBytes);
        return static_cast<la_status>(glr::report_error(LA_ERR_UNSUPPORTED, msg));
    }
    void* ws = nullptr;
    if (need > 0 && B > 0 && H > 0) {
        st = current_scratch(&ws);
        if (st != LA_OK) return st;
    }
    return gdelta_chunk_fwd(q, k, v, log_alpha, beta, s0, o, s_out, B, H, T, dk, dv, chunk, dtype, ws, need,
                            stream);
}
