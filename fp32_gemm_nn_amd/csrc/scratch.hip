// The static device scratch of mi_sgemm_noalloc and the lookup of its
// address on each device. A translation unit of its own, so that only
// processes that call mi_sgemm_noalloc load its code object (and with it the
// 64 MiB array) onto a GPU.
//
// In host code the name `scratch` is a host-side stand-in for the array, not
// a device address: it is never passed to a kernel or a copy. Every use goes
// through the address hipGetSymbolAddress returns for the device, kept per
// device below.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "scratch.h"

// Partial blocks (kPartialFloats floats), then the tile counters as 32-bit
// integers. One copy per GPU; the loader hands it over zero-filled.
static __device__ __align__(256) float scratch[misgemm_scratch::kPartialFloats + misgemm_scratch::kCounters];

namespace misgemm_scratch {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<float *> g_ptr[kMaxDevices];
std::mutex g_lookup;

}  // namespace

bool device_scratch(int dev, float **partials, int **counters, bool *first) {
    *first = false;
    if (dev < 0 || dev >= kMaxDevices) return false;
    float *p = g_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int saved = -1;
            if (hipGetDevice(&saved) != hipSuccess) {
                (void)hipGetLastError();
                return false;
            }
            if (saved != dev && hipSetDevice(dev) != hipSuccess) {
                (void)hipGetLastError();
                return false;
            }
            void *addr = nullptr;
            const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (saved != dev) (void)hipSetDevice(saved);
            if (e != hipSuccess || addr == nullptr) {
                (void)hipGetLastError();
                return false;
            }
            p = static_cast<float *>(addr);
            g_ptr[dev].store(p, std::memory_order_release);
            *first = true;
        }
    }
    *partials = p;
    *counters = reinterpret_cast<int *>(p + kPartialFloats);
    return true;
}

}  // namespace misgemm_scratch
