// Device scratch of gattn_decode_noalloc: the split-KV partials of a decode call live in this
// file-scope device array instead of a caller-supplied workspace, for callers that cannot allocate.
//
// Every GPU the library runs on holds its own copy of `scratch` (GATTN_NOALLOC_SCRATCH_BYTES) from
// the moment the library's code is loaded on it until the process ends. In host code the array's
// name is only a stand-in: the device address of this device's copy is looked up once per device
// with hipGetSymbolAddress (with that device current) and cached, and only that address is ever
// handed to kernels. Calls on one device share its copy; calls that overlap on one device (other
// streams, other host threads) race on it. Nothing in it needs to start at any particular value:
// every partial the combine reads is written by the same call's split kernel first.
#include <atomic>
#include <mutex>

#include "../../include/gattn.h"
#include "kernels.h"

namespace gattn {

namespace {

static __device__ __align__(256) uint8_t scratch[GATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_lookup;

}  // namespace

hipError_t noalloc_scratch(void **ptr, size_t *bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (!p)
                return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    *bytes = GATTN_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace gattn
