// noalloc.hip -- the fixed scratch array of bmmc_execute_noalloc, the entry
// point (in api.cpp) that allocates no device memory, for callers that cannot
// allocate (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// Only a two-pass plan needs memory beyond its input and output: the array
// between its two passes.  Here that array is the file-scope device array
// `scratch` below, of a fixed size, which every GPU the library runs on holds
// from the code object's load until the process ends.  Its address is taken
// once per device with hipGetSymbolAddress (the array's name in host code is a
// host-side stand-in, not a device address) and kept per device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/bmmc.h"
#include "launch.h"

// The array between the two passes of every bmmc_execute_noalloc call on a
// device (calls that overlap in time on one device race on it).
static __device__ __align__(256) uint8_t scratch[BMMC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
int device_scratch(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return BMMC_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return BMMC_ERR_UNSUPPORTED;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return BMMC_ERR_HIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BMMC_OK;
}

}  // namespace

namespace bmmc {

int noalloc_scratch(void **out) { return device_scratch(out); }

}  // namespace bmmc
