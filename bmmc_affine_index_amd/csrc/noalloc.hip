// noalloc.hip -- bmmc_execute_noalloc: bmmc_execute without any device
// allocation, for callers that cannot allocate (code under stream capture,
// tight serving loops, harnesses that forbid hipMalloc).
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
#include "plan.h"

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

extern "C" int bmmc_execute_noalloc(const bmmc_plan *p, const void *in, void *out,
                                    void *stream) {
    // every argument check comes before the first HIP call
    const int arg = bmmc::check_execute_buffers(p, in, out);
    if (arg != BMMC_OK) return arg;
    void *buf = nullptr;
    if (p->npasses > 1) {
        // the array between the passes must fit the fixed buffer
        if (((size_t)p->elem_bytes << p->n) > (size_t)BMMC_NOALLOC_SCRATCH_BYTES)
            return BMMC_ERR_SCRATCH_LIMIT;
        const int st = device_scratch(&buf);
        if (st != BMMC_OK) return st;
    }
    return bmmc::execute_with_scratch(p, in, out, buf, static_cast<hipStream_t>(stream));
}
