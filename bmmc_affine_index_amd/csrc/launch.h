// launch.h -- host entry points of the kernel families (defined in kernels/).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bmmc.h"

namespace bmmc {

// LDS-staged tile pass (BMMC_KERNEL_TILED).
int launch_tiled(const bmmc_pass_desc &d, const void *in, void *out, hipStream_t s);
// Chunk moves (BMMC_KERNEL_CHUNK) and the one-unit naive pass (BMMC_KERNEL_NAIVE).
int launch_chunk(const bmmc_pass_desc &d, const void *in, void *out, hipStream_t s);
// Identity-order copy of nbytes.
int launch_copy(const void *in, void *out, size_t nbytes, hipStream_t s);

// bmmc_execute's argument checks (NULL, alignment, overlap), host-only.
int check_execute_buffers(const bmmc_plan *p, const void *in, const void *out);
// bmmc_execute through a scratch array the caller provides (one array's
// bytes on the current device; one-pass plans ignore it).  Defined in api.cpp.
int execute_with_scratch(const bmmc_plan *p, const void *in, void *out, void *scratch,
                         hipStream_t s);

// The device address of the fixed scratch array of bmmc_execute_noalloc
// (BMMC_NOALLOC_SCRATCH_BYTES) on the current device.  Defined in noalloc.hip.
int noalloc_scratch(void **out);

// Whether the tile kernel is compiled for this unit size, side, iteration
// count, launch style, thread count, staging and load form.
bool tiled_supported(int unit_log2, int t, int iters_log2, int launch, int threads_log2,
                     int split_stage, int buffer_loads);

// The dispatch packet gives the grid size in work-items as a 32-bit count,
// so one launch covers at most 2^31 work-items here; bigger passes are split
// into several launches (the kernels take the first workgroup's index).
constexpr uint64_t kMaxWorkItemsPerLaunch = uint64_t(1) << 31;
constexpr uint64_t max_blocks_per_launch(uint32_t threads) {
    return kMaxWorkItemsPerLaunch / threads;
}

}  // namespace bmmc
