// launch_stubs.cpp -- stand-ins for the device-side half of the library in
// the host-only sanitizer build (tests/test_sanitize_host.py): the kernels'
// launchers and the fixed scratch array of bmmc_execute_noalloc.  The CPU
// tests that load that build never reach them; if one did, it gets an error
// status, as a HIP call without a GPU would return.
#include "../../bmmc_affine_index_amd/csrc/launch.h"

namespace bmmc {

int launch_tiled(const bmmc_pass_desc &, const void *, void *, hipStream_t) {
    return BMMC_ERR_HIP;
}
int launch_chunk(const bmmc_pass_desc &, const void *, void *, hipStream_t) {
    return BMMC_ERR_HIP;
}
int launch_copy(const void *, void *, size_t, hipStream_t) { return BMMC_ERR_HIP; }
int noalloc_scratch(void **) { return BMMC_ERR_HIP; }

}  // namespace bmmc
