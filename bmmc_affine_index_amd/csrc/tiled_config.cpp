// tiled_config.cpp -- which tile-pass launches the compiled kernels cover (host-only).
#include "kernels/tiled_cfg.h"
#include "launch.h"

namespace bmmc {

bool tiled_supported(int unit_log2, int t, int iters_log2, int launch, int threads_log2,
                     int split_stage, int buffer_loads) {
    if (unit_log2 < 0 || unit_log2 > 4 || t < 1) return false;
    // buffer loads: one whole tile per workgroup, units of 4 bytes or more
    if (buffer_loads && (buffer_loads != 1 || launch != BMMC_LAUNCH_ONE_TILE ||
                         iters_log2 != 0 || split_stage != 0 || unit_log2 < 2))
        return false;
    // split staging: one tile per workgroup, at least two passes per tile
    if (split_stage && (split_stage != 1 || launch != BMMC_LAUNCH_ONE_TILE || iters_log2 != 0 ||
                        2 * t - ((4 - unit_log2) < t ? (4 - unit_log2) : t) - threads_log2 < 1))
        return false;
    // the 256-thread kernels, and the 512-thread ones where a tile has more
    // than 256 chunks and one tile per workgroup
    const int narrow = tile_threads_log2(unit_log2, t, kTileMaxNTL);
    const int wide = tile_threads_log2(unit_log2, t, kTileWideNTL);
    if (threads_log2 != narrow && !(threads_log2 == wide && wide > narrow && iters_log2 == 0))
        return false;
    if ((launch == BMMC_LAUNCH_PERSISTENT || launch == BMMC_LAUNCH_STREAMED) &&
        (iters_log2 != 0 || unit_log2 < 0 || unit_log2 > 4 || t < 1 ||
         (uint64_t(2) << (2 * t + unit_log2)) > 131072))
        return false;
    if (launch == BMMC_LAUNCH_STREAMED) {
        // each role must be whole waves: 2t - (units per chunk, log2) >= 6
        const int wl = (4 - unit_log2) < t ? (4 - unit_log2) : t;
        if (2 * t - wl < 6) return false;
    }
    return tiled_config_exists(unit_log2, t, iters_log2);
}

}  // namespace bmmc
