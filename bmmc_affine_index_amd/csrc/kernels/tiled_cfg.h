// tiled_cfg.h -- geometry of the tile kernel's compiled configurations
// (plain C++: shared by the kernels and the host code that checks a plan).
#pragma once

#include <stdint.h>

namespace bmmc {

// log2 of the most threads one tile is moved by: 256 by default, 512 as a
// plan option (bmmc_plan_options.tile_threads_log2).  With 512 a wave holds
// half as many chunks and each SIMD runs twice the waves, which hides the
// LDS and barrier latency between a tile's loads and its stores: measured on
// MI355X, bit reversal n = 28 on the streamed launch moves from 0.850 to
// 0.865 of copy; one-tile launches of 64 KiB tiles lose 1% (random BMMC).
// 1024 threads lose up to 55% on one-tile launches (occupancy).
constexpr int kTileMaxNTL = 8;
constexpr int kTileWideNTL = 9;

// Buffer loads (bmmc_plan_options.buffer_loads) address the input by 32-bit
// byte offsets within a buffer whose size field holds the array's bytes:
// arrays of at most 2^31 bytes.
constexpr int kBufferLoadMaxLog2 = 31;

template <int UL, int T, int IT, int TL = kTileMaxNTL> struct TiledCfg {
    static constexpr int U = 1 << UL;
    static constexpr int WL = (4 - UL) < T ? (4 - UL) : T;  // log2 units per chunk
    static constexpr int W = 1 << WL;
    static constexpr int CB = U << WL;                      // chunk bytes
    static constexpr int CPSL = T - WL;                     // log2 chunks per row
    static constexpr int CHL = 2 * T - WL;                  // log2 chunks per tile
    static constexpr int NTL = CHL < TL ? CHL : TL;        // log2 threads
    static constexpr int NT = 1 << NTL;
    static constexpr int RPPL = NTL - CPSL;                 // log2 rows per pass
    static constexpr int JL = CHL - NTL;                    // log2 passes per tile
    static constexpr int J = 1 << JL;
    static constexpr int TILE = U << (2 * T);               // bytes per tile
    static constexpr int LDS = TILE << IT;
    static_assert(RPPL >= 0 && JL >= 0, "tile geometry");
};

// Largest tile side per unit size (log2 bytes 0..4) and largest iteration
// count of the one-tile launch that are compiled.
constexpr int kMaxT[5] = {8, 7, 7, 6, 6};
constexpr int kMaxIT = 3;

// Whether the one-tile kernel is compiled for unit size 2^ul bytes, side 2^t
// units and 2^it tiles per workgroup: the sides and counts above, with at
// most 64 KiB of LDS.
constexpr bool tiled_config_exists(int ul, int t, int it) {
    return ul >= 0 && ul <= 4 && t >= 1 && t <= kMaxT[ul] && it >= 0 && it <= kMaxIT &&
           ((int64_t(1) << ul) << (2 * t) << it) <= 65536;
}

template <int UL, int T, int IT> constexpr bool valid_cfg() {
    return tiled_config_exists(UL, T, IT);
}

// log2 of the threads that move one tile of 2^(2t) units of 2^ul bytes when
// at most 2^tl may: one 16-byte chunk (or the whole row, for short rows) per
// thread and pass.
constexpr int tile_threads_log2(int ul, int t, int tl) {
    const int wl = (4 - ul) < t ? (4 - ul) : t;
    const int chl = 2 * t - wl;
    return chl < tl ? chl : tl;
}

}  // namespace bmmc
