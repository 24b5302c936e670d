// tiled.hip -- the LDS-staged tile pass for gfx950.
//
// One workgroup moves one tile (or 2^IT tiles) of 2^(2T) units: the 2^T input
// segments (rows) of the tile are read with coalesced vector loads, staged in
// LDS through an XOR swizzle, and read back in output order so that every
// store writes whole output segments ("Efficient GPU Implementation of Affine
// Index Permutations on Arrays": tiled BMMCs run almost as fast as a copy,
// fully coalesced and bank-conflict free; appendix: the tiled and banks
// bit-reversal kernels stage a 32 x 32 tile in shared memory between a
// coalesced read and a coalesced write).
//
// Differences from the pages' kernels, for gfx950:
//  * one generic kernel for every (A, c): the planner passes XOR tables of
//    column contributions instead of generating a kernel per permutation; an
//    address costs one XOR per chunk beyond the wave-uniform part;
//  * 64-lane waves move 16-byte chunks (dwordx4 global access, b128 LDS
//    writes), and tiles are 64 x 64 units for 4-byte units (256-byte
//    segments);
//  * the LDS swizzle is an XOR of row bits into the chunk index, chosen per
//    plan so that the output-order reads hit distinct banks.
#include "../launch.h"
#include "common.h"
#include "tiled_cfg.h"

namespace bmmc {

// Tile bases: the wave reduction when the workgroup is made of full waves,
// the scalar loop otherwise.  A one-tile launch of a small array runs one
// workgroup per compute unit, whose scalar cache is cold: the loop's chain
// of dependent table loads measured 13-16% of a 4 MiB pass.  A base comes in
// two steps, the lane's table load (base_issue) and the reduction
// (base_finish), so that a kernel needing several bases issues all their
// loads before it waits: left to itself the compiler waits for each base's
// load before it issues the next, one memory round trip per base.
template <class C, typename T>
__device__ __forceinline__ T base_issue(const T *tab, uint64_t blk) {
    if constexpr (C::NT >= 64) return dev::wave_load(tab);
    else return dev::xor_bits_uniform(tab, blk);
}

template <class C, typename T>
__device__ __forceinline__ T base_finish(T e, uint64_t blk) {
    if constexpr (C::NT >= 64) return dev::wave_select_xor(e, blk);
    else return e;
}

// Both steps at once, with the table load under each lane's condition.
template <class C, typename T>
__device__ __forceinline__ T tile_base(const T *tab, uint64_t blk) {
    if constexpr (C::NT >= 64) return dev::xor_bits_wave(tab, blk);
    else return dev::xor_bits_uniform(tab, blk);
}

// The walk a workgroup of the persistent and streamed launches takes: its
// index with the low three bits XORed with the next three (a permutation of
// every aligned group of eight).  Workgroups go to the eight XCDs round-robin
// (w mod 8), so without it each XCD would walk every eighth tile range; with
// it the ranges of one XCD spread over all residues.  Measured on MI355X:
// +1% on bit reversal n = 28, +1.6% on random 16-byte BPCs n = 27, +3.5% on
// the 64 MiB transpose (streamed), -0.4% on the 16384 x 16384 transpose.
__device__ __forceinline__ uint64_t walker_index(uint32_t w) {
    return (uint64_t)(w ^ ((w >> 3) & 7u));
}

// Per-lane address parts, fixed for the whole launch: the XOR of the table
// entries of the thread-index bits of a chunk (chunk c = (j << NTL) | tid).
struct LaneParts {
    uint64_t in_lane, out_lane;
    uint32_t wr_lane, rd_lane;
};

template <class C, int T>
__device__ __forceinline__ LaneParts lane_parts(const bmmc_pass_desc &d, uint32_t tid) {
    LaneParts p;
    p.in_lane = dev::xor_bits_lane<C::NTL>(d.ld_in, tid);
    p.wr_lane = dev::xor_bits_lane<C::NTL>(d.ld_lds, tid);
    p.out_lane = dev::xor_bits_lane<C::NTL>(d.st_out, tid);
    p.rd_lane = dev::xor_bits_lane<C::NTL>(d.st_lds, tid);
    return p;
}

// Issue the global loads of one tile: pass j covers chunks (j << NTL) | tid.
template <class C, int T, bool NT>
__device__ __forceinline__ void load_tile(dev::Chunk<C::CB> (&v)[C::J], const uint8_t *in,
                                          uint64_t in_base, const bmmc_pass_desc &d,
                                          const LaneParts &p) {
#pragma unroll
    for (int j = 0; j < C::J; ++j) {
        const uint64_t in_j = in_base ^ dev::xor_bits_lane<C::JL>(d.ld_in + C::NTL, (uint32_t)j);
        v[j] = dev::gload_nt<C::CB, NT>(in + (in_j ^ p.in_lane));
    }
}

// load_tile with buffer loads: the same byte offsets, as 32-bit offsets
// within the input's buffer (arrays of at most 2^31 bytes).
template <class C, int T, bool NT>
__device__ __forceinline__ void load_tile_buf(dev::Chunk<C::CB> (&v)[C::J],
                                              __amdgpu_buffer_rsrc_t in, uint64_t in_base,
                                              const bmmc_pass_desc &d, const LaneParts &p) {
#pragma unroll
    for (int j = 0; j < C::J; ++j) {
        const uint64_t in_j = in_base ^ dev::xor_bits_lane<C::JL>(d.ld_in + C::NTL, (uint32_t)j);
        v[j] = dev::bload<C::CB, NT>(in, (uint32_t)(in_j ^ p.in_lane));
    }
}

// load_tile with the per-pass input offsets given (the XORs of the table
// entries of the pass bits, read beforehand).
template <class C, int T, bool NT>
__device__ __forceinline__ void load_tile_jo(dev::Chunk<C::CB> (&v)[C::J], const uint8_t *in,
                                             uint64_t in_base, const uint64_t (&jo)[C::J],
                                             const LaneParts &p) {
#pragma unroll
    for (int j = 0; j < C::J; ++j) v[j] = dev::gload_nt<C::CB, NT>(in + ((in_base ^ jo[j]) ^ p.in_lane));
}

// Write the tile's chunks of passes J0 .. JN-1 to LDS through the swizzle.
template <class C, int T, int J0 = 0, int JN = C::J>
__device__ __forceinline__ void stage_tile(uint8_t *tile_lds, const dev::Chunk<C::CB> (&v)[C::J],
                                           const bmmc_pass_desc &d, const LaneParts &p) {
#pragma unroll
    for (int j = J0; j < JN; ++j) {
        const uint32_t wr_j = dev::xor_bits_lane<C::JL>(d.ld_lds + C::NTL, (uint32_t)j);
        dev::lds_store<C::CB>(tile_lds + (wr_j ^ p.wr_lane), v[j]);
    }
}

// Read the tile back in output order and store whole output chunks (drain
// passes J0 .. JN-1).
template <class C, int T, bool NT, int J0 = 0, int JN = C::J>
__device__ __forceinline__ void drain_tile(uint8_t *out, const uint8_t *tile_lds, uint64_t obase,
                                           uint32_t rbase, const bmmc_pass_desc &d,
                                           const LaneParts &p) {
#pragma unroll
    for (int j = J0; j < JN; ++j) {
        const uint64_t out_j =
            obase ^ dev::xor_bits_lane<C::JL>(d.st_out + C::NTL, (uint32_t)j);
        const uint32_t rd_j =
            rbase ^ dev::xor_bits_lane<C::JL>(d.st_lds + C::NTL, (uint32_t)j) ^ p.rd_lane;
        dev::Chunk<C::CB> ch;
        dev::zero(ch);
#pragma unroll
        for (int e = 0; e < C::W; ++e) {
            const uint32_t rd_e = dev::xor_bits_lane<C::WL>(d.st_unit, (uint32_t)e);
            dev::put_unit<C::CB, C::U>(ch, e, dev::lds_load_unit<C::U>(tile_lds + (rd_j ^ rd_e)));
        }
        dev::gstore_nt<C::CB, NT>(out + (out_j ^ p.out_lane), ch);
    }
}

// One workgroup per tile, or per 2^IT tiles whose loads are all issued
// before the barrier (the pages' iterated variant).
template <int UL, int T, int IT, bool NT, int TL>
__global__ void __launch_bounds__((TiledCfg<UL, T, IT, TL>::NT))
    bmmc_tiled_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                      const bmmc_pass_desc d, uint64_t blk0) {
    using C = TiledCfg<UL, T, IT, TL>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
    const LaneParts p = lane_parts<C, T>(d, threadIdx.x);
    const uint64_t tile0 = (blk0 + blockIdx.x) << IT;

    dev::Chunk<C::CB> v[1 << IT][C::J];
#pragma unroll
    for (int s = 0; s < (1 << IT); ++s)
        load_tile<C, T, NT>(v[s], in, tile_base<C>(d.in_blk, tile0 | (uint64_t)s), d, p);
#pragma unroll
    for (int s = 0; s < (1 << IT); ++s) stage_tile<C, T>(lds + s * C::TILE, v[s], d, p);
    __syncthreads();
    // The output and LDS bases are computed here, after the barrier, one
    // after the other.  Issued with the input base, before the tile's loads,
    // they made the 4096 x 4096 4-byte transpose (t = 7, two workgroups per
    // compute unit, two rounds of them) 7% slower, and issued together here
    // 2% slower: its stores gain from starting later.  Small arrays, which
    // would gain from the earlier bases, run faster on the streamed launch.
#pragma unroll
    for (int s = 0; s < (1 << IT); ++s) {
        const uint64_t blk = tile0 | (uint64_t)s;
        drain_tile<C, T, NT>(out, lds + s * C::TILE, tile_base<C>(d.out_blk, blk) ^ d.out_c,
                             tile_base<C>(d.lds_blk, blk) ^ d.lds_c, d, p);
    }
}

// One workgroup per tile, the input read with buffer loads (32-bit offsets
// from a base in scalar registers instead of 64-bit addresses per lane); the
// rest as bmmc_tiled_kernel with one tile.  The array holds at most 2^31
// bytes.  Measured on MI355X against global loads of the same plan: from
// -1% to +4% by matrix (the slowest random 16-byte BPC gains most), so the
// tuning decides.
template <int UL, int T, bool NT, int TL>
__global__ void __launch_bounds__((TiledCfg<UL, T, 0, TL>::NT))
    bmmc_tiled_bufload_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                              const bmmc_pass_desc d, uint64_t blk0) {
    using C = TiledCfg<UL, T, 0, TL>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
    const LaneParts p = lane_parts<C, T>(d, threadIdx.x);
    const uint64_t blk = blk0 + blockIdx.x;
    const __amdgpu_buffer_rsrc_t rin = dev::buffer_rsrc(in, 1u << (d.nbits + d.unit_log2));

    dev::Chunk<C::CB> v[C::J];
    load_tile_buf<C, T, NT>(v, rin, tile_base<C>(d.in_blk, blk), d, p);
    stage_tile<C, T>(lds, v, d, p);
    __syncthreads();
    drain_tile<C, T, NT>(out, lds, tile_base<C>(d.out_blk, blk) ^ d.out_c,
                         tile_base<C>(d.lds_blk, blk) ^ d.lds_c, d, p);
}

// One workgroup per tile, staged in LDS half at a time.  The planner builds
// the tables so that the chunks of passes j < J/2 hold one half of the tile's
// units on the load side and on the drain side alike (each tile's drain base
// already picks the matching half), and the LDS offsets of either half cover
// half a tile.  With half the LDS per workgroup, twice the tiles hold LDS on a
// compute unit at once, each with all its loads issued up front; the second
// half's staging waits only for its own loads and for the barrier after the
// first half's reads.
template <int UL, int T, bool NT, int TL>
__global__ void __launch_bounds__((TiledCfg<UL, T, 0, TL>::NT))
    bmmc_tiled_split_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                            const bmmc_pass_desc d, uint64_t blk0) {
    using C = TiledCfg<UL, T, 0, TL>;
    static_assert(C::J >= 2, "two passes per tile at least");
    constexpr int H = C::J / 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::TILE / 2];
    const LaneParts p = lane_parts<C, T>(d, threadIdx.x);
    const uint64_t blk = blk0 + blockIdx.x;

    dev::Chunk<C::CB> v[C::J];
    load_tile<C, T, NT>(v, in, tile_base<C>(d.in_blk, blk), d, p);
    stage_tile<C, T, 0, H>(lds, v, d, p);
    __syncthreads();
    const uint64_t obase = tile_base<C>(d.out_blk, blk) ^ d.out_c;
    const uint32_t rbase = tile_base<C>(d.lds_blk, blk) ^ d.lds_c;
    drain_tile<C, T, NT, 0, H>(out, lds, obase, rbase, d, p);
    __syncthreads();  // every read of the first half is done before it is overwritten
    stage_tile<C, T, H, C::J>(lds, v, d, p);
    __syncthreads();
    drain_tile<C, T, NT, H, C::J>(out, lds, obase, rbase, d, p);
}

// Persistent: 2^grid_log2 workgroups; workgroup w, as walker v =
// walker_index(w), walks 2^r tiles in Gray order, either its own block range
// (v * 2^r XOR gray(k)) or interleaved with the others
// (gray(k) * 2^grid_log2 XOR v), so consecutive tiles of a
// workgroup differ in one block bit and the wave-uniform bases change by one
// table entry each.  The LDS holds
// two tiles: while tile k is read back and stored, the loads of tile k+1 are
// already in flight.  One barrier per tile suffices: a buffer is rewritten
// two tiles later, after every thread has passed the barrier that follows
// its reads.
template <int UL, int T, bool NT, int TL>
__global__ void __launch_bounds__((TiledCfg<UL, T, 0, TL>::NT))
    bmmc_tiled_persistent_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                                 const bmmc_pass_desc d) {
    using C = TiledCfg<UL, T, 0, TL>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::TILE];
    const LaneParts p = lane_parts<C, T>(d, threadIdx.x);
    const int r = d.blk_bits - d.grid_log2;
    const bool interleaved = d.walk == BMMC_WALK_INTERLEAVED;
    const uint64_t walker = walker_index(blockIdx.x);
    const uint64_t first = interleaved ? walker : (walker << r);
    const int shift = interleaved ? d.grid_log2 : 0;  // the walked block bits start here
    const uint64_t count = uint64_t(1) << r;

    const uint64_t e_in = base_issue<C>(d.in_blk, first);
    const uint64_t e_out = base_issue<C>(d.out_blk, first);
    const uint32_t e_rd = base_issue<C>(d.lds_blk, first);
    __builtin_amdgcn_sched_barrier(0);
    uint64_t in_base = base_finish<C>(e_in, first);

    dev::Chunk<C::CB> v[C::J];
    load_tile<C, T, NT>(v, in, in_base, d, p);
    __builtin_amdgcn_sched_barrier(0);
    uint64_t out_base = base_finish<C>(e_out, first) ^ d.out_c;
    uint32_t rd_base = base_finish<C>(e_rd, first) ^ d.lds_c;
    // Every tile but the last refills the registers with the next tile's
    // loads before draining.  Loads and stores share one counter, which
    // completes in issue order; the staging wait can leave the previous
    // tile's stores in flight only if every path into it has the same
    // accesses outstanding, so the refill is unconditional and the first
    // tile is peeled (the loop is then always entered with one tile of loads
    // followed by one tile of stores).
    auto step = [&](uint64_t k) {
        uint8_t *buf = lds + (k & 1) * C::TILE;
        stage_tile<C, T>(buf, v, d, p);
        __syncthreads();
        const int bit = shift + __builtin_ctzll(k + 1);
        in_base ^= d.in_blk[bit];
        load_tile<C, T, NT>(v, in, in_base, d, p);
        __builtin_amdgcn_sched_barrier(0);
        drain_tile<C, T, NT>(out, buf, out_base, rd_base, d, p);
        out_base ^= d.out_blk[bit];
        rd_base ^= d.lds_blk[bit];
    };
    uint64_t k = 0;
    if (count > 1) {
        step(0);
        for (k = 1; k + 1 < count; ++k) step(k);
    }
    uint8_t *buf = lds + (k & 1) * C::TILE;
    stage_tile<C, T>(buf, v, d, p);
    __syncthreads();
    drain_tile<C, T, NT>(out, buf, out_base, rd_base, d, p);
}

// Streamed: the persistent walk with the waves split by role.  Waves of the
// first half only load tiles and stage them in LDS; waves of the second half
// only drain tiles and store them.  On gfx9-family GPUs loads and stores share
// one wait counter, so a wave that has stores in flight cannot wait for its
// loads alone; with one kind of access per wave every wait is exact, loads of
// tile k+1 stay in flight while tile k drains, and stores are never waited
// for.  One barrier per tile orders the halves: the loaders write buffer k&1
// before barrier k, the storers read it after barrier k and have finished
// before barrier k+1, after which the loaders may write it again (tile k+2).
// Launches of at most 2^kSmallBlkBits tiles (arrays of a few MiB) have a
// variant of the streamed kernel whose loader waves take their input base from
// that many table entries by scalar loads, issued with the kernel's other
// argument loads.  The wave's vector load of the table otherwise costs a memory
// round trip before the first tile load, which a pass of a few microseconds
// pays in full: measured on MI355X, a 4 MiB pass spent 0.41 us on it, and 0.08 us
// on the scalar form (0.19 us when the choice was a run-time branch).
constexpr int kSmallBlkBits = 8;

template <int UL, int T, int DEPTH, bool NT, bool SB, int TL>
__global__ void __launch_bounds__((2 * TiledCfg<UL, T, 0, TL>::NT))
    bmmc_tiled_streamed_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                               const bmmc_pass_desc d) {
    using C = TiledCfg<UL, T, 0, TL>;
    static_assert(DEPTH == 1 || DEPTH == 2, "tiles of loads in flight per loader wave");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::TILE];
    static_assert(C::NT >= 64, "each role must be whole waves");
    // The role is the same for every lane of a wave (NT is a multiple of 64);
    // reading it from the first lane tells the compiler so, which keeps the
    // loaders' running tile index in scalar registers.
    const bool loader = __builtin_amdgcn_readfirstlane((int)threadIdx.x) < C::NT;
    // each role computes only its own lane parts: fewer table loads per wave,
    // which the compiler can then issue together
    const uint32_t tid = threadIdx.x & (C::NT - 1);
    // small arrays: the loaders' table entries are read with the pass's own
    // parameters, before anything waits for either (one round trip in all)
    uint64_t blk[kSmallBlkBits], lin[C::NTL + C::JL];
    uint32_t llds[C::NTL];
    if constexpr (SB) {
#pragma unroll
        for (int k = 0; k < kSmallBlkBits; ++k) blk[k] = d.in_blk[k];
#pragma unroll
        for (int k = 0; k < C::NTL + C::JL; ++k) lin[k] = d.ld_in[k];
#pragma unroll
        for (int k = 0; k < C::NTL; ++k) llds[k] = d.ld_lds[k];
    }
    const int blk_bits = d.blk_bits, grid_log2 = d.grid_log2, walk = d.walk;
    if constexpr (SB) {
        // an empty asm that takes an XOR of every entry (and of the input
        // pointer) keeps the reads here,
        // where they wait together with the parameters' (the compiler would
        // otherwise sink them into the loaders' branch, behind that wait)
        uint64_t keep = (uint64_t)(uintptr_t)in;
#pragma unroll
        for (int k = 0; k < kSmallBlkBits; ++k) keep ^= blk[k];
#pragma unroll
        for (int k = 0; k < C::NTL + C::JL; ++k) keep ^= lin[k];
#pragma unroll
        for (int k = 0; k < C::NTL; ++k) keep ^= llds[k];
        asm volatile("" ::"s"(keep));
    }
    const int r = blk_bits - grid_log2;
    const bool interleaved = walk == BMMC_WALK_INTERLEAVED;
    const uint64_t walker = walker_index(blockIdx.x);
    const uint64_t first = interleaved ? walker : (walker << r);
    const int shift = interleaved ? grid_log2 : 0;
    const uint64_t count = uint64_t(1) << r;

    // Each role runs its own loop with exactly `count` barriers, so every
    // wave meets the same barriers; keeping the roles' code apart leaves each
    // loop straight-line, which lets the compiler wait for the oldest tile's
    // loads only (a shared loop body merges both roles' paths and its waits
    // fall back to "everything outstanding").
    if (loader) {
        LaneParts p;
        p.out_lane = 0;
        p.rd_lane = 0;
        // running input base of the last tile loaded (tiles are loaded in
        // walk order, DEPTH ahead of the one being staged)
        uint64_t in_base;
        uint64_t jo[C::J];  // small-array path: per-pass offsets of the first tile
        if constexpr (SB) {
            in_base = dev::xor_bits_lane<kSmallBlkBits>(blk, (uint32_t)first);
            p.in_lane = dev::xor_bits_lane<C::NTL>(lin, tid);
            p.wr_lane = dev::xor_bits_lane<C::NTL>(llds, tid);
#pragma unroll
            for (int j = 0; j < C::J; ++j)
                jo[j] = dev::xor_bits_lane<C::JL>(lin + C::NTL, (uint32_t)j);
        } else {
            p.in_lane = dev::xor_bits_lane<C::NTL>(d.ld_in, tid);
            p.wr_lane = dev::xor_bits_lane<C::NTL>(d.ld_lds, tid);
            in_base = base_finish<C>(base_issue<C>(d.in_blk, first), first);
        }
        uint64_t loaded = 0;  // tiles loaded so far
        dev::Chunk<C::CB> v[DEPTH][C::J];
        // next tile in walk order: one table entry per step (Gray code)
        auto advance = [&]() {
            in_base ^= d.in_blk[shift + __builtin_ctzll(loaded)];
            ++loaded;
        };
        if constexpr (SB)
            load_tile_jo<C, T, NT>(v[0], in, in_base, jo, p);
        else
            load_tile<C, T, NT>(v[0], in, in_base, d, p);
        loaded = 1;
        if (count == 1) {
            stage_tile<C, T>(lds, v[0], d, p);
            __syncthreads();
            return;
        }
        if constexpr (DEPTH == 2) {
            // tile 1's loads after tile 0's: waits count loads in issue order
            __builtin_amdgcn_sched_barrier(0);
            advance();
            load_tile<C, T, NT>(v[1], in, in_base, d, p);
        }
        // Steady state: every staged buffer is refilled DEPTH tiles ahead.
        // count is a power of two >= 2, so while k + DEPTH < count the DEPTH
        // tiles after k + DEPTH - 1 all exist and the refills need no
        // condition (a conditional refill would leave the compiler unsure how
        // many loads are outstanding, and it would then wait for all of them).
        uint64_t k = 0;
        for (; k + DEPTH < count; k += DEPTH) {
#pragma unroll
            for (int s = 0; s < DEPTH; ++s) {
                stage_tile<C, T>(lds + ((k + s) & 1) * C::TILE, v[s], d, p);
                __syncthreads();
                advance();
                load_tile<C, T, NT>(v[s], in, in_base, d, p);
                // keep the refill ahead of the next staging: staging waits
                // for the older tile only while the refill is in flight
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last DEPTH tiles: nothing left to load
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
            stage_tile<C, T>(lds + ((k + s) & 1) * C::TILE, v[s], d, p);
            __syncthreads();
        }
    } else {
        LaneParts p;
        p.in_lane = 0;
        p.wr_lane = 0;
        p.out_lane = dev::xor_bits_lane<C::NTL>(d.st_out, tid);
        p.rd_lane = dev::xor_bits_lane<C::NTL>(d.st_lds, tid);
        // running bases of the next tile to drain
        const uint64_t e_out = base_issue<C>(d.out_blk, first);
        const uint32_t e_rd = base_issue<C>(d.lds_blk, first);
        __builtin_amdgcn_sched_barrier(0);
        uint64_t out_base = base_finish<C>(e_out, first) ^ d.out_c;
        uint32_t rd_base = base_finish<C>(e_rd, first) ^ d.lds_c;
        for (uint64_t k = 0; k < count; ++k) {
            __syncthreads();
            drain_tile<C, T, NT>(out, lds + (k & 1) * C::TILE, out_base, rd_base, d, p);
            if (k + 1 < count) {
                const int bit = shift + __builtin_ctzll(k + 1);
                out_base ^= d.out_blk[bit];
                rd_base ^= d.lds_blk[bit];
            }
        }
    }
}

namespace {

struct TiledArgs {
    const bmmc_pass_desc *d;
    const uint8_t *in;
    uint8_t *out;
    hipStream_t s;
};

template <int UL, int T, int IT, bool NT, int TL> int launch_nt(const TiledArgs &a) {
    using C = TiledCfg<UL, T, IT, TL>;
    if (a.d->launch == BMMC_LAUNCH_STREAMED) {
        if constexpr (IT == 0 && 2 * C::TILE <= 131072 && C::NT >= 64 && 2 * C::NT <= 1024) {
            const dim3 grid(1u << a.d->grid_log2), block(2 * C::NT);
            const bool small = a.d->blk_bits <= kSmallBlkBits;
            if (a.d->depth == 2) {
                if (small)
                    hipLaunchKernelGGL((bmmc_tiled_streamed_kernel<UL, T, 2, NT, true, TL>), grid,
                                       block, 0, a.s, a.in, a.out, *a.d);
                else
                    hipLaunchKernelGGL((bmmc_tiled_streamed_kernel<UL, T, 2, NT, false, TL>), grid,
                                       block, 0, a.s, a.in, a.out, *a.d);
            } else {
                if (small)
                    hipLaunchKernelGGL((bmmc_tiled_streamed_kernel<UL, T, 1, NT, true, TL>), grid,
                                       block, 0, a.s, a.in, a.out, *a.d);
                else
                    hipLaunchKernelGGL((bmmc_tiled_streamed_kernel<UL, T, 1, NT, false, TL>), grid,
                                       block, 0, a.s, a.in, a.out, *a.d);
            }
            return hipGetLastError() == hipSuccess ? BMMC_OK : BMMC_ERR_HIP;
        } else {
            return BMMC_ERR_UNSUPPORTED;
        }
    }
    if (a.d->launch == BMMC_LAUNCH_PERSISTENT) {
        if constexpr (IT == 0 && 2 * C::TILE <= 131072) {
            hipLaunchKernelGGL((bmmc_tiled_persistent_kernel<UL, T, NT, TL>),
                               dim3(1u << a.d->grid_log2), dim3(C::NT), 0, a.s, a.in, a.out,
                               *a.d);
            return hipGetLastError() == hipSuccess ? BMMC_OK : BMMC_ERR_HIP;
        } else {
            return BMMC_ERR_UNSUPPORTED;
        }
    }
    if (a.d->buffer_loads) {
        if constexpr (IT == 0 && UL >= 2) {
            const uint64_t blocks = uint64_t(1) << a.d->blk_bits;
            const uint64_t per = max_blocks_per_launch(C::NT);
            for (uint64_t b0 = 0; b0 < blocks; b0 += per) {
                const uint64_t nb = blocks - b0 < per ? blocks - b0 : per;
                hipLaunchKernelGGL((bmmc_tiled_bufload_kernel<UL, T, NT, TL>),
                                   dim3((uint32_t)nb), dim3(C::NT), 0, a.s, a.in, a.out, *a.d,
                                   b0);
            }
            return hipGetLastError() == hipSuccess ? BMMC_OK : BMMC_ERR_HIP;
        } else {
            return BMMC_ERR_UNSUPPORTED;
        }
    }
    if (a.d->split_stage) {
        if constexpr (IT == 0 && C::J >= 2) {
            const uint64_t blocks = uint64_t(1) << a.d->blk_bits;
            const uint64_t per = max_blocks_per_launch(C::NT);
            for (uint64_t b0 = 0; b0 < blocks; b0 += per) {
                const uint64_t nb = blocks - b0 < per ? blocks - b0 : per;
                hipLaunchKernelGGL((bmmc_tiled_split_kernel<UL, T, NT, TL>), dim3((uint32_t)nb),
                                   dim3(C::NT), 0, a.s, a.in, a.out, *a.d, b0);
            }
            return hipGetLastError() == hipSuccess ? BMMC_OK : BMMC_ERR_HIP;
        } else {
            return BMMC_ERR_UNSUPPORTED;
        }
    }
    const uint64_t blocks = uint64_t(1) << (a.d->blk_bits - IT);
    const uint64_t per = max_blocks_per_launch(C::NT);
    for (uint64_t b0 = 0; b0 < blocks; b0 += per) {
        const uint64_t nb = blocks - b0 < per ? blocks - b0 : per;
        hipLaunchKernelGGL((bmmc_tiled_kernel<UL, T, IT, NT, TL>), dim3((uint32_t)nb), dim3(C::NT),
                           0, a.s, a.in, a.out, *a.d, b0);
    }
    return hipGetLastError() == hipSuccess ? BMMC_OK : BMMC_ERR_HIP;
}

// cache_hint 3: non-temporal loads and stores; 0: plain.
template <int UL, int T, int IT, int TL> int launch_hint(const TiledArgs &a) {
    return a.d->cache_hint ? launch_nt<UL, T, IT, true, TL>(a)
                           : launch_nt<UL, T, IT, false, TL>(a);
}

// threads_log2 picks the 256- or 512-thread instantiation; the wide one is
// compiled only where a tile has more than 256 chunks and for one tile per
// workgroup (the iterated variant keeps 256).
template <int UL, int T, int IT> int launch_one(const TiledArgs &a) {
    constexpr int narrow = tile_threads_log2(UL, T, kTileMaxNTL);
    if constexpr (IT == 0 && tile_threads_log2(UL, T, kTileWideNTL) > narrow) {
        if (a.d->threads_log2 == tile_threads_log2(UL, T, kTileWideNTL))
            return launch_hint<UL, T, IT, kTileWideNTL>(a);
    }
    if (a.d->threads_log2 != narrow) return BMMC_ERR_UNSUPPORTED;
    return launch_hint<UL, T, IT, kTileMaxNTL>(a);
}

// Walks the compiled (UL, T, IT) space; `launch` = false only answers
// whether the configuration exists.
template <int UL, int T, int IT>
int dispatch(int ul, int t, int it, const TiledArgs *a) {
    if constexpr (UL > 4) {
        return BMMC_ERR_UNSUPPORTED;
    } else if constexpr (T > kMaxT[UL]) {
        return dispatch<UL + 1, 1, 0>(ul, t, it, a);
    } else if constexpr (IT > kMaxIT || !valid_cfg<UL, T, IT>()) {
        return dispatch<UL, T + 1, 0>(ul, t, it, a);
    } else {
        if (ul == UL && t == T && it == IT) return a ? launch_one<UL, T, IT>(*a) : BMMC_OK;
        return dispatch<UL, T, IT + 1>(ul, t, it, a);
    }
}

}  // namespace

int launch_tiled(const bmmc_pass_desc &d, const void *in, void *out, hipStream_t s) {
    if (d.iters_log2 > d.blk_bits || d.grid_log2 > d.blk_bits || d.grid_log2 < 0)
        return BMMC_ERR_INVALID_ARG;
    if (d.launch != BMMC_LAUNCH_PERSISTENT && d.launch != BMMC_LAUNCH_ONE_TILE &&
        d.launch != BMMC_LAUNCH_STREAMED)
        return BMMC_ERR_INVALID_ARG;
    if (d.launch != BMMC_LAUNCH_ONE_TILE && d.walk != BMMC_WALK_RANGES &&
        d.walk != BMMC_WALK_INTERLEAVED)
        return BMMC_ERR_INVALID_ARG;
    if (d.cache_hint != 0 && d.cache_hint != 3) return BMMC_ERR_UNSUPPORTED;
    if (d.split_stage != 0 &&
        (d.split_stage != 1 || d.launch != BMMC_LAUNCH_ONE_TILE || d.iters_log2 != 0))
        return BMMC_ERR_INVALID_ARG;
    if (d.buffer_loads != 0 &&
        (d.buffer_loads != 1 || d.launch != BMMC_LAUNCH_ONE_TILE || d.iters_log2 != 0 ||
         d.split_stage != 0 || d.unit_log2 < 2 || d.nbits + d.unit_log2 > kBufferLoadMaxLog2))
        return BMMC_ERR_INVALID_ARG;
    TiledArgs a{&d, static_cast<const uint8_t *>(in), static_cast<uint8_t *>(out), s};
    return dispatch<0, 1, 0>(d.unit_log2, d.t, d.iters_log2, &a);
}

}  // namespace bmmc
