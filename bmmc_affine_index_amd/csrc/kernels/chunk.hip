// chunk.hip -- passes that move whole chunks without LDS (gfx950).
//
// Three users:
//  * chunk passes (a gather): the segment relabel of a two-pass plan and
//    maps that move whole segments.
//    Chunks of up to 16 bytes move as units and the complement's low bits
//    permute the units inside a chunk ("Efficient GPU Implementation of
//    Affine Index Permutations on Arrays", introduction: the first of the
//    two tiled factors is applied first; its factor T2 here keeps every
//    2^t-unit segment contiguous).  Each lane writes output chunks in order
//    and reads its source at A^-1.(y XOR c): measured on MI355X, reading
//    scattered pieces of 128 bytes or more costs nothing against a copy,
//    while scattered writes cost 11-15% at any piece size;
//  * chunk scatters: complement-only maps (A = I, c != 0), read in order and
//    stored at permuted places; gathered, each wave would read its chunks in
//    descending order, which measured 10% slower than descending stores;
//  * the naive pass (a scatter), with one-unit chunks: each lane reads
//    consecutive input and stores to A.i XOR c (the appendix's naive
//    bit-reversal kernel computes the output address from the input address
//    the same way; one-unit reads could not be gathered efficiently).
//
// The offset of the permuted side is XOR over the set bits of the chunk
// index of a table (in_blk for the gather, out_blk for the scatter) XOR a
// constant: the lane's low 8 bits are folded once per thread, the rest is
// wave-uniform.
#include "../launch.h"
#include "common.h"

namespace bmmc {

constexpr int kChunkNTL = 8;  // 256 threads
// One chunk per thread: measured against two and four per thread on array
// reversal, block permutations and the segment relabel, it is 4-33% faster
// (more, smaller workgroups; the copy ceiling behaves the same way).
constexpr int kChunkCPTL = 0;

// Gathers of at most 2^(kChunkNTL + kSmallChunkBlkBits) chunks (16 MiB of
// 16-byte chunks) have a variant that takes the workgroup's source base from
// scalar loads of the table entries above the lane bits, all issued with the
// pass's other parameters and then selected by the workgroup's index bits, so
// that the data loads wait for one round trip in all (as the copy's do).  The
// wave's vector load of the table costs a second round trip, which a pass of
// a few microseconds pays in full.
constexpr int kSmallChunkBlkBits = 12;

template <int UL, int WL, bool NT, bool GATHER, bool SB = false>
__global__ void __launch_bounds__(1 << kChunkNTL)
    bmmc_chunk_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                      const bmmc_pass_desc d, uint64_t blk0) {
    constexpr int U = 1 << UL;
    constexpr int W = 1 << WL;
    constexpr int CB = U << WL;
    constexpr int CPT = 1 << kChunkCPTL;
    static_assert(!SB || GATHER, "the scalar form serves gathers");
    const uint32_t tid = threadIdx.x;
    const uint64_t nchunks = uint64_t(1) << d.blk_bits;
    const uint64_t *tab = GATHER ? d.in_blk : d.out_blk;
    uint64_t b0 = blk0;
    uint64_t e[SB ? kSmallChunkBlkBits : 1];
    if constexpr (SB) {
#pragma unroll
        for (int k = 0; k < kSmallChunkBlkBits; ++k) e[k] = d.in_blk[kChunkNTL + k];
        // An empty asm that takes every entry, the lane bits' entries and the
        // input pointer keeps their loads here, where they wait together with
        // the parameters'; blk0 passes through it, so that nothing computed
        // from it is scheduled between the loads (the compiler would otherwise
        // wait for the first loads before issuing the rest, or issue the lane
        // bits' loads behind the guard on the array's end: a second round
        // trip either way).
        static_assert(kSmallChunkBlkBits == 12 && kChunkNTL == 8, "operand list below");
        asm volatile(""
                     : "+s"(b0)
                     : "s"(e[0]), "s"(e[1]), "s"(e[2]), "s"(e[3]), "s"(e[4]), "s"(e[5]),
                       "s"(e[6]), "s"(e[7]), "s"(e[8]), "s"(e[9]), "s"(e[10]), "s"(e[11]),
                       "s"(tab[0]), "s"(tab[1]), "s"(tab[2]), "s"(tab[3]), "s"(tab[4]),
                       "s"(tab[5]), "s"(tab[6]), "s"(tab[7]), "s"(in), "s"(d.in_c),
                       "s"(d.blk_bits));
    }
    const uint64_t first = (b0 + blockIdx.x) << (kChunkNTL + kChunkCPTL);
    const uint64_t lane_off = dev::xor_bits_lane<kChunkNTL>(tab, tid);
    // A gather needs the wave-uniform part of each group's source offset
    // before its loads.  Past the scalar form's size the whole wave computes
    // it (lane k loads entry k, a wave XOR reduction keeps the entries of the
    // set bits; the bits of xu below kChunkNTL are 0), one vector load instead
    // of a chain of dependent scalar loads, with every lane active, before the
    // guard on the array's end (measured on MI355X against that chain: a 4 MiB
    // block permutation +7%).  A scatter
    // computes its output base from scalar loads after issuing its loads,
    // which hides them (the wave form cost a 4 MiB reversal 10%).
    uint64_t ubase[CPT] = {};
    if constexpr (SB) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const uint64_t xu = (first + ((uint64_t)k << kChunkNTL)) >> kChunkNTL;
            uint64_t acc = d.in_c;
#pragma unroll
            for (int b = 0; b < kSmallChunkBlkBits; ++b) acc ^= ((xu >> b) & 1u) ? e[b] : 0;
            ubase[k] = acc;
        }
    } else if constexpr (GATHER) {
        const uint64_t entry = dev::wave_load(tab);
#pragma unroll
        for (int k = 0; k < CPT; ++k)
            ubase[k] = dev::wave_select_xor(entry, first + ((uint64_t)k << kChunkNTL)) ^ d.in_c;
    }

    dev::Chunk<CB> v[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const uint64_t xu = first + ((uint64_t)k << kChunkNTL);
        const uint64_t x = xu + tid;
        if (x >= nchunks) continue;
        const uint64_t src = GATHER ? (ubase[k] ^ lane_off) : x * CB;
        v[k] = dev::gload_nt<CB, NT>(in + src);
    }
    const uint32_t ux = (uint32_t)d.unit_xor;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const uint64_t xu = first + ((uint64_t)k << kChunkNTL);
        const uint64_t x = xu + tid;
        if (x >= nchunks) continue;
        dev::Chunk<CB> c = v[k];
        if constexpr (WL > 0) {
            // unit e of the output chunk is unit e XOR ux of the input chunk:
            // one butterfly stage per set bit of ux (ux is wave-uniform)
#pragma unroll
            for (int b = 0; b < WL; ++b) {
                if ((ux >> b) & 1u) {
                    dev::Chunk<CB> r;
                    dev::zero(r);
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        dev::put_unit<CB, U>(r, e, dev::get_unit<CB, U>(c, e ^ (1 << b)));
                    c = r;
                }
            }
        }
        const uint64_t dst =
            GATHER ? x * CB : (dev::xor_bits_uniform(d.out_blk, xu) ^ lane_off ^ d.out_c);
        dev::gstore_nt<CB, NT>(out + dst, c);
    }
}

namespace {

template <int UL, int WL>
int launch_chunk_t(const bmmc_pass_desc &d, const uint8_t *in, uint8_t *out, hipStream_t s) {
    const uint64_t nchunks = uint64_t(1) << d.blk_bits;
    const uint64_t per_block = uint64_t(1) << (kChunkNTL + kChunkCPTL);
    const uint64_t blocks = (nchunks + per_block - 1) / per_block;
    const uint64_t per = max_blocks_per_launch(1u << kChunkNTL);
    for (uint64_t b0 = 0; b0 < blocks; b0 += per) {
        const uint64_t nb = blocks - b0 < per ? blocks - b0 : per;
        // chunk passes gather, chunk scatters scatter, both with non-temporal
        // hints; the naive pass scatters with plain accesses
        if (d.kernel == BMMC_KERNEL_CHUNK && d.blk_bits <= kChunkNTL + kSmallChunkBlkBits)
            hipLaunchKernelGGL((bmmc_chunk_kernel<UL, WL, true, true, true>), dim3((uint32_t)nb),
                               dim3(1 << kChunkNTL), 0, s, in, out, d, b0);
        else if (d.kernel == BMMC_KERNEL_CHUNK)
            hipLaunchKernelGGL((bmmc_chunk_kernel<UL, WL, true, true>), dim3((uint32_t)nb),
                               dim3(1 << kChunkNTL), 0, s, in, out, d, b0);
        else if (d.kernel == BMMC_KERNEL_CHUNK_SCATTER)
            hipLaunchKernelGGL((bmmc_chunk_kernel<UL, WL, true, false>), dim3((uint32_t)nb),
                               dim3(1 << kChunkNTL), 0, s, in, out, d, b0);
        else
            hipLaunchKernelGGL((bmmc_chunk_kernel<UL, WL, false, false>), dim3((uint32_t)nb),
                               dim3(1 << kChunkNTL), 0, s, in, out, d, b0);
    }
    return hipGetLastError() == hipSuccess ? BMMC_OK : BMMC_ERR_HIP;
}

template <int UL, int WL>
int dispatch_chunk(int ul, int wl, const bmmc_pass_desc &d, const uint8_t *in, uint8_t *out,
                   hipStream_t s) {
    if constexpr (UL > 4) {
        return BMMC_ERR_UNSUPPORTED;
    } else if constexpr (UL + WL > 4) {
        return dispatch_chunk<UL + 1, 0>(ul, wl, d, in, out, s);
    } else {
        if (ul == UL && wl == WL) return launch_chunk_t<UL, WL>(d, in, out, s);
        return dispatch_chunk<UL, WL + 1>(ul, wl, d, in, out, s);
    }
}

}  // namespace

int launch_chunk(const bmmc_pass_desc &d, const void *in, void *out, hipStream_t s) {
    // chunk passes are built with hints (3), naive passes without (0)
    if (d.cache_hint != (d.kernel == BMMC_KERNEL_NAIVE ? 0 : 3)) return BMMC_ERR_UNSUPPORTED;
    return dispatch_chunk<0, 0>(d.unit_log2, d.chunk_log2, d, static_cast<const uint8_t *>(in),
                                static_cast<uint8_t *>(out), s);
}

}  // namespace bmmc
