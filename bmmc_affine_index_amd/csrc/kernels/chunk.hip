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

template <int UL, int WL, bool NT, bool GATHER>
__global__ void __launch_bounds__(1 << kChunkNTL)
    bmmc_chunk_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                      const bmmc_pass_desc d, uint64_t blk0) {
    constexpr int U = 1 << UL;
    constexpr int W = 1 << WL;
    constexpr int CB = U << WL;
    constexpr int CPT = 1 << kChunkCPTL;
    const uint32_t tid = threadIdx.x;
    const uint64_t nchunks = uint64_t(1) << d.blk_bits;
    const uint64_t first = (blk0 + blockIdx.x) << (kChunkNTL + kChunkCPTL);
    const uint64_t *tab = GATHER ? d.in_blk : d.out_blk;
    const uint64_t lane_off = dev::xor_bits_lane<kChunkNTL>(tab, tid);
    // A gather needs the wave-uniform part of each group's source offset
    // before its loads: the whole wave computes it (lane k loads entry k, a
    // wave XOR reduction keeps the entries of the set bits; the bits of xu
    // below kChunkNTL are 0), one vector load instead of a chain of scalar
    // loads, with every lane active, before the guard on the array's end
    // (measured on MI355X: a 4 MiB block permutation +7%).  A scatter
    // computes its output base from scalar loads after issuing its loads,
    // which hides them (the wave form cost a 4 MiB reversal 10%).
    uint64_t ubase[CPT] = {};
    if constexpr (GATHER) {
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
        if (d.kernel == BMMC_KERNEL_CHUNK)
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
