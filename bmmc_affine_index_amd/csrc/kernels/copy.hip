// copy.hip -- the ceiling: an identity-order copy with the permutation
// kernels' vector width and launch shape ("A kernel that is correct": a copy
// moves the same bytes as a transpose in the easiest order, and its measured
// bandwidth, not the datasheet's, is the ceiling to compare against).
#include "../launch.h"
#include "common.h"

namespace bmmc {

constexpr int kCopyNTL = 8;  // 256 threads

// Non-temporal loads and stores: the data is streamed once.  Measured on
// MI355X with buffers rotating over 2 GiB (GB/s of bytes read + written,
// three runs each agreeing within 1%):
//   bytes   one-shot, 1 x 16 B/lane   grid-stride, 2048 groups, 4 x 16 B/lane
//   4 MiB        2976                      2700
//   8 MiB        4300                      4070
//   16 MiB       4590                      5620
//   32 MiB       5160                      5290
//   64 MiB       5770                      5865
//   128 MiB      6160                      6100
//   1 GiB        6491                      5897
// and the hints add 5-15% over plain loads and stores from 4 MiB up.  At
// 32 MiB a one-shot launch with 4 x 16 B per lane measured 5560, faster than
// the grid-stride loop's one trip over the same 2048 workgroups (the reason is
// not known); arrays in (16 MiB, 32 MiB] take that launch.
template <int CPTL>
__global__ void __launch_bounds__(1 << kCopyNTL)
    bmmc_copy_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out, uint64_t n16,
                     uint64_t blk0) {
    constexpr int CPT = 1 << CPTL;
    const uint64_t first = ((blk0 + blockIdx.x) << (kCopyNTL + CPTL)) + threadIdx.x;
    dev::Chunk<16> v[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const uint64_t x = first + ((uint64_t)k << kCopyNTL);
        if (x < n16) v[k] = dev::gload_nt<16, true>(in + x * 16);
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const uint64_t x = first + ((uint64_t)k << kCopyNTL);
        if (x < n16) dev::gstore_nt<16, true>(out + x * 16, v[k]);
    }
}

template <int CPTL>
__global__ void __launch_bounds__(1 << kCopyNTL)
    bmmc_copy_stride_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                            uint64_t n16) {
    constexpr int CPT = 1 << CPTL;
    const uint64_t step = (uint64_t)gridDim.x << (kCopyNTL + CPTL);
    for (uint64_t base = ((uint64_t)blockIdx.x << (kCopyNTL + CPTL)) + threadIdx.x;
         base < n16; base += step) {
        dev::Chunk<16> v[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const uint64_t x = base + ((uint64_t)k << kCopyNTL);
            if (x < n16) v[k] = dev::gload_nt<16, true>(in + x * 16);
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const uint64_t x = base + ((uint64_t)k << kCopyNTL);
            if (x < n16) dev::gstore_nt<16, true>(out + x * 16, v[k]);
        }
    }
}

// the one-shot form with 4 x 16 B per lane serves (kCopyWideMinBytes,
// kCopyWideMaxBytes], the grid-stride form the rest of
// (kCopyStrideMinBytes, kCopyStrideMaxBytes]
constexpr uint64_t kCopyWideMinBytes = uint64_t(16) << 20;
constexpr uint64_t kCopyWideMaxBytes = uint64_t(32) << 20;
constexpr int kCopyWideCPTL = 2;
constexpr uint64_t kCopyStrideMinBytes = uint64_t(8) << 20;
constexpr uint64_t kCopyStrideMaxBytes = uint64_t(64) << 20;
constexpr int kCopyStrideCPTL = 2;
constexpr uint32_t kCopyStrideBlocks = 2048;  // 8 per compute unit on a 256-CU MI355X

// Bytes that do not fill a 16-byte vector, or unaligned buffers.
__global__ void __launch_bounds__(256)
    bmmc_copy_bytes_kernel(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                           uint64_t nbytes, uint64_t blk0) {
    const uint64_t x = (blk0 + blockIdx.x) * 256u + threadIdx.x;
    if (x < nbytes) out[x] = in[x];
}

int launch_copy(const void *in_v, void *out_v, size_t nbytes, hipStream_t s) {
    const uint8_t *in = static_cast<const uint8_t *>(in_v);
    uint8_t *out = static_cast<uint8_t *>(out_v);
    const bool aligned = (((uintptr_t)in | (uintptr_t)out) & 15u) == 0;
    uint64_t done = 0;
    if (aligned) {
        const uint64_t n16 = nbytes / 16;
        if (nbytes > kCopyWideMinBytes && nbytes <= kCopyWideMaxBytes) {
            const uint64_t per = uint64_t(1) << (kCopyNTL + kCopyWideCPTL);
            const uint64_t blocks = (n16 + per - 1) / per;  // at most 2048
            hipLaunchKernelGGL(bmmc_copy_kernel<kCopyWideCPTL>, dim3((uint32_t)blocks),
                               dim3(1 << kCopyNTL), 0, s, in, out, n16, uint64_t(0));
        } else if (nbytes > kCopyStrideMinBytes && nbytes <= kCopyStrideMaxBytes) {
            const uint64_t per = uint64_t(1) << (kCopyNTL + kCopyStrideCPTL);
            const uint64_t blocks = (n16 + per - 1) / per;
            const uint32_t g = blocks < kCopyStrideBlocks ? (uint32_t)blocks : kCopyStrideBlocks;
            hipLaunchKernelGGL(bmmc_copy_stride_kernel<kCopyStrideCPTL>, dim3(g),
                               dim3(1 << kCopyNTL), 0, s, in, out, n16);
        } else {
            const uint64_t blocks = (n16 + (1u << kCopyNTL) - 1) >> kCopyNTL;
            const uint64_t per = max_blocks_per_launch(1u << kCopyNTL);
            for (uint64_t b0 = 0; b0 < blocks; b0 += per) {
                const uint64_t nb = blocks - b0 < per ? blocks - b0 : per;
                hipLaunchKernelGGL(bmmc_copy_kernel<0>, dim3((uint32_t)nb), dim3(1 << kCopyNTL),
                                   0, s, in, out, n16, b0);
            }
        }
        done = n16 * 16;
    }
    const uint64_t rest = nbytes - done;
    if (rest) {
        const uint64_t blocks = (rest + 255) / 256;
        const uint64_t per = max_blocks_per_launch(256);
        for (uint64_t b0 = 0; b0 < blocks; b0 += per) {
            const uint64_t nb = blocks - b0 < per ? blocks - b0 : per;
            hipLaunchKernelGGL(bmmc_copy_bytes_kernel, dim3((uint32_t)nb), dim3(256), 0, s,
                               in + done, out + done, rest, b0);
        }
    }
    return hipGetLastError() == hipSuccess ? BMMC_OK : BMMC_ERR_HIP;
}

}  // namespace bmmc
