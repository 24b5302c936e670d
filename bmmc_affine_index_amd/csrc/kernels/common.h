// common.h -- device helpers shared by the permutation kernels (gfx950).
//
// Data is moved as opaque "chunks" of 1..16 bytes: one global load or store
// per lane per chunk (dwordx4 for 16-byte chunks).  A chunk holds 2^wl units;
// the tile kernel reads units back from LDS one at a time and reassembles a
// chunk in output order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/bmmc.h"

namespace bmmc {
namespace dev {

template <int BYTES> struct Chunk;
template <> struct Chunk<16> { uint32_t w[4]; };
template <> struct Chunk<8> { uint32_t w[2]; };
template <> struct Chunk<4> { uint32_t w[1]; };
template <> struct Chunk<2> { uint16_t h; };
template <> struct Chunk<1> { uint8_t b; };

template <int BYTES> struct Unit;
template <> struct Unit<16> { uint32_t w[4]; };
template <> struct Unit<8> { uint32_t w[2]; };
template <> struct Unit<4> { uint32_t w[1]; };
template <> struct Unit<2> { uint16_t h; };
template <> struct Unit<1> { uint8_t b; };

// ---- global memory ------------------------------------------------------
template <int BYTES> __device__ __forceinline__ Chunk<BYTES> gload(const uint8_t *p);
template <> __device__ __forceinline__ Chunk<16> gload<16>(const uint8_t *p) {
    uint4 v = *reinterpret_cast<const uint4 *>(p);
    return Chunk<16>{{v.x, v.y, v.z, v.w}};
}
template <> __device__ __forceinline__ Chunk<8> gload<8>(const uint8_t *p) {
    uint2 v = *reinterpret_cast<const uint2 *>(p);
    return Chunk<8>{{v.x, v.y}};
}
template <> __device__ __forceinline__ Chunk<4> gload<4>(const uint8_t *p) {
    return Chunk<4>{{*reinterpret_cast<const uint32_t *>(p)}};
}
template <> __device__ __forceinline__ Chunk<2> gload<2>(const uint8_t *p) {
    return Chunk<2>{*reinterpret_cast<const uint16_t *>(p)};
}
template <> __device__ __forceinline__ Chunk<1> gload<1>(const uint8_t *p) {
    return Chunk<1>{*p};
}

template <int BYTES> __device__ __forceinline__ void gstore(uint8_t *p, const Chunk<BYTES> &c);
template <> __device__ __forceinline__ void gstore<16>(uint8_t *p, const Chunk<16> &c) {
    *reinterpret_cast<uint4 *>(p) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
}
template <> __device__ __forceinline__ void gstore<8>(uint8_t *p, const Chunk<8> &c) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(c.w[0], c.w[1]);
}
template <> __device__ __forceinline__ void gstore<4>(uint8_t *p, const Chunk<4> &c) {
    *reinterpret_cast<uint32_t *>(p) = c.w[0];
}
template <> __device__ __forceinline__ void gstore<2>(uint8_t *p, const Chunk<2> &c) {
    *reinterpret_cast<uint16_t *>(p) = c.h;
}
template <> __device__ __forceinline__ void gstore<1>(uint8_t *p, const Chunk<1> &c) {
    *p = c.b;
}

// Non-temporal variants (streaming data: no reuse expected in the caches).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));

// NT is a template parameter: the cache policy is an immediate of the
// instruction, and a run-time choice would put every access under a branch,
// which forces the compiler's memory-counter waits down to zero at the joins.
template <int BYTES, bool NT>
__device__ __forceinline__ Chunk<BYTES> gload_nt(const uint8_t *p) {
    if constexpr (NT && BYTES == 16) {
        nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(p));
        return Chunk<16>{{v.x, v.y, v.z, v.w}};
    } else if constexpr (NT && BYTES == 8) {
        nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2 *>(p));
        return Chunk<8>{{v.x, v.y}};
    } else if constexpr (NT && BYTES == 4) {
        return Chunk<4>{{__builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p))}};
    } else {
        return gload<BYTES>(p);
    }
}

template <int BYTES, bool NT>
__device__ __forceinline__ void gstore_nt(uint8_t *p, const Chunk<BYTES> &c) {
    if constexpr (NT && BYTES == 16) {
        nt_u32x4 v = {c.w[0], c.w[1], c.w[2], c.w[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4 *>(p));
    } else if constexpr (NT && BYTES == 8) {
        nt_u32x2 v = {c.w[0], c.w[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x2 *>(p));
    } else if constexpr (NT && BYTES == 4) {
        __builtin_nontemporal_store(c.w[0], reinterpret_cast<uint32_t *>(p));
    } else {
        gstore<BYTES>(p, c);
    }
}

// Buffer loads: the base address and the byte size of the array sit in a
// four-dword resource in scalar registers, and each lane supplies only a
// 32-bit byte offset.  Word 3 of the resource: raw (untyped) access with the
// 32-bit data format, stride 0, so the size field counts bytes and a load
// past it returns zero instead of touching memory.
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const uint8_t *base,
                                                              uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, (int)bytes,
                                             kBufferRsrcWord3);
}

// One chunk of 4, 8 or 16 bytes at byte offset `off`, with the non-temporal
// policy when NT (the operand is an immediate of the instruction).
template <int BYTES, bool NT>
__device__ __forceinline__ Chunk<BYTES> bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    constexpr int kPolicy = NT ? 2 : 0;  // the nt bit of the cache-policy operand
    if constexpr (BYTES == 16) {
        const nt_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicy);
        return Chunk<16>{{v.x, v.y, v.z, v.w}};
    } else if constexpr (BYTES == 8) {
        const nt_u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicy);
        return Chunk<8>{{v.x, v.y}};
    } else {
        static_assert(BYTES == 4, "buffer loads move chunks of 4, 8 or 16 bytes");
        return Chunk<4>{{__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicy)}};
    }
}

// ---- LDS ----------------------------------------------------------------
template <int BYTES> __device__ __forceinline__ void lds_store(uint8_t *p, const Chunk<BYTES> &c) {
    if constexpr (BYTES == 16)
        *reinterpret_cast<uint4 *>(p) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
    else if constexpr (BYTES == 8)
        *reinterpret_cast<uint2 *>(p) = make_uint2(c.w[0], c.w[1]);
    else if constexpr (BYTES == 4)
        *reinterpret_cast<uint32_t *>(p) = c.w[0];
    else if constexpr (BYTES == 2)
        *reinterpret_cast<uint16_t *>(p) = c.h;
    else
        *p = c.b;
}

template <int U> __device__ __forceinline__ Unit<U> lds_load_unit(const uint8_t *p) {
    if constexpr (U == 16) {
        uint4 v = *reinterpret_cast<const uint4 *>(p);
        return Unit<16>{{v.x, v.y, v.z, v.w}};
    } else if constexpr (U == 8) {
        uint2 v = *reinterpret_cast<const uint2 *>(p);
        return Unit<8>{{v.x, v.y}};
    } else if constexpr (U == 4) {
        return Unit<4>{{*reinterpret_cast<const uint32_t *>(p)}};
    } else if constexpr (U == 2) {
        return Unit<2>{*reinterpret_cast<const uint16_t *>(p)};
    } else {
        return Unit<1>{*p};
    }
}

// Place unit number e (0 <= e < CB/U) of a chunk.  The chunk must start
// zeroed when units are narrower than a dword.
template <int CB, int U>
__device__ __forceinline__ void put_unit(Chunk<CB> &c, int e, const Unit<U> &u) {
    if constexpr (U >= 4) {
#pragma unroll
        for (int i = 0; i < U / 4; ++i) c.w[e * (U / 4) + i] = u.w[i];
    } else if constexpr (CB >= 4) {
        const int byte = e * U;
        uint32_t v;
        if constexpr (U == 2) v = (uint32_t)u.h;
        else v = (uint32_t)u.b;
        c.w[byte / 4] |= v << (8 * (byte % 4));
    } else if constexpr (CB == 2) {
        // U == 1, two bytes
        c.h |= (uint16_t)((uint32_t)u.b << (8 * e));
    } else {
        c.b = u.b;
    }
}

template <int CB, int U>
__device__ __forceinline__ Unit<U> get_unit(const Chunk<CB> &c, int e) {
    if constexpr (U >= 4) {
        Unit<U> u;
#pragma unroll
        for (int i = 0; i < U / 4; ++i) u.w[i] = c.w[e * (U / 4) + i];
        return u;
    } else if constexpr (CB >= 4) {
        const int byte = e * U;
        uint32_t v = c.w[byte / 4] >> (8 * (byte % 4));
        if constexpr (U == 2) return Unit<2>{(uint16_t)v};
        else return Unit<1>{(uint8_t)v};
    } else if constexpr (CB == 2) {
        return Unit<1>{(uint8_t)(c.h >> (8 * e))};
    } else {
        return Unit<1>{c.b};
    }
}

template <int CB> __device__ __forceinline__ void zero(Chunk<CB> &c) {
    if constexpr (CB >= 4) {
#pragma unroll
        for (int i = 0; i < CB / 4; ++i) c.w[i] = 0;
    } else if constexpr (CB == 2) {
        c.h = 0;
    } else {
        c.b = 0;
    }
}

// XOR of the table entries selected by the set bits of a wave-uniform value.
template <typename T>
__device__ __forceinline__ T xor_bits_uniform(const T *tab, uint64_t v) {
    T acc = 0;
    while (v) {
        int k = __builtin_ctzll(v);
        v &= v - 1;
        acc ^= tab[k];
    }
    return acc;
}

// XOR over the 64 lanes of a wave (every lane must be active); the result is
// the same in every lane.  Row-wise inclusive XOR scan with DPP shifts of 1,
// 2, 4 and 8 (invalid sources read as 0), then the row totals are carried
// across rows with the row_bcast:15 and row_bcast:31 patterns; lane 63 then
// holds the total.
__device__ __forceinline__ uint32_t wave_xor_u32(uint32_t v) {
    v ^= __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v ^= __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v ^= __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v ^= __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v ^= __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, true);  // row_bcast:15
    v ^= __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, true);  // row_bcast:31
    return __builtin_amdgcn_readlane(v, 63);
}

// xor_bits_uniform computed by a whole wave: lane k loads entry k when bit k
// of v is set, and the wave XOR-reduces.  One vector load replaces a chain of
// dependent scalar loads, one per set bit, which a workgroup alone on its
// compute unit pays in full at the start of a short kernel.  Every lane of
// the wave must be active.  The load and the reduction are apart so that a
// kernel can issue the loads of several such sums before it waits for any.
template <typename T>
__device__ __forceinline__ T wave_load(const T *tab) {
    // every lane loads an in-bounds entry, so no branch splits the waits
    const uint32_t lane = __lane_id();
    return tab[lane < BMMC_MAX_BITS ? lane : BMMC_MAX_BITS - 1];
}

template <typename T>
__device__ __forceinline__ T wave_select_xor(T x, uint64_t v) {
    const uint32_t lane = __lane_id();
    const T e = (lane < BMMC_MAX_BITS && ((v >> lane) & 1u)) ? x : T(0);
    if constexpr (sizeof(T) == 8) {
        const uint32_t lo = wave_xor_u32((uint32_t)e), hi = wave_xor_u32((uint32_t)(e >> 32));
        return ((T)hi << 32) | lo;
    } else {
        return (T)wave_xor_u32((uint32_t)e);
    }
}

// The same sum with the load under the lane's condition: lanes whose bit is
// clear load nothing.
template <typename T>
__device__ __forceinline__ T xor_bits_wave(const T *tab, uint64_t v) {
    const uint32_t lane = __lane_id();
    const bool on = lane < BMMC_MAX_BITS && ((v >> lane) & 1u);
    return wave_select_xor(on ? tab[lane] : T(0), v);
}

// XOR of the first NB table entries selected by the bits of a per-lane value.
template <int NB, typename T>
__device__ __forceinline__ T xor_bits_lane(const T *tab, uint32_t v) {
    T acc = 0;
#pragma unroll
    for (int k = 0; k < NB; ++k) acc ^= ((v >> k) & 1u) ? tab[k] : T(0);
    return acc;
}

}  // namespace dev
}  // namespace bmmc
