// plan.h -- internal plan representation and the host planner.
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/bmmc.h"
#include "gf2.h"

struct bmmc_plan {
    int n = 0;
    int elem_bytes = 0;
    uint64_t A[BMMC_MAX_N] = {};
    uint64_t c = 0;
    bmmc_plan_options opt = {};  // as the caller gave them (0 = planner's choice)
    bmmc_plan_info info = {};
    int npasses = 0;
    bmmc_pass_desc pass[BMMC_MAX_PASSES] = {};
    // element-level factor of each pass (n rows) and its complement
    uint64_t factor_A[BMMC_MAX_PASSES][BMMC_MAX_N] = {};
    uint64_t factor_c[BMMC_MAX_PASSES] = {};
    // scratch for two-pass plans, allocated on first execute
    mutable std::mutex scratch_mu;
    mutable void *scratch = nullptr;
    mutable int scratch_device = -1;
};

namespace bmmc {

// Build a plan: validation, inversion, classification, route choice and the
// kernel tables of every pass.  Host-only; returns a BMMC_* status.
int build_plan(int n, const uint64_t *A, uint64_t c, size_t elem_bytes,
               const bmmc_plan_options *opt, bmmc_plan *p);

// Largest tile side (log2 units) the tile kernel is compiled for at a unit
// size of 2^unit_log2 bytes, and the LDS byte budget of one workgroup.
int max_tile_log2(int unit_log2);
constexpr uint32_t kMaxLdsBytes = 65536;
// The persistent launch double-buffers tiles of up to 64 KiB (gfx950 gives a
// workgroup up to 160 KiB of LDS).
constexpr uint32_t kMaxPersistentLdsBytes = 131072;
// Persistent launch: 2^8 workgroups, one per compute unit on a 256-CU
// MI355X (measured against 2^9 .. 2^11 on the benchmark workloads).
constexpr int kDefaultGridLog2 = 8;
// Tile order when the caller leaves it to the planner: tiles in flight
// together are dense on the output side (block_map 5), since on MI355X HBM
// scattered writes cost more than scattered reads.  Measured untuned, as a
// fraction of the best of orders 1, 4, 5 and 6 on the same plan: 0.94 on
// average over 25 random BPCs and 0.98 over 25 random BMMCs (4-byte units,
// n = 22 .. 30), against 0.93 and 0.97 for the identity order; over the
// pages' four workload kinds at n = 20 .. 30 its worst case was 0.80 of the
// best untimed plan, against 0.59 for the identity order.
constexpr int kDefaultBlockMap = 5;

}  // namespace bmmc
