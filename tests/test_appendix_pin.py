"""The appendix pin: the paper's printed 15-bit bit-reversal kernels replayed
on the CPU.

"Efficient GPU Implementation of Affine Index Permutations on Arrays"
(FHPNC'23), appendix, prints the kernels its generator emits for bit-reversal
on 2^15 4-byte elements: tiled, tiled without bank conflicts, and tiled with
eight tiles per thread block.  tests/golden/appendix_bitrev15_kernels.txt
restates where each of their address computations sends the bits of the
block, warp, thread and iteration indices.  Here every (block, iteration,
warp, thread) of each kernel is replayed: the global read into the
shared-memory slot, then the drain from the slot to the global write.  The
result must be the oracle's bit-rev(15), every element must be read and
written once and every slot used once per tile; the banks kernel's accesses
must fall on 32 distinct banks per warp where the plain tiled kernel's drain
falls on one.  Finally this library's plan for the same permutation (32 x 32
tiles of 4-byte units) must tile the array the same way and give the same
result when its kernel tables are replayed on the host.
"""
import os

import numpy as np
import pytest

import oracle
import bmmc_affine_index_amd as bm
from bmmc_affine_index_amd import workloads as wl

from emulate import replay_pass, run_plan_on_host

FIXTURE = os.path.join(os.path.dirname(__file__), "golden", "appendix_bitrev15_kernels.txt")
N = 15


def _kernels():
    meta, moves = {}, {}
    with open(FIXTURE) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "kernel":
                meta[parts[1]] = {k: int(v) for k, v in (p.split("=") for p in parts[2:])}
            else:
                name, addr, var = parts[:3]
                moves.setdefault(name, {}).setdefault(addr, []).append(
                    (var, [int(b) for b in parts[3:]]))
    return meta, moves


def _place(fields, var_values):
    """Assemble an address from the variables' bits moved to their places."""
    out = np.zeros_like(next(iter(var_values.values())))
    for var, dests in fields:
        v = var_values[var]
        for k, dst in enumerate(dests):
            out |= ((v >> k) & 1) << dst
    return out


def _replay(name, meta, moves):
    m = meta[name]
    grid, iters = m["grid"], m["iters"]
    b, it, w, t = np.meshgrid(np.arange(grid), np.arange(iters), np.arange(32), np.arange(32),
                              indexing="ij")
    vals = {"block": b.ravel().astype(np.int64), "iter": it.ravel().astype(np.int64),
            "warp": w.ravel().astype(np.int64), "thread": t.ravel().astype(np.int64)}
    a = {addr: _place(f, vals) for addr, f in moves[name].items()}
    if m["skew"]:
        for k in ("tile_w", "tile_r"):
            row, col = (a[k] >> 5) & 31, a[k] & 31
            a[k] = (a[k] & ~1023) | (row << 5) | ((row + col) & 31)
    return vals, a


@pytest.mark.parametrize("name", ["tiled", "banks", "iters"])
def test_printed_kernel_replays_to_the_oracle(name):
    meta, moves = _kernels()
    vals, a = _replay(name, meta, moves)
    size = 1 << N
    slots = 1024 * meta[name]["iters"]
    assert meta[name]["grid"] * slots == size
    # global read and write: each index exactly once
    assert np.array_equal(np.sort(a["in"]), np.arange(size))
    assert np.array_equal(np.sort(a["out"]), np.arange(size))
    # shared memory: each slot of each block's tiles written and read once
    for k in ("tile_w", "tile_r"):
        key = vals["block"] * slots + a[k]
        assert a[k].max() < slots and np.array_equal(np.sort(key), np.arange(size)), k
    # load phase, barrier, drain phase
    x = np.arange(size, dtype=np.int32)
    smem = np.full(meta[name]["grid"] * slots, -1, dtype=np.int32)
    smem[vals["block"] * slots + a["tile_w"]] = x[a["in"]]
    out = np.full(size, -1, dtype=np.int32)
    out[a["out"]] = smem[vals["block"] * slots + a["tile_r"]]
    want = oracle.apply(wl.bit_reverse_matrix(N), 0, x)
    assert np.array_equal(out, want)
    # and the one-index facts the same appendix states (bit 0 -> bit 14)
    assert out[1 << 14] == 1 and out[1] == 1 << 14 and out[1 << 7] == 1 << 7


def _banks_per_warp(name, addr):
    meta, moves = _kernels()
    vals, a = _replay(name, meta, moves)
    groups = {}
    for key, slot in zip(zip(vals["block"], vals["iter"], vals["warp"]), a[addr]):
        groups.setdefault(key, []).append(int(slot) % 32)
    return [len(set(v)) for v in groups.values()]


def test_banks_kernel_is_conflict_free_and_tiled_is_not():
    # the skewed layout: every warp's 32 slots on 32 distinct banks, both ways
    assert set(_banks_per_warp("banks", "tile_w")) == {32}
    assert set(_banks_per_warp("banks", "tile_r")) == {32}
    # the plain layouts read a tile column: all 32 lanes on one bank
    assert set(_banks_per_warp("tiled", "tile_w")) == {32}
    assert set(_banks_per_warp("tiled", "tile_r")) == {1}
    assert set(_banks_per_warp("iters", "tile_r")) == {1}


def test_library_plan_tiles_like_the_printed_kernels():
    """The library's one-tile plan at the same tile side (32 x 32 units of 4
    bytes) covers the same tiles as the printed kernels (input bits 0-4 and
    10-14 inside a tile, bits 5-9 number the tiles) and its host-replayed
    tables give the same output."""
    meta, moves = _kernels()
    vals, a = _replay("tiled", meta, moves)
    paper_tiles = {frozenset(a["in"][vals["block"] == blk].tolist()) for blk in range(32)}
    A = wl.bit_reverse_matrix(N)
    P = bm.Plan(N, A, 0, 4, tile_log2=5, launch=bm.LAUNCH_ONE_TILE, block_map=1)
    assert P.info.passes == 1 and P.info.tile_log2 == 5 and P.info.unit_bytes == 4
    d = P.passes()[0]
    assert d.blk_bits == 5
    # the units each of the plan's tiles reads, from its kernel tables
    chunk_bits = 2 * d.t - d.chunk_log2
    span = {0}
    for p in range(chunk_bits):
        span |= {s ^ int(d.ld_in[p]) for s in span}
    span = {(s >> d.unit_log2) + e for s in span for e in range(1 << d.chunk_log2)}
    plan_tiles = set()
    for blk in range(1 << d.blk_bits):
        base = 0
        for k in range(d.blk_bits):
            if (blk >> k) & 1:
                base ^= int(d.in_blk[k]) >> d.unit_log2
        plan_tiles.add(frozenset(base ^ s for s in span))
    assert plan_tiles == paper_tiles
    x = np.arange(1 << N, dtype=np.int32)
    smem_out = run_plan_on_host(P, x)
    assert np.array_equal(smem_out, oracle.apply(A, 0, x))
    assert len(replay_pass(d)) == 1 << N
