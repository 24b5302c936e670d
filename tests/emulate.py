"""Host replay of a plan's kernel tables (test helper, numpy only).

Replays every (workgroup, thread, pass, unit) of each kernel exactly as the
HIP kernels combine the tables of ``bmmc_pass_desc`` (include/bmmc.h), and
checks on the way that
  * every input unit is read once and every output unit written once,
  * every LDS slot of a tile is written once and read once, in range,
  * each wave's global access covers whole, aligned segments (coalescing),
then returns the source unit of every output unit.  Comparing the permuted
data with the oracle checks the planner without a GPU.
"""
from __future__ import annotations

import numpy as np

KERNEL_COPY, KERNEL_CHUNK, KERNEL_TILED, KERNEL_NAIVE, KERNEL_CHUNK_SCATTER = 0, 1, 2, 3, 4


def _xor_table(vals: np.ndarray, table, nbits: int) -> np.ndarray:
    vals = np.asarray(vals, dtype=np.uint64)
    acc = np.zeros(vals.shape, dtype=np.uint64)
    for k in range(nbits):
        bit = (vals >> np.uint64(k)) & np.uint64(1)
        acc ^= np.where(bit == 1, np.uint64(table[k]), np.uint64(0))
    return acc


def tiled_geometry(unit_log2: int, t: int, threads_log2: int):
    """Chunk width, chunks per row, thread and pass bits of a tile; the
    threads are the pass descriptor's threads_log2 (at most the chunk count)."""
    wl = min(4 - unit_log2, t)
    cpsl = t - wl
    chl = 2 * t - wl
    if not 1 <= threads_log2 <= chl:
        raise ReplayError("threads_log2 %d does not fit a tile of 2^%d chunks" % (threads_log2, chl))
    ntl = threads_log2
    rppl = ntl - cpsl
    jl = t - rppl
    return dict(wl=wl, cpsl=cpsl, ntl=ntl, rppl=rppl, jl=jl)


class ReplayError(AssertionError):
    pass


LAUNCH_ONE_TILE, LAUNCH_PERSISTENT, LAUNCH_STREAMED = 1, 2, 3


def check_persistent_walk(d):
    """Replays the persistent launch's walk: workgroup w, as walker
    v = w ^ ((w >> 3) & 7), starts at block v << r (ranges) or v (interleaved)
    and moves to the next block by XORing block bit ctz(k + 1) into its
    running bases.  Every block must be visited exactly once, and the running
    input base must equal the directly computed one at every step."""
    r = d.blk_bits - d.grid_log2
    if r < 0 or d.grid_log2 < 0:
        raise ReplayError("grid larger than the number of tiles")
    if d.walk not in (1, 2):
        raise ReplayError("unknown walk")
    shift = d.grid_log2 if d.walk == 2 else 0
    seen = np.zeros(1 << d.blk_bits, dtype=np.int64)
    for w in range(1 << d.grid_log2):
        v = w ^ ((w >> 3) & 7)
        blk = v if d.walk == 2 else v << r
        base = int(_xor_table(np.uint64(blk), d.in_blk, d.blk_bits))
        for k in range(1 << r):
            if base != int(_xor_table(np.uint64(blk), d.in_blk, d.blk_bits)):
                raise ReplayError("running base diverged")
            seen[blk] += 1
            if k + 1 < (1 << r):
                bit = shift + ((k + 1) & -(k + 1)).bit_length() - 1
                blk ^= 1 << bit
                base ^= int(d.in_blk[bit])
    if np.any(seen != 1):
        raise ReplayError("persistent walk does not visit every tile once")


def check_buffer_loads(d) -> None:
    """A pass that reads its input with buffer loads addresses it by 32-bit
    offsets: one whole tile per workgroup, units of 4 bytes or more and at
    most 2^31 bytes of array (the input offsets themselves are range-checked
    with every other access)."""
    bl = int(getattr(d, "buffer_loads", 0))
    if bl not in (0, 1):
        raise ReplayError("buffer_loads must be 0 or 1")
    if bl and (d.launch != LAUNCH_ONE_TILE or d.iters_log2 != 0 or
               int(getattr(d, "split_stage", 0)) or d.unit_log2 < 2 or
               d.nbits + d.unit_log2 > 31):
        raise ReplayError("buffer loads need one whole tile per workgroup, units of 4 bytes "
                          "or more and at most 2^31 bytes")


def replay_tiled(d, check_coalescing: bool = True) -> np.ndarray:
    """Source unit index of each output unit for one TILED pass."""
    ul, t, nb = d.unit_log2, d.t, d.nbits
    U = 1 << ul
    g = tiled_geometry(ul, t, d.threads_log2)
    wl, cpsl, ntl, jl = g["wl"], g["cpsl"], g["ntl"], g["jl"]
    W, CB, NT, J = 1 << wl, U << wl, 1 << ntl, 1 << jl
    cbits = ntl + jl
    TILE = U << (2 * t)
    blk_bits = d.blk_bits
    nblk = 1 << blk_bits
    split = int(getattr(d, "split_stage", 0))
    if split not in (0, 1):
        raise ReplayError("split_stage must be 0 or 1")
    check_buffer_loads(d)
    if d.launch in (LAUNCH_PERSISTENT, LAUNCH_STREAMED):
        if d.lds_bytes != 2 * TILE or d.iters_log2 != 0:
            raise ReplayError("persistent launch needs two LDS tiles")
        if split:
            raise ReplayError("split staging is a one-tile launch")
        check_persistent_walk(d)
    elif split:
        if d.iters_log2 != 0 or 2 * d.lds_bytes != TILE or jl < 1:
            raise ReplayError("split staging needs half a tile of LDS and two passes")
    elif d.lds_bytes != TILE << d.iters_log2:
        raise ReplayError("lds_bytes does not match the tile geometry")
    total_units = 1 << nb

    b = np.arange(nblk, dtype=np.uint64)[:, None]
    cidx = np.arange(NT * J, dtype=np.uint64)[None, :]  # chunk index (j << ntl) | tid

    in_off = _xor_table(b, d.in_blk, blk_bits) ^ _xor_table(cidx, d.ld_in, cbits)
    wr = _xor_table(cidx, d.ld_lds, cbits)
    in_off, wr = np.broadcast_arrays(in_off, wr)
    # LDS bytes one staging uses: the tile, or half of it when split
    LT = TILE >> split
    if np.any(in_off % np.uint64(CB)) or np.any(wr % np.uint64(CB)):
        raise ReplayError("misaligned chunk")
    if np.any(wr + np.uint64(CB) > np.uint64(LT)):
        raise ReplayError("LDS write out of range")
    if np.any(in_off + np.uint64(CB) > np.uint64(total_units * U)):
        raise ReplayError("global read out of range")

    out_off = (_xor_table(b, d.out_blk, blk_bits) ^ np.uint64(d.out_c)
               ^ _xor_table(cidx, d.st_out, cbits))
    rbase = (_xor_table(b, d.lds_blk, blk_bits) ^ np.uint64(d.lds_c)
             ^ _xor_table(cidx, d.st_lds, cbits))
    out_off, rbase = np.broadcast_arrays(out_off, rbase)
    if np.any(out_off % np.uint64(CB)):
        raise ReplayError("misaligned output chunk")
    if np.any(out_off + np.uint64(CB) > np.uint64(total_units * U)):
        raise ReplayError("global write out of range")

    # stagings: every chunk at once, or the chunks whose top chunk-index bit
    # is h in half h (loads and drain alike)
    allc = np.arange(NT * J)
    stagings = [allc] if not split else [allc[((allc >> (cbits - 1)) & 1) == h] for h in (0, 1)]
    read_in = np.zeros(total_units, dtype=np.int64)
    result = np.full(total_units, -1, dtype=np.int64)
    for cols in stagings:
        # LDS of every block, holding source unit indices
        lds = np.full((nblk, LT // U), -1, dtype=np.int64)
        bidx = np.broadcast_to(np.arange(nblk)[:, None], (nblk, cols.size))
        for e in range(W):
            slot = (wr[:, cols] // np.uint64(U) + np.uint64(e)).astype(np.int64)
            src = (in_off[:, cols] // np.uint64(U) + np.uint64(e)).astype(np.int64)
            if np.any(lds[bidx, slot] != -1):
                raise ReplayError("LDS slot written twice")
            lds[bidx, slot] = src
        if np.any(lds < 0):
            raise ReplayError("LDS slot never written")
        np.add.at(read_in, lds.reshape(-1), 1)
        reads = np.zeros((nblk, LT // U), dtype=np.int64)
        for e in range(W):
            rd = rbase[:, cols] ^ _xor_table(np.uint64(e), d.st_unit, wl)
            if np.any(rd % np.uint64(U)) or np.any(rd + np.uint64(U) > np.uint64(LT)):
                raise ReplayError("LDS read misaligned or out of range")
            slot = (rd // np.uint64(U)).astype(np.int64)
            np.add.at(reads, (bidx, slot), 1)
            dst = (out_off[:, cols] // np.uint64(U) + np.uint64(e)).astype(np.int64)
            if np.any(result[dst] != -1):
                raise ReplayError("output unit written twice")
            result[dst] = lds[bidx, slot]
        if np.any(reads != 1):
            raise ReplayError("LDS slot not read exactly once")
    if np.any(read_in != 1):
        raise ReplayError("input unit not read exactly once")
    if np.any(result < 0):
        raise ReplayError("output unit never written")

    if check_coalescing:
        # load: the lanes of an input row read it whole; drain: every group
        # of 2^pc lanes stores one contiguous aligned piece (128 bytes, or the
        # whole output row when shorter).  Rectangular tiles have rows of
        # 2^in_row_log2 units on the input side and 2^out_row_log2 on the
        # output side (both t for square tiles).
        a, b = d.in_row_log2, d.out_row_log2
        if a + b != 2 * t or min(a, b) < wl:
            raise ReplayError("row lengths do not match the tile geometry")
        pc_load = a - wl
        pc_drain = min(b - wl, max(0, 7 - (ul + wl)))
        for arr, pcx in ((in_off, pc_load), (out_off, pc_drain)):
            G = 1 << pcx
            a = arr.reshape(nblk, (NT * J) // G, G)
            starts = a.min(axis=2)
            if np.any(starts % np.uint64(G * CB)):
                raise ReplayError("lane group not aligned")
            rel = np.sort(a - starts[:, :, None], axis=2)
            want = (np.arange(G, dtype=np.uint64) * np.uint64(CB))[None, None, :]
            if not np.array_equal(rel, np.broadcast_to(want, rel.shape)):
                raise ReplayError("a lane group's access is not contiguous")
    return result


def replay_chunk(d) -> np.ndarray:
    """CHUNK (a gather): output chunk x is read from XOR in_blk over x's bits
    XOR in_c; NAIVE and CHUNK_SCATTER (scatters): input chunk x is stored at
    XOR out_blk over x's bits XOR out_c.  Either way unit e of the output chunk is unit
    e XOR unit_xor of the input chunk."""
    ul, nb, wl = d.unit_log2, d.nbits, d.chunk_log2
    U, W = 1 << ul, 1 << wl
    nchunks = 1 << d.blk_bits
    x = np.arange(nchunks, dtype=np.uint64)
    result = np.full(1 << nb, -1, dtype=np.int64)
    if d.kernel == KERNEL_CHUNK:
        src = _xor_table(x, d.in_blk, d.blk_bits) ^ np.uint64(d.in_c)
        if np.any(src % np.uint64(U * W)) or np.any(src // np.uint64(U) >= np.uint64(1 << nb)):
            raise ReplayError("chunk load misaligned or out of range")
        seen = np.zeros(nchunks, dtype=np.int64)
        np.add.at(seen, (src // np.uint64(U * W)).astype(np.int64), 1)
        if np.any(seen != 1):
            raise ReplayError("input chunk not read exactly once")
        for e in range(W):
            dst = (x * np.uint64(W) + np.uint64(e)).astype(np.int64)
            result[dst] = (src // np.uint64(U) + np.uint64(e ^ d.unit_xor)).astype(np.int64)
        return result
    off = _xor_table(x, d.out_blk, d.blk_bits) ^ np.uint64(d.out_c)
    if np.any(off % np.uint64(U * W)):
        raise ReplayError("misaligned chunk store")
    for e in range(W):
        dst = (off // np.uint64(U) + np.uint64(e)).astype(np.int64)
        src = (x * np.uint64(W) + np.uint64(e ^ d.unit_xor)).astype(np.int64)
        if np.any(dst >= (1 << nb)) or np.any(result[dst] != -1):
            raise ReplayError("chunk store out of range or twice")
        result[dst] = src
    if np.any(result < 0):
        raise ReplayError("output unit never written")
    return result


def replay_pass(d) -> np.ndarray:
    if d.kernel == KERNEL_TILED:
        return replay_tiled(d)
    if d.kernel in (KERNEL_CHUNK, KERNEL_NAIVE, KERNEL_CHUNK_SCATTER):
        return replay_chunk(d)
    if d.kernel == KERNEL_COPY:
        return np.arange(1 << d.nbits, dtype=np.int64)
    raise ReplayError("unknown kernel %d" % d.kernel)


def run_plan_on_host(plan, data: np.ndarray) -> np.ndarray:
    """Apply every pass of ``plan`` (a bmmc_affine_index_amd.Plan) to a host
    array by replaying the kernel tables; returns the permuted copy."""
    raw = np.ascontiguousarray(data).view(np.uint8).reshape(-1)
    cur = raw
    for d in plan.passes():
        U = 1 << d.unit_log2
        units = cur.reshape(-1, U)
        src = replay_pass(d)
        cur = units[src].reshape(-1)
    return cur.view(data.dtype).reshape(data.shape)


def bank_cycles(addr, nbytes: int, banks: int) -> int:
    """Cycles of one wave LDS access under the planner's bank model."""
    per = (4 * banks) // nbytes if nbytes >= 4 else banks
    per = max(1, min(64, per))
    total = 0
    addr = [int(a) for a in addr]
    for g0 in range(0, len(addr), per):
        words = set()
        for a in addr[g0:g0 + per]:
            for w in range(max(1, nbytes // 4)):
                words.add(a // 4 + w)
        cnt = {}
        for w in words:
            cnt[w % banks] = cnt.get(w % banks, 0) + 1
        total += max(cnt.values()) if cnt else 1
    return total


def tiled_read_addresses(d):
    """LDS byte addresses of wave 0's first output-order read (unit 0)."""
    g = tiled_geometry(d.unit_log2, d.t, d.threads_log2)
    lane_bits = min(6, g["ntl"])
    out = []
    for l in range(1 << lane_bits):
        a = 0
        for p in range(lane_bits):
            if (l >> p) & 1:
                a ^= d.st_lds[p]
        out.append(a)
    return out


def tiled_write_addresses(d):
    g = tiled_geometry(d.unit_log2, d.t, d.threads_log2)
    lane_bits = min(6, g["ntl"])
    out = []
    for l in range(1 << lane_bits):
        a = 0
        for p in range(lane_bits):
            if (l >> p) & 1:
                a ^= d.ld_lds[p]
        out.append(a)
    return out


def check_pass_sampled(d, A, c, elem_log2: int, blocks, map_indices) -> int:
    """Sampled replay for passes too large to replay whole: for each block in
    `blocks` (tiles of a TILED pass, chunks of a CHUNK/NAIVE pass) every chunk
    and unit is replayed through the tables, checked for alignment and range
    (global offsets below 2^(nbits + unit_log2) bytes, LDS slots inside the
    tile, each slot written and read once), and each unit's destination is
    compared with `map_indices(A, c, elements)` of the pass's element-level
    factor (A, c).  Returns the number of units checked."""
    ul, nb = d.unit_log2, d.nbits
    U = 1 << ul
    k = ul - elem_log2  # element-index bits inside a unit
    total_bytes = np.uint64(U) << np.uint64(nb)
    checked = 0
    blocks = np.asarray(sorted(set(int(b) for b in blocks)), dtype=np.uint64)
    if np.any(blocks >= np.uint64(1 << d.blk_bits)):
        raise ReplayError("sampled block out of range")

    def expect(src_units, dst_units):
        want = map_indices(A, c, src_units.astype(np.uint64) << np.uint64(k)) >> np.uint64(k)
        if not np.array_equal(want, dst_units.astype(np.uint64)):
            raise ReplayError("unit sent to the wrong place")

    if d.kernel == KERNEL_CHUNK:  # gather: sampled output chunks
        wl = d.chunk_log2
        W = 1 << wl
        src = _xor_table(blocks, d.in_blk, d.blk_bits) ^ np.uint64(d.in_c)
        if np.any(src % np.uint64(U * W)) or np.any(src + np.uint64(U * W) > total_bytes):
            raise ReplayError("chunk load misaligned or out of range")
        for e in range(W):
            expect(src // np.uint64(U) + np.uint64(e ^ d.unit_xor),
                   blocks * np.uint64(W) + np.uint64(e))
            checked += blocks.size
        return checked
    if d.kernel in (KERNEL_NAIVE, KERNEL_CHUNK_SCATTER):  # scatter: sampled input chunks
        wl = d.chunk_log2
        W = 1 << wl
        off = _xor_table(blocks, d.out_blk, d.blk_bits) ^ np.uint64(d.out_c)
        if np.any(off % np.uint64(U * W)) or np.any(off + np.uint64(U * W) > total_bytes):
            raise ReplayError("chunk store misaligned or out of range")
        for e in range(W):
            src = blocks * np.uint64(W) + np.uint64(e ^ d.unit_xor)
            expect(src, off // np.uint64(U) + np.uint64(e))
            checked += src.size
        return checked
    if d.kernel != KERNEL_TILED:
        raise ReplayError("no sampled replay for kernel %d" % d.kernel)

    t = d.t
    g = tiled_geometry(ul, t, d.threads_log2)
    wl, ntl, jl = g["wl"], g["ntl"], g["jl"]
    W, CB, NT, J = 1 << wl, U << wl, 1 << ntl, 1 << jl
    cbits = ntl + jl
    TILE = U << (2 * t)
    split = int(getattr(d, "split_stage", 0))
    if split and (d.launch != LAUNCH_ONE_TILE or d.iters_log2 != 0 or 2 * d.lds_bytes != TILE
                  or jl < 1):
        raise ReplayError("split staging needs a one-tile launch, half a tile of LDS and two passes")
    check_buffer_loads(d)
    LT = TILE >> split  # LDS bytes of one staging
    cidx = np.arange(NT * J, dtype=np.uint64)
    ld_in = _xor_table(cidx, d.ld_in, cbits)
    ld_lds = _xor_table(cidx, d.ld_lds, cbits)
    st_out = _xor_table(cidx, d.st_out, cbits)
    st_lds = _xor_table(cidx, d.st_lds, cbits)
    if np.any(ld_lds % np.uint64(CB)) or np.any(ld_lds + np.uint64(CB) > np.uint64(LT)):
        raise ReplayError("LDS write misaligned or out of range")
    allc = np.arange(NT * J)
    stagings = [allc] if not split else [allc[((allc >> (cbits - 1)) & 1) == h] for h in (0, 1)]
    for b in blocks:
        in_off_all = _xor_table(b, d.in_blk, d.blk_bits) ^ ld_in
        if np.any(in_off_all % np.uint64(CB)) or np.any(in_off_all + np.uint64(CB) > total_bytes):
            raise ReplayError("global read misaligned or out of range")
        out_all = (_xor_table(b, d.out_blk, d.blk_bits) ^ np.uint64(d.out_c)) ^ st_out
        rbase_all = (_xor_table(b, d.lds_blk, d.blk_bits) ^ np.uint64(d.lds_c)) ^ st_lds
        if np.any(out_all % np.uint64(CB)) or np.any(out_all + np.uint64(CB) > total_bytes):
            raise ReplayError("global write misaligned or out of range")
        for cols in stagings:
            in_off, wr = in_off_all[cols], ld_lds[cols]
            lds = np.full(LT // U, -1, dtype=np.int64)
            for e in range(W):
                slot = (wr // np.uint64(U) + np.uint64(e)).astype(np.int64)
                if np.any(lds[slot] != -1):
                    raise ReplayError("LDS slot written twice")
                lds[slot] = (in_off // np.uint64(U) + np.uint64(e)).astype(np.int64)
            out_off, rbase = out_all[cols], rbase_all[cols]
            reads = np.zeros(LT // U, dtype=np.int64)
            for e in range(W):
                rd = rbase ^ _xor_table(np.uint64(e), d.st_unit, wl)
                if np.any(rd % np.uint64(U)) or np.any(rd + np.uint64(U) > np.uint64(LT)):
                    raise ReplayError("LDS read misaligned or out of range")
                slot = (rd // np.uint64(U)).astype(np.int64)
                np.add.at(reads, slot, 1)
                expect(lds[slot], out_off // np.uint64(U) + np.uint64(e))
                checked += slot.size
            if np.any(reads != 1) or np.any(lds < 0):
                raise ReplayError("LDS slot not written and read exactly once")
    return checked
