"""Seeded random (matrix, data, plan options) cases over the whole option
space: every matrix class, element size, route, launch style, tile side, tile
order, grid, walk, depth, cache hint and LDS layout, drawn together.  Holds
none of the method's arithmetic: matrices come from the seeded generators of
the workloads module (or simple block-diagonal compositions of them), and the
oracle supplies every expected value.

A case is only handed to the GPU after the host replay of its kernel tables
(tests/emulate.py) has checked every global and LDS access for range and
exactly-once coverage and reproduced the oracle's permutation."""
from dataclasses import dataclass, field

import numpy as np

import oracle
import bmmc_affine_index_amd as bm
from bmmc_affine_index_amd import workloads as wl

KINDS = ("general", "bpc", "bitrev", "transpose", "complement", "blockperm", "lowkeep")
ELEMS = (1, 2, 4, 8, 16)
N_SQUARE = 600
N_SKEW = 180   # rectangular tiles (tile_skew), drawn from a stream of their own
N_SPLIT = 160  # one-tile launches staged in LDS half at a time (split_stage)
N_BUF = 120    # one-tile launches that read the input with buffer loads (buffer_loads)
N_SKEW2 = 60   # the two-pass route with rectangular tiles
N_CASES = N_SQUARE + N_SKEW + N_SPLIT + N_BUF + N_SKEW2
MASTER_SEED = 0x5EED_B44C
SKEW_SEED = 0x5EED_5CE7
SPLIT_SEED = 0x5EED_5B17
BUF_SEED = 0x5EED_B0FF
SKEW2_SEED = 0x5EED_2BA5


@dataclass
class Case:
    index: int
    kind: str
    n: int
    elem: int
    seed: int
    options: dict = field(default_factory=dict)

    def matrix(self):
        n, s = self.n, self.seed
        if self.kind == "bitrev":
            return wl.bit_reverse_matrix(n), 0
        if self.kind == "transpose":
            return wl.transpose_matrix(n // 2, n - n // 2), 0
        if self.kind == "bpc":
            return wl.random_bpc(n, s)
        if self.kind == "complement":
            return wl.identity_matrix(n), (s * 0x9E3779B97F4A7C15) & ((1 << n) - 1)
        if self.kind in ("blockperm", "lowkeep"):
            # the low k index bits map to themselves; a random invertible map
            # of the other n - k bits (whole blocks move, or, with k small,
            # units merge over the kept low bits)
            k = max(0, min(n - 1, (s % 7) + (3 if self.kind == "blockperm" else 0)))
            Q, cq = wl.random_bmmc(n - k, s, lambda r: oracle.rank(r) == n - k)
            A = np.array([1 << r for r in range(k)] + [int(q) << k for q in Q], dtype=np.uint64)
            return A, (int(cq) << k) if self.kind == "lowkeep" else 0
        return wl.random_bmmc(n, s, lambda r: oracle.rank(r) == n)

    def data(self):
        return wl.fill_random_bytes(self.n, self.elem, self.seed ^ 0xDA7A)

    def ident(self):
        return "case%03d-%s-n%d-e%d-%s" % (self.index, self.kind, self.n, self.elem, "-".join(
            "%s%d" % (k, v) for k, v in sorted(self.options.items())))


def cases():
    """The fixed list of N_CASES cases (the same on every call)."""
    rng = np.random.Generator(np.random.PCG64(MASTER_SEED))
    out = []
    for i in range(N_SQUARE):
        kind = KINDS[int(rng.integers(len(KINDS)))]
        elem = ELEMS[int(rng.integers(len(ELEMS)))]
        n = int(rng.integers(1, 19))
        if kind == "blockperm" and n < 5:
            n += 5
        opts = {}
        route = int(rng.choice([bm.ROUTE_AUTO, bm.ROUTE_AUTO, bm.ROUTE_FUSED,
                                bm.ROUTE_TWO_PASS, bm.ROUTE_NAIVE]))
        if route:
            opts["route"] = route
        launch = int(rng.choice([bm.LAUNCH_AUTO, bm.LAUNCH_ONE_TILE, bm.LAUNCH_PERSISTENT,
                                 bm.LAUNCH_STREAMED]))
        if launch:
            opts["launch"] = launch
        t = int(rng.choice([0, 0, 0, 3, 4, 5, 6, 7]))
        if t:
            opts["tile_log2"] = t
        bmap = int(rng.choice([0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 13]))
        if bmap:
            opts["block_map"] = bmap
        if launch in (bm.LAUNCH_AUTO, bm.LAUNCH_ONE_TILE) and rng.random() < 0.3:
            opts["iters_log2"] = int(rng.integers(1, 3))
        if launch in (bm.LAUNCH_PERSISTENT, bm.LAUNCH_STREAMED):
            g = int(rng.choice([0, 0, 1, 3, 5]))
            if g:
                opts["grid_log2"] = g
            w = int(rng.choice([0, bm.WALK_RANGES, bm.WALK_INTERLEAVED]))
            if w:
                opts["walk"] = w
        if launch == bm.LAUNCH_STREAMED and rng.random() < 0.5:
            opts["depth"] = int(rng.integers(1, 3))
        hint = int(rng.choice([0, 0, 1, 2]))
        if hint:
            opts["cache_hint"] = hint
        if rng.random() < 0.15:
            opts["no_swizzle"] = 1
        out.append(Case(i, kind, n, elem, int(rng.integers(1, 1 << 30)), opts))
    # rectangular tiles: single-pass routes with input and output rows of
    # different lengths; a skew the library refuses for the drawn size is
    # brought towards 0 until it accepts one (planning is host-only)
    rng = np.random.Generator(np.random.PCG64(SKEW_SEED))
    for i in range(N_SKEW):
        kind = KINDS[int(rng.integers(len(KINDS)))]
        elem = ELEMS[int(rng.integers(len(ELEMS)))]
        n = int(rng.integers(6, 19))
        opts = {}
        route = int(rng.choice([bm.ROUTE_AUTO, bm.ROUTE_FUSED]))
        if route:
            opts["route"] = route
        launch = int(rng.choice([bm.LAUNCH_AUTO, bm.LAUNCH_ONE_TILE, bm.LAUNCH_PERSISTENT,
                                 bm.LAUNCH_STREAMED]))
        if launch:
            opts["launch"] = launch
        t = int(rng.choice([0, 0, 4, 5, 6, 7]))
        if t:
            opts["tile_log2"] = t
        bmap = int(rng.choice([0, 1, 3, 5, 6, 8, 11]))
        if bmap:
            opts["block_map"] = bmap
        if launch == bm.LAUNCH_STREAMED and rng.random() < 0.5:
            opts["depth"] = int(rng.integers(1, 3))
        if rng.random() < 0.15:
            opts["no_swizzle"] = 1
        skew = int(rng.choice([1, -1, 2, -2, 3, -3]))
        if rng.random() < 0.4:
            opts["tile_threads_log2"] = 9
        case = Case(N_SQUARE + i, kind, n, elem, int(rng.integers(1, 1 << 30)), opts)
        A, c = case.matrix()
        while skew:
            try:
                bm.Plan(n, A, c, elem, tile_skew=skew, **opts)
                break
            except bm.BmmcError:
                skew -= 1 if skew > 0 else -1
        if skew:
            case.options["tile_skew"] = skew
        out.append(case)
    # split staging: one-tile launches whose tiles pass through LDS half at a
    # time, over both routes, tile shapes and thread counts; where the library
    # refuses the split for the drawn shape, the skew is brought towards 0,
    # and a case it refuses at every skew is kept unsplit
    rng = np.random.Generator(np.random.PCG64(SPLIT_SEED))
    tiled_kinds = ("general", "bpc", "bitrev", "transpose", "blockperm", "lowkeep")
    for i in range(N_SPLIT):
        kind = tiled_kinds[int(rng.integers(len(tiled_kinds)))]
        elem = ELEMS[int(rng.integers(len(ELEMS)))]
        n = int(rng.integers(10, 19))
        opts = {}
        route = int(rng.choice([bm.ROUTE_AUTO, bm.ROUTE_FUSED, bm.ROUTE_TWO_PASS]))
        if route:
            opts["route"] = route
        if rng.random() < 0.5:
            opts["launch"] = bm.LAUNCH_ONE_TILE
        t = int(rng.choice([0, 0, 5, 6, 7]))
        if t:
            opts["tile_log2"] = t
        bmap = int(rng.choice([0, 1, 3, 5, 6, 8, 12]))
        if bmap:
            opts["block_map"] = bmap
        hint = int(rng.choice([0, 0, 1, 2]))
        if hint:
            opts["cache_hint"] = hint
        if rng.random() < 0.1:
            opts["no_swizzle"] = 1
        if rng.random() < 0.4:
            opts["tile_threads_log2"] = 9
        skew = int(rng.choice([0, 0, 1, -1, 2, -2])) if route != bm.ROUTE_TWO_PASS else 0
        case = Case(N_SQUARE + N_SKEW + i, kind, n, elem, int(rng.integers(1, 1 << 30)), opts)
        A, c = case.matrix()
        while True:
            try:
                bm.Plan(n, A, c, elem, tile_skew=skew, split_stage=1, **opts)
                case.options["split_stage"] = 1
                if skew:
                    case.options["tile_skew"] = skew
                break
            except bm.BmmcError:
                if not skew:
                    break
                skew -= 1 if skew > 0 else -1
        out.append(case)
    # buffer loads: one-tile launches of whole tiles whose input is read by
    # 32-bit offsets, over both routes, tile shapes, thread counts and orders;
    # mostly units of 4 bytes or more (1- and 2-byte elements get there when
    # the matrix keeps low bits); a case the library refuses them for is kept
    # without
    rng = np.random.Generator(np.random.PCG64(BUF_SEED))
    for i in range(N_BUF):
        kind = tiled_kinds[int(rng.integers(len(tiled_kinds)))]
        elem = int(rng.choice([1, 2, 4, 4, 8, 16, 16]))
        n = int(rng.integers(10, 19))
        opts = {}
        route = int(rng.choice([bm.ROUTE_AUTO, bm.ROUTE_FUSED, bm.ROUTE_TWO_PASS]))
        if route:
            opts["route"] = route
        if rng.random() < 0.5:
            opts["launch"] = bm.LAUNCH_ONE_TILE
        t = int(rng.choice([0, 0, 4, 5, 6, 7]))
        if t:
            opts["tile_log2"] = t
        bmap = int(rng.choice([0, 1, 2, 3, 5, 6, 8, 12]))
        if bmap:
            opts["block_map"] = bmap
        hint = int(rng.choice([0, 0, 1, 2]))
        if hint:
            opts["cache_hint"] = hint
        if rng.random() < 0.1:
            opts["no_swizzle"] = 1
        if rng.random() < 0.4:
            opts["tile_threads_log2"] = 9
        skew = int(rng.choice([0, 0, 1, -1, 2, -2])) if route != bm.ROUTE_TWO_PASS else 0
        if skew:
            opts["tile_skew"] = skew
        case = Case(N_SQUARE + N_SKEW + N_SPLIT + i, kind, n, elem,
                    int(rng.integers(1, 1 << 30)), opts)
        A, c = case.matrix()
        try:
            bm.Plan(n, A, c, elem, buffer_loads=1, **opts)
            case.options["buffer_loads"] = 1
        except bm.BmmcError:
            pass
        out.append(case)
    # the two-pass route with rectangular tiles: the relabel moves segments as
    # long as the tile's input rows; a skew the library refuses for the
    # drawn size is brought towards 0 until it accepts one
    rng = np.random.Generator(np.random.PCG64(SKEW2_SEED))
    for i in range(N_SKEW2):
        elem = ELEMS[int(rng.integers(len(ELEMS)))]
        n = int(rng.integers(10, 19))
        opts = {"route": bm.ROUTE_TWO_PASS}
        launch = int(rng.choice([bm.LAUNCH_AUTO, bm.LAUNCH_ONE_TILE, bm.LAUNCH_PERSISTENT,
                                 bm.LAUNCH_STREAMED]))
        if launch:
            opts["launch"] = launch
        t = int(rng.choice([0, 0, 4, 5, 6, 7]))
        if t:
            opts["tile_log2"] = t
        bmap = int(rng.choice([0, 1, 3, 5, 6, 8]))
        if bmap:
            opts["block_map"] = bmap
        if rng.random() < 0.4:
            opts["tile_threads_log2"] = 9
        skew = int(rng.choice([1, -1, 2, -2]))
        case = Case(N_SQUARE + N_SKEW + N_SPLIT + N_BUF + i, "general", n, elem,
                    int(rng.integers(1, 1 << 30)), opts)
        A, c = case.matrix()
        while skew:
            try:
                bm.Plan(n, A, c, elem, tile_skew=skew, **opts)
                break
            except bm.BmmcError:
                skew -= 1 if skew > 0 else -1
        if skew:
            case.options["tile_skew"] = skew
        # some one-tile launches read their input with buffer loads
        if launch == bm.LAUNCH_ONE_TILE and rng.random() < 0.5:
            try:
                bm.Plan(n, A, c, elem, buffer_loads=1, **case.options)
                case.options["buffer_loads"] = 1
            except bm.BmmcError:
                pass
        out.append(case)
    return out


def plan_or_none(case: Case):
    """The case's plan, or None when the library rejects the combination of
    options (an argument error, not a fault: no GPU call is involved)."""
    A, c = case.matrix()
    try:
        return bm.Plan(case.n, A, c, case.elem, **case.options)
    except bm.BmmcError:
        return None
