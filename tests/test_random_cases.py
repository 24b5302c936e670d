"""Host replay of the seeded random option cases (tests/random_cases.py):
every plan the library accepts is replayed from its kernel tables, with every
global and LDS access checked for range and exactly-once coverage, and must
reproduce the oracle's permutation.  No GPU call is made."""
import numpy as np
import pytest

import oracle
import bmmc_affine_index_amd as bm
from emulate import run_plan_on_host
from random_cases import N_CASES, cases, plan_or_none

BATCHES = 6


def test_cases_are_fixed_and_span_the_options():
    a, b = cases(), cases()
    assert [c.ident() for c in a] == [c.ident() for c in b]
    assert len(a) == N_CASES
    seen = {k for c in a for k in c.options}
    assert {"route", "launch", "tile_log2", "block_map", "iters_log2", "grid_log2", "walk",
            "depth", "cache_hint", "no_swizzle", "tile_skew", "tile_threads_log2",
            "split_stage", "buffer_loads"} <= seen
    skews = {c.options.get("tile_skew", 0) for c in a}
    assert {1, -1, 2, -2} <= skews
    split = [c for c in a if c.options.get("split_stage")]
    assert len(split) >= 100
    assert {c.options.get("tile_skew", 0) for c in split} >= {0, 1, -1}
    assert {c.options.get("route", 0) for c in split} >= {0, 2, 3}
    assert {c.elem for c in split} == {1, 2, 4, 8, 16}
    staged_in_halves = 0
    for c in split:
        A, cc = c.matrix()
        P = bm.Plan(c.n, A, cc, c.elem, **c.options)
        staged_in_halves += any(d.kernel == bm.KERNEL_TILED and d.split_stage for d in P.passes())
    assert staged_in_halves >= 80
    buf = [c for c in a if c.options.get("buffer_loads")]
    assert len(buf) >= 80
    assert {c.options.get("route", 0) for c in buf} >= {0, 2, 3}
    assert {c.options.get("tile_skew", 0) for c in buf} >= {0, 1, -1, 2, -2}
    assert {c.options.get("tile_threads_log2", 0) for c in buf} == {0, 9}
    assert {c.elem for c in buf} >= {4, 8, 16}
    for c in buf:
        A, cc = c.matrix()
        P = bm.Plan(c.n, A, cc, c.elem, **c.options)
        assert all(d.buffer_loads == 1 for d in P.passes() if d.kernel == bm.KERNEL_TILED)
    assert {c.kind for c in a} == {"general", "bpc", "bitrev", "transpose", "complement",
                                   "blockperm", "lowkeep"}
    assert {c.elem for c in a} == {1, 2, 4, 8, 16}


@pytest.mark.parametrize("batch", range(BATCHES))
def test_random_cases_replay_on_host(batch):
    mine = cases()[batch::BATCHES]
    ran = 0
    for case in mine:
        P = plan_or_none(case)
        if P is None:
            continue
        A, c = case.matrix()
        x = case.data()
        assert np.array_equal(run_plan_on_host(P, x), oracle.apply(A, c, x)), case.ident()
        ran += 1
    assert ran >= 0.9 * len(mine)
