"""CPU tests of the C-ABI library: exports, argument checks, the planner's F2
algebra (classification, tile test, factorisation) and a host replay of every
kernel table against the oracle.  No GPU call is made."""
import os
import re

import numpy as np
import pytest

import oracle
import bmmc_affine_index_amd as bm
from bmmc_affine_index_amd import workloads as wl

from emulate import (ReplayError, bank_cycles, check_pass_sampled, run_plan_on_host,
                     tiled_geometry, tiled_read_addresses, tiled_write_addresses)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _inv(n, seed):
    return wl.random_bmmc(n, seed, lambda r: oracle.rank(r) == n)


# --------------------------------------------------------------------------
# The library and its exports
# --------------------------------------------------------------------------

def test_library_exports_every_header_function():
    names = set()
    for h in ("bmmc.h", "bmmc_testing.h"):
        header = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"^\S[^;()]*?\b(bmmc_\w+)\s*\(", header, flags=re.M))
    assert names == set(bm.EXPORTED)
    L = bm.lib()
    for name in names:
        assert hasattr(L, name), name


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors have the C header's sizes and field offsets."""
    import ctypes
    import subprocess
    structs = {"bmmc_pass_desc": bm.bmmc_pass_desc, "bmmc_plan_info": bm.bmmc_plan_info,
               "bmmc_plan_options": bm.bmmc_plan_options}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "bmmc.h"',
             "int main(void) {"]
    for name, cls in structs.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (name, name))
        for field, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (name, field, name, field))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    out = dict(l.split() for l in subprocess.check_output([str(exe)]).decode().splitlines())
    for name, cls in structs.items():
        assert int(out[name]) == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert int(out[name + "." + field]) == getattr(cls, field).offset, (name, field)


# --------------------------------------------------------------------------
# Argument validation (returns before any GPU call)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,A,c,e,status", [
    (0, [], 0, 4, bm.ERR_INVALID_ARG),
    (33, [1 << r for r in range(33)], 0, 4, bm.ERR_INVALID_ARG),
    (3, [1, 2, 4], 0, 3, bm.ERR_INVALID_ARG),
    (3, [1, 2, 4], 0, 32, bm.ERR_INVALID_ARG),
    (3, [1, 2, 4], 0, 0, bm.ERR_INVALID_ARG),
    (3, [1, 2, 8], 0, 4, bm.ERR_INVALID_ARG),       # stray bit in A
    (3, [1, 2, 4], 8, 4, bm.ERR_INVALID_ARG),       # stray bit in c
    (3, [1, 2, 3], 0, 4, bm.ERR_SINGULAR),
    (32, [1 << r for r in range(32)], 0, 32, bm.ERR_INVALID_ARG),
    (32, [1 << r for r in range(32)], 0, 32, bm.ERR_INVALID_ARG),
])
def test_plan_create_errors(n, A, c, e, status):
    h = bm.bmmc_plan_create(n, A, c, e)
    assert h == 0
    assert bm.bmmc_last_error() == status
    assert bm.bmmc_status_string(status)


def test_plan_create_largest_sizes():
    # the largest arrays: 2^32 elements of 16 bytes (2^36 bytes), general A
    A, c = _inv(32, 32)
    for e in (4, 16):
        h = bm.bmmc_plan_create(32, A, c, e)
        assert h != 0, bm.bmmc_last_error()
        info = bm.bmmc_plan_get_info(h)
        assert info.unit_bits + (info.unit_bytes.bit_length() - 1) == 32 + (e.bit_length() - 1)
        bm.bmmc_plan_destroy(h)


def test_execute_argument_errors_without_gpu():
    p = bm.Plan(10, wl.bit_reverse_matrix(10), 0, 4)
    assert bm.bmmc_execute(p.handle, 0, 4096, None) == bm.ERR_INVALID_ARG
    assert bm.bmmc_execute(0, 4096, 8192, None) == bm.ERR_INVALID_ARG
    # misaligned
    assert bm.bmmc_execute(p.handle, 1 << 20 | 4, 1 << 24, None) == bm.ERR_INVALID_ARG
    # overlapping ranges (the array is 4 KiB)
    assert bm.bmmc_execute(p.handle, 1 << 20, (1 << 20) + 2048, None) == bm.ERR_ALIAS
    assert bm.bmmc_copy(1 << 20, (1 << 20) + 16, 64, None) == bm.ERR_ALIAS
    assert bm.bmmc_copy(0, 1 << 20, 64, None) == bm.ERR_INVALID_ARG
    assert bm.bmmc_copy(0, 0, 0, None) == bm.OK
    for k in (-1, 1):
        with pytest.raises(bm.BmmcError):
            bm.bmmc_plan_get_pass(p.handle, k)


def test_execute_noalloc_refuses_without_gpu():
    """bmmc_execute_noalloc makes every check before its first HIP call: the
    buffer rules of bmmc_execute, and a two-pass plan larger than the fixed
    scratch buffer (these fake addresses are never touched)."""
    p = bm.Plan(10, wl.bit_reverse_matrix(10), 0, 4)
    assert bm.bmmc_execute_noalloc(p.handle, 0, 4096, None) == bm.ERR_INVALID_ARG
    assert bm.bmmc_execute_noalloc(0, 4096, 8192, None) == bm.ERR_INVALID_ARG
    assert bm.bmmc_execute_noalloc(p.handle, 1 << 20 | 4, 1 << 24, None) == bm.ERR_INVALID_ARG
    assert bm.bmmc_execute_noalloc(p.handle, 1 << 20, (1 << 20) + 2048, None) == bm.ERR_ALIAS
    n = 25  # 2^25 int32: twice the buffer
    A, c = _inv(n, 25)
    q = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS)
    assert q.info.passes == 2 and q.info.scratch_bytes > bm.NOALLOC_SCRATCH_BYTES
    assert bm.bmmc_execute_noalloc(q.handle, 1 << 40, 1 << 41, None) == bm.ERR_SCRATCH_LIMIT
    assert "scratch" in bm.bmmc_status_string(bm.ERR_SCRATCH_LIMIT)
    # the header's size is the binding's
    header = open(os.path.join(ROOT, "include", "bmmc.h")).read()
    assert re.search(r"#define BMMC_NOALLOC_SCRATCH_BYTES \(\(size_t\)1 << 26\)", header)
    assert bm.NOALLOC_SCRATCH_BYTES == 1 << 26


def test_injected_scratch_failure_without_gpu():
    """A two-pass plan whose scratch allocation fails returns
    ERR_OUT_OF_MEMORY from bmmc_execute and bmmc_plan_tune_pairs, before any
    HIP call (these fake addresses are never touched), and keeps no scratch;
    each injected failure is used once."""
    n = 16
    A, c = _inv(n, 16)
    p = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS)
    assert p.info.passes == 2
    i, o = 1 << 40, (1 << 40) + (1 << 30)
    try:
        assert bm.bmmc_testing_fail_scratch_allocs(-1) == bm.ERR_INVALID_ARG
        assert bm.bmmc_testing_fail_scratch_allocs(3) == bm.OK
        assert bm.bmmc_execute(p.handle, i, o, None) == bm.ERR_OUT_OF_MEMORY
        assert bm.bmmc_execute(p.handle, i, o, None) == bm.ERR_OUT_OF_MEMORY
        opts = p.options()
        assert bm.bmmc_plan_tune_pairs(p.handle, [(i, o)], None, 3) == bm.ERR_OUT_OF_MEMORY
        assert p.options() == opts  # a failed tuning leaves the plan as it was
        # one-pass plans and the entry point that allocates nothing never ask
        q = bm.Plan(n, wl.bit_reverse_matrix(n), 0, 4)
        assert q.info.passes == 1 and q.info.scratch_bytes == 0
    finally:
        assert bm.bmmc_testing_fail_scratch_allocs(0) == bm.OK


def test_tune_argument_errors_without_gpu():
    """bmmc_plan_tune validates before any HIP call: the same buffer rules as
    bmmc_execute and reps in [0, 1000] (these fake addresses are never
    touched)."""
    p = bm.Plan(10, wl.bit_reverse_matrix(10), 0, 4)
    assert bm.bmmc_plan_tune(0, 4096, 8192) == bm.ERR_INVALID_ARG
    assert bm.bmmc_plan_tune(p.handle, 0, 4096) == bm.ERR_INVALID_ARG
    assert bm.bmmc_plan_tune(p.handle, 1 << 20 | 4, 1 << 24) == bm.ERR_INVALID_ARG
    assert bm.bmmc_plan_tune(p.handle, 1 << 20, (1 << 20) + 2048) == bm.ERR_ALIAS
    assert bm.bmmc_plan_tune(p.handle, 1 << 20, 1 << 24, None, -1) == bm.ERR_INVALID_ARG
    assert bm.bmmc_plan_tune(p.handle, 1 << 20, 1 << 24, None, 1001) == bm.ERR_INVALID_ARG


def test_tune_pairs_argument_errors_without_gpu():
    p = bm.Plan(10, wl.bit_reverse_matrix(10), 0, 4)
    assert bm.bmmc_plan_tune_pairs(p.handle, []) == bm.ERR_INVALID_ARG
    pairs = [(1 << 20, 1 << 24), (2 << 20, 2 << 24)]
    assert bm.bmmc_plan_tune_pairs(0, pairs) == bm.ERR_INVALID_ARG
    assert bm.bmmc_plan_tune_pairs(p.handle, pairs + [(0, 1 << 26)]) == bm.ERR_INVALID_ARG
    assert bm.bmmc_plan_tune_pairs(p.handle, pairs + [(3 << 20, (3 << 20) + 64)]) == bm.ERR_ALIAS
    assert bm.bmmc_plan_tune_pairs(p.handle, pairs, None, -1) == bm.ERR_INVALID_ARG
    many = [((k + 1) << 20, (k + 1) << 32) for k in range(4097)]  # one above the limit
    assert bm.bmmc_plan_tune_pairs(p.handle, many) == bm.ERR_INVALID_ARG
    with pytest.raises(bm.BmmcError):
        p.tune(pairs=[])


def test_pass_records_block_order():
    A, c = wl.random_bmmc(16, 5, lambda r: oracle.rank(r) == 16)
    for bmap in (0, 1, 3, 5, 6, 7, 2, 9):
        d = bm.Plan(16, A, c, 4, block_map=bmap).passes()[0]
        # 0 leaves the order to the planner, whose default is output-dense (5)
        assert d.kernel == bm.KERNEL_TILED and d.block_map == (bmap or 5)


def test_destroy_null_is_safe():
    bm.bmmc_plan_destroy(0)


# --------------------------------------------------------------------------
# Classification
# --------------------------------------------------------------------------

def test_classification_of_named_cases():
    P = bm.Plan(20, wl.bit_reverse_matrix(20), 0, 4)
    assert P.info.kind == bm.KIND_BPC and P.info.passes == 1
    assert P.info.unit_bytes == 4 and P.info.tile_log2 == 6
    P = bm.Plan(24, wl.transpose_matrix(12, 12), 0, 4)
    assert P.info.kind == bm.KIND_BPC and P.info.passes == 1
    P = bm.Plan(12, wl.identity_matrix(12), 0, 4)
    assert P.info.kind == bm.KIND_IDENTITY and P.passes()[0].kernel == bm.KERNEL_COPY
    P = bm.Plan(12, wl.identity_matrix(12), 0xABC, 4)
    assert P.info.kind == bm.KIND_IDENTITY and P.passes()[0].kernel == bm.KERNEL_CHUNK_SCATTER
    # whole 2^10-element blocks moved by a random map of the block index: a gather
    Q, _ = _inv(10, 10)
    A = [1 << r for r in range(10)] + [int(q) << 10 for q in Q]
    P = bm.Plan(20, A, 5, 4)
    assert P.passes()[0].kernel == bm.KERNEL_CHUNK
    A, c = _inv(20, 20)
    P = bm.Plan(20, A, c, 4)
    assert P.info.kind == bm.KIND_GENERAL and P.info.passes == 1
    P = bm.Plan(20, A, c, 4, route=bm.ROUTE_TWO_PASS)
    assert P.info.passes == 2 and P.info.route == bm.ROUTE_TWO_PASS
    assert P.info.scratch_bytes == 4 << 20


def test_unit_merging():
    # low bits that stay in place widen the unit up to 16 bytes
    n = 10
    perm = list(range(2)) + list(np.random.default_rng(1).permutation(np.arange(2, n)))
    A = wl.bit_permutation_matrix(perm)
    P = bm.Plan(n, A, 0, 4)
    assert P.info.unit_bytes == 16 and P.info.unit_bits == n - 2
    # a complement bit in the low bits stops the merge
    P = bm.Plan(n, A, 1, 4)
    assert P.info.unit_bytes == 4


def test_bpc_is_always_tiled():
    """Every BPC is a tiled BMMC (one pass)."""
    for seed in range(40):
        n = 8 + seed % 20
        A, c = wl.random_bpc(n, seed)
        P = bm.Plan(n, A, c, 4)
        assert P.info.kind in (bm.KIND_BPC, bm.KIND_IDENTITY)
        assert P.info.passes == 1


def _bruteforce_tiled(A, n, t):
    """Is there a set H of t high bits such that every coset of
    span(low t bits, H) maps onto whole output segments?"""
    from itertools import combinations
    N = 1 << n
    ys = np.array([oracle.map_index(A, 0, i) for i in range(N)], dtype=np.int64)
    for H in combinations(range(t, n), t):
        mask = (1 << t) - 1
        for h in H:
            mask |= 1 << h
        ok = True
        # representatives of the cosets: indices with zero bits in the mask
        for base in range(N):
            if base & mask:
                continue
            members = [base]
            for b in range(n):
                if (mask >> b) & 1:
                    members += [m | (1 << b) for m in members]
            segs = {}
            for m in members:
                y = ys[m]
                segs.setdefault(y >> t, set()).add(y & ((1 << t) - 1))
            if any(len(v) != (1 << t) for v in segs.values()):
                ok = False
                break
        if ok:
            return True
    return False


@pytest.mark.parametrize("n,t", [(6, 2), (7, 2), (8, 3)])
def test_tile_test_matches_bruteforce(n, t):
    rng = np.random.Generator(np.random.PCG64(n * 10 + t))
    agree = tiled = 0
    for k in range(25):
        if k % 3 == 0:
            A, c = wl.random_bpc(n, 500 + k)
        else:
            A, c = _inv(n, 600 + k + 100 * n)
        # 16-byte elements: no unit merging, so the unit map is A itself
        P = bm.Plan(n, A, 0, 16, tile_log2=t)
        got = P.info.kind in (bm.KIND_BPC, bm.KIND_TILED, bm.KIND_IDENTITY)
        want = _bruteforce_tiled(A, n, t)
        assert got == want, (A, t)
        agree += 1
        tiled += want
    assert agree == 25 and 0 < tiled < 25


# --------------------------------------------------------------------------
# Factorisation
# --------------------------------------------------------------------------

def _dense(A, n):
    return ((np.asarray(A, dtype=np.uint64)[:, None] >> np.arange(n, dtype=np.uint64)) & 1
            ).astype(np.int64)


@pytest.mark.parametrize("n,seed", [(14, 1), (16, 2), (20, 20), (24, 4), (30, 30)])
def test_two_pass_factors_multiply_back(n, seed):
    A, c = _inv(n, seed)
    P = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS)
    # a random A is not tiled once n > 2t, so it needs both factors
    assert P.info.kind == bm.KIND_GENERAL
    assert P.info.passes == 2
    (A2, c2), (A1, c1) = P.factors()
    prod = (_dense(A1, n) @ _dense(A2, n)) % 2
    assert np.array_equal(prod, _dense(A, n))
    assert c2 == 0
    # A1.c2 XOR c1 = c  (c2 = 0)
    assert c1 == c
    t = P.info.tile_log2
    # T2 keeps every 2^t-element segment together: low t rows and columns are identity
    D2 = _dense(A2, n)
    assert np.array_equal(D2[:t, :t], np.eye(t, dtype=np.int64))
    assert not D2[:t, t:].any() and not D2[t:, :t].any()
    # T1's tile rows lie in {t, ..., 2t-1}: its inverse's first t columns
    # have no high rows outside that range
    B1 = _dense(oracle.inverse(A1), n)
    assert not B1[2 * t:, :t].any()
    # each factor is a single tiled pass
    for k, d in enumerate(P.passes()):
        assert d.kernel == (bm.KERNEL_CHUNK if k == 0 else bm.KERNEL_TILED)


@pytest.mark.parametrize("skew", [1, -1, 2, -2])
@pytest.mark.parametrize("n,seed", [(16, 1), (20, 2), (24, 3), (30, 4)])
def test_two_pass_rectangular_factors(n, seed, skew):
    """With tiles of input rows of 2^a units and output rows of 2^b (a = t - s,
    b = t + s), A = T1.T2 still holds, T2 keeps every 2^a-element segment
    together and T1's tile rows lie in {a, ..., a+b-1}."""
    A, c = _inv(n, seed)
    t = 6
    P = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS, tile_log2=t, tile_skew=skew)
    assert P.info.passes == 2
    a, b = t - skew, t + skew
    (A2, c2), (A1, c1) = P.factors()
    assert np.array_equal((_dense(A1, n) @ _dense(A2, n)) % 2, _dense(A, n))
    assert c2 == 0 and c1 == c
    D2 = _dense(A2, n)
    assert np.array_equal(D2[:a, :a], np.eye(a, dtype=np.int64))
    assert not D2[:a, a:].any() and not D2[a:, :a].any()
    B1 = _dense(oracle.inverse(A1), n)
    assert not B1[a + b:, :b].any()
    d0, d1 = P.passes()
    assert d0.kernel == bm.KERNEL_CHUNK and d1.kernel == bm.KERNEL_TILED
    assert (d1.in_row_log2, d1.out_row_log2) == (a, b)


# --------------------------------------------------------------------------
# Host replay of the kernel tables against the oracle
# --------------------------------------------------------------------------

def _cases():
    cases = []
    for e in (1, 2, 4, 8, 16):
        cases.append(("bitrev", 12, e, dict()))
        cases.append(("transpose", 12, e, dict()))
        cases.append(("bpc", 13, e, dict()))
        cases.append(("general", 12, e, dict()))
        cases.append(("general", 12, e, dict(route=bm.ROUTE_TWO_PASS)))
        cases.append(("general", 11, e, dict(route=bm.ROUTE_NAIVE)))
        cases.append(("complement", 10, e, dict()))
    for t in (1, 2, 3, 4, 5):
        cases.append(("general", 12, 4, dict(tile_log2=t)))
        cases.append(("bpc", 12, 4, dict(tile_log2=t)))
    for it in (1, 2, 3):
        cases.append(("general", 16, 4, dict(iters_log2=it)))
        cases.append(("bitrev", 16, 4, dict(iters_log2=it)))
    for e in (1, 4, 16):
        cases.append(("general", 15, e, dict(launch=bm.LAUNCH_ONE_TILE)))
        cases.append(("general", 15, e, dict(launch=bm.LAUNCH_PERSISTENT, grid_log2=2)))
        cases.append(("bpc", 15, e, dict(launch=bm.LAUNCH_PERSISTENT, grid_log2=2,
                                         walk=bm.WALK_INTERLEAVED)))
    for e in (1, 4, 16):
        cases.append(("general", 15, e, dict(launch=bm.LAUNCH_STREAMED, grid_log2=2)))
        cases.append(("bpc", 16, e, dict(launch=bm.LAUNCH_STREAMED, walk=bm.WALK_INTERLEAVED)))
    for bmap in (2, 3, 4, 5, 17):
        cases.append(("general", 16, 4, dict(block_map=bmap)))
        cases.append(("bitrev", 16, 16, dict(block_map=bmap, launch=bm.LAUNCH_ONE_TILE)))
    for bmap in (3, 4, 5, 6, 7):
        cases.append(("bitrev", 17, 4, dict(block_map=bmap, launch=bm.LAUNCH_PERSISTENT,
                                            grid_log2=3)))
        cases.append(("general", 17, 8, dict(block_map=bmap, launch=bm.LAUNCH_STREAMED,
                                             walk=bm.WALK_INTERLEAVED, grid_log2=2)))
    cases.append(("general", 14, 4, dict(no_swizzle=1)))
    cases.append(("general", 5, 4, dict()))
    cases.append(("general", 2, 4, dict()))
    cases.append(("general", 1, 4, dict()))
    cases.append(("bitrev", 1, 1, dict()))
    cases.append(("bitrev", 3, 16, dict()))
    cases.append(("general", 18, 4, dict()))
    return cases


def _matrix(kind, n, seed):
    if kind == "bitrev":
        return wl.bit_reverse_matrix(n), 0
    if kind == "transpose":
        return wl.transpose_matrix(n // 2, n - n // 2), 0
    if kind == "bpc":
        return wl.random_bpc(n, seed)
    if kind == "complement":
        return wl.identity_matrix(n), (0x2AAAAAAAA + seed) & ((1 << n) - 1)
    return _inv(n, seed)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "%s-n%d-e%d-%s" % (
    c[0], c[1], c[2], "-".join("%s%s" % kv for kv in sorted(c[3].items()))))
def test_replay_matches_oracle(case):
    kind, n, e, kw = case
    A, c = _matrix(kind, n, 1000 + n + e)
    P = bm.Plan(n, A, c, e, **kw)
    x = wl.fill_random_bytes(n, e, seed=n * 31 + e)
    got = run_plan_on_host(P, x)
    want = oracle.apply(A, c, x)
    assert np.array_equal(got, want), P.describe()


def test_replay_full_size_transpose_tables():
    """The 4096 x 4096 fp32 transpose plan, replayed over all 4096 tiles."""
    A, c = wl.workload_matrix("c2")
    P = bm.Plan(24, A, c, 4)
    x = wl.workload_data("c2")
    got = run_plan_on_host(P, x)
    assert np.array_equal(got.view(np.uint32), x.reshape(4096, 4096).T.reshape(-1).view(np.uint32))


def test_replay_detects_planted_table_errors():
    from emulate import replay_pass
    A, c = _inv(12, 5)
    P = bm.Plan(12, A, c, 4)
    # a read map that is no longer a bijection reads a slot twice
    d = P.passes()[0]
    d.st_lds[3] = d.st_lds[2]
    with pytest.raises(ReplayError):
        replay_pass(d)
    # a still-bijective but wrong map is caught by the comparison with the oracle
    d = P.passes()[0]
    d.st_lds[3] ^= d.st_lds[2]
    x = np.arange(1 << 12, dtype=np.int32)
    got = x[replay_pass(d)]
    assert not np.array_equal(got, oracle.apply(A, c, x))


# --------------------------------------------------------------------------
# LDS banks under the planner's model
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind,n,e,skew", [("bitrev", 20, 4, 0), ("transpose", 24, 4, 0),
                                           ("general", 20, 4, 0), ("general", 30, 4, 0),
                                           ("bpc", 27, 16, 0), ("bitrev", 28, 4, 0),
                                           ("bitrev", 28, 4, 1), ("bitrev", 28, 4, -1),
                                           ("general", 30, 4, 1), ("bpc", 27, 16, 1),
                                           ("transpose", 24, 4, -1), ("bitrev", 28, 4, 9),
                                           ("general", 30, 4, 9), ("bpc", 27, 16, 9)])
def test_swizzle_makes_reads_conflict_free(kind, n, e, skew):
    """skew 9 stands for 512 threads per tile (square tiles)."""
    A, c = _matrix(kind, n, 7)
    kw = {}
    if skew:
        kw = dict(tile_log2=7 if e == 4 else 6)
        kw.update(dict(tile_threads_log2=9) if skew == 9 else dict(tile_skew=skew))
    P = bm.Plan(n, A, c, e, **kw)
    if skew == 9:
        assert P.passes()[-1].threads_log2 == 9
    d = P.passes()[-1]
    assert d.kernel == bm.KERNEL_TILED
    U = 1 << d.unit_log2
    ra = tiled_read_addresses(d)
    wa = tiled_write_addresses(d)
    CB = U << min(4 - d.unit_log2, d.t)
    lanes = len(ra)
    # conflict-free under the measured model (32 banks, half a wave per
    # cycle for 4-byte reads; 8 lanes per cycle for 16-byte accesses), and
    # under a 64-bank full-wave model
    for banks in (32, 64):
        ideal_r = -(-lanes * max(U, 4) // (4 * banks))
        ideal_w = -(-lanes * CB // (4 * banks))
        assert bank_cycles(ra, U, banks) == ideal_r, (banks, P.describe())
        assert bank_cycles(wa, CB, banks) == ideal_w
    # the plain layout is conflicted for the transpose (the ablation)
    if kind == "transpose" and not skew:
        P0 = bm.Plan(n, A, c, e, no_swizzle=1)
        r0 = tiled_read_addresses(P0.passes()[0])
        assert bank_cycles(r0, U, 64) > bank_cycles(ra, U, 64)


def _top_bits(tab, k):
    return [int(v).bit_length() - 1 for v in tab[:k]]


def _reduced_out_top_bits(d, unit_log2):
    """Top bits of the output block offsets reduced modulo the tile's output
    span (the in-segment bits and the segment vectors in st_out): what a block
    bit moves the tile's set of output segments by."""
    basis = []  # (pivot, vector), fully reduced
    def reduce(v):
        for p, b in basis:
            if (v >> p) & 1:
                v ^= b
        return v
    def add(v):
        v = reduce(v)
        if v:
            p = v.bit_length() - 1
            for i, (q, b) in enumerate(basis):
                if (b >> p) & 1:
                    basis[i] = (q, b ^ v)
            basis.append((p, v))
    for b in range(unit_log2 + d.t):
        add(1 << b)
    for v in d.st_out:
        add(int(v))
    return [reduce(int(v)).bit_length() - 1 for v in d.out_blk[:d.blk_bits]]


@pytest.mark.parametrize("seed", range(4))
def test_locality_block_orders(seed):
    """Block orders 3-7 draw block vectors nearest first on the input side
    (input-aligned) or the output side (output-aligned); the tiles stay a
    partition of the array, which the replay tests check."""
    n, e = 22, 4
    A, c = wl.random_bmmc(n, seed, lambda r: oracle.rank(r) == n)

    def desc(mode, launch):
        P = bm.Plan(n, A, c, e, launch=launch, block_map=mode)
        return bm.bmmc_plan_get_pass(P.handle, 0)

    d4 = desc(4, bm.LAUNCH_ONE_TILE)
    d5 = desc(5, bm.LAUNCH_ONE_TILE)
    m = d4.blk_bits
    ins = _top_bits(d4.in_blk, m)
    outs = _reduced_out_top_bits(d5, 2)
    assert ins == sorted(ins) and len(set(ins)) == m
    assert outs == sorted(outs) and len(set(outs)) == m
    # output-aligned vectors move the output by single bits above the segment
    assert outs[0] >= 2 + d5.t and outs[-1] <= 2 + n - 1
    d3 = desc(3, bm.LAUNCH_ONE_TILE)
    # alternating picks; a candidate already spanned by earlier picks is skipped
    even = _top_bits(d3.in_blk, m)[0::2]
    odd = _reduced_out_top_bits(d3, 2)[1::2]
    assert even[0] == ins[0] and even == sorted(even) and set(even) <= set(ins)
    assert odd[0] == outs[0] and odd == sorted(odd) and set(odd) <= set(outs)
    # range walk: the concurrent (top grid_log2) bits take the output side
    d6 = desc(6, bm.LAUNCH_PERSISTENT)
    g = d6.grid_log2
    assert 0 < g < m
    assert _reduced_out_top_bits(d6, 2)[m - g:] == outs[:g]
    # the other bits take input-aligned vectors, nearest first, skipping any
    # that the concurrent picks already span
    low = _top_bits(d6.in_blk, m)[:m - g]
    assert low == sorted(low) and set(low) <= set(ins)


# --------------------------------------------------------------------------
# Maximum sizes: sampled replay of the kernel tables against the oracle
# --------------------------------------------------------------------------

MAX_CASES = [  # (n, elem_bytes, kind, plan options): up to 2^36 bytes per array
    (32, 1, "general", {}),
    (32, 1, "general", dict(launch=bm.LAUNCH_ONE_TILE)),
    (32, 1, "general", dict(route=bm.ROUTE_TWO_PASS)),
    (32, 16, "general", {}),
    (32, 16, "general", dict(launch=bm.LAUNCH_ONE_TILE, block_map=5)),
    (32, 16, "bitrev", {}),
    (32, 4, "bitrev", dict(tile_log2=7, block_map=6)),
    (31, 8, "bpc", dict(block_map=3)),
    (32, 2, "transpose", dict(launch=bm.LAUNCH_STREAMED)),
    (32, 1, "general", dict(route=bm.ROUTE_NAIVE)),
    (32, 16, "general", dict(tile_log2=2, launch=bm.LAUNCH_ONE_TILE)),
    (32, 4, "bitrev", dict(tile_log2=7, tile_skew=1)),
    (32, 8, "general", dict(tile_skew=-1, launch=bm.LAUNCH_PERSISTENT)),
    (32, 4, "bitrev", dict(tile_log2=7, tile_threads_log2=9, launch=bm.LAUNCH_STREAMED)),
    (32, 16, "general", dict(tile_threads_log2=9, launch=bm.LAUNCH_ONE_TILE)),
    (32, 4, "bitrev", dict(tile_log2=7, split_stage=1)),
    (32, 16, "general", dict(split_stage=1, tile_skew=1)),
    (32, 1, "general", dict(split_stage=1, route=bm.ROUTE_TWO_PASS)),
    (31, 8, "bpc", dict(split_stage=1, tile_threads_log2=9, tile_skew=-1)),
    (32, 2, "transpose", dict(split_stage=1, launch=bm.LAUNCH_ONE_TILE, block_map=6)),
]


def _max_matrix(kind, n, seed):
    if kind == "bitrev":
        return wl.bit_reverse_matrix(n), 0
    if kind == "transpose":
        return wl.transpose_matrix(n // 2, n - n // 2), 0
    if kind == "bpc":
        return wl.random_bpc(n, seed)
    return wl.random_bmmc(n, seed, lambda r: oracle.rank(r) == n)


def _sampled_blocks(nblk, seed, count=48):
    rng = np.random.Generator(np.random.PCG64(seed))
    edge = [0, 1, 2, nblk - 1, nblk - 2, nblk // 2, nblk // 2 - 1]
    return [b for b in edge if 0 <= b < nblk] + [int(v) for v in rng.integers(0, nblk, size=count)]


@pytest.mark.parametrize("case", MAX_CASES, ids=lambda c: "n%d-e%d-%s-%s" % (
    c[0], c[1], c[2], "-".join("%s%s" % kv for kv in sorted(c[3].items()))))
def test_maximum_size_plans_sampled(case):
    """Plans at the largest sizes the ABI accepts (2^32 elements, 2^36 bytes):
    sampled tiles or chunks of every pass, including the first and last
    blocks, replayed through the tables and compared with the oracle's map
    of that pass's factor; all offsets must stay below the array's size."""
    n, e, kind, kw = case
    A, c = _max_matrix(kind, n, 3100 + n + e)
    P = bm.Plan(n, A, c, e, **kw)
    assert (e << n) <= 1 << 36
    elog = e.bit_length() - 1
    total = 0
    for k, d in enumerate(P.passes()):
        fa, fc = P.factors()[k]
        total += check_pass_sampled(d, fa, fc, elog, _sampled_blocks(1 << d.blk_bits, k + n),
                                    oracle.map_indices)
    assert total > 0


def test_sampled_replay_catches_planted_mistakes():
    """A wrong table entry, a wrong factor or a misaligned base each fail the
    sampled replay (the mistakes are planted in the host copy of the tables)."""
    n, e = 24, 4
    A, c = _max_matrix("general", n, 9)
    P = bm.Plan(n, A, c, e)
    d = P.passes()[0]
    fa, fc = P.factors()[0]
    blocks = _sampled_blocks(1 << d.blk_bits, 1)
    assert check_pass_sampled(d, fa, fc, 2, blocks, oracle.map_indices) > 0
    with pytest.raises(ReplayError):
        check_pass_sampled(d, fa, fc ^ 1, 2, blocks, oracle.map_indices)
    bad = bm.bmmc_pass_desc.from_buffer_copy(d)
    bad.out_blk[3] ^= bad.out_blk[4]
    with pytest.raises(ReplayError):
        check_pass_sampled(bad, fa, fc, 2, blocks, oracle.map_indices)
    bad = bm.bmmc_pass_desc.from_buffer_copy(d)
    bad.in_blk[0] ^= 16
    with pytest.raises(ReplayError):
        check_pass_sampled(bad, fa, fc, 2, blocks, oracle.map_indices)
    bad = bm.bmmc_pass_desc.from_buffer_copy(d)
    bad.st_lds[2], bad.st_lds[3] = bad.st_lds[3], bad.st_lds[2]
    with pytest.raises(ReplayError):
        check_pass_sampled(bad, fa, fc, 2, blocks, oracle.map_indices)



def _desc_bytes(d):
    import ctypes
    return ctypes.string_at(ctypes.addressof(d), ctypes.sizeof(d))


@pytest.mark.parametrize("case", [
    ("general", 20, 4, {}), ("general", 16, 1, dict(route=bm.ROUTE_TWO_PASS)),
    ("bitrev", 24, 4, {}), ("bitrev", 12, 16, {}), ("bpc", 27, 16, {}),
    ("general", 18, 8, dict(launch=bm.LAUNCH_ONE_TILE, iters_log2=2)),
    ("general", 22, 2, dict(block_map=5, tile_log2=7)), ("bpc", 14, 4, dict(no_swizzle=1)),
    ("general", 20, 4, dict(launch=bm.LAUNCH_STREAMED, depth=1, grid_log2=6, walk=2)),
    ("general", 9, 4, dict(route=bm.ROUTE_NAIVE)), ("identity", 12, 4, {}),
    ("complement", 12, 4, {}), ("general", 30, 4, dict(cache_hint=1)),
    ("bitrev", 28, 4, dict(tile_log2=7, tile_skew=1)), ("general", 24, 4, dict(tile_skew=-2)),
    ("bpc", 27, 16, dict(tile_skew=1, launch=bm.LAUNCH_PERSISTENT)),
    ("bitrev", 28, 4, dict(tile_log2=7, tile_threads_log2=9, launch=bm.LAUNCH_STREAMED)),
    ("general", 20, 4, dict(tile_threads_log2=9, tile_skew=1)),
], ids=lambda c: "%s-n%d-e%d-%s" % (c[0], c[1], c[2],
                                    "-".join("%s%s" % kv for kv in sorted(c[3].items()))))
def test_options_rebuild_the_same_tables(case):
    """bmmc_plan_get_options writes every choice out; creating a plan from
    them gives byte-identical kernel tables, and the explicit options are a
    fixed point."""
    kind, n, e, kw = case
    if kind == "identity":
        A, c = wl.identity_matrix(n), 0
    elif kind == "complement":
        A, c = wl.identity_matrix(n), 0x5A5 & ((1 << n) - 1)
    elif kind == "bitrev":
        A, c = wl.bit_reverse_matrix(n), 0
    elif kind == "bpc":
        A, c = wl.random_bpc(n, n)
    else:
        A, c = wl.random_bmmc(n, n, lambda r: oracle.rank(r) == n)
    P = bm.Plan(n, A, c, e, **kw)
    opts = P.options()
    Q = bm.Plan(n, A, c, e, **opts)
    assert Q.info.passes == P.info.passes and Q.info.tile_log2 == P.info.tile_log2
    for dp, dq in zip(P.passes(), Q.passes()):
        assert _desc_bytes(dp) == _desc_bytes(dq)
    assert Q.options() == opts
    for k, v in kw.items():
        assert opts[k] == v


# --------------------------------------------------------------------------
# Rectangular tiles (tile_skew)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name,skew,threads", [("c3", 1, 8), ("c3", -1, 8), ("c4", 1, 8),
                                               ("c4", -1, 8), ("c2", 1, 8), ("c5", 1, 8),
                                               ("c5", -1, 8), ("c3", 0, 9), ("c3", 1, 9),
                                               ("c4", 0, 9), ("c5", -1, 9)])
def test_skewed_tiles_at_workload_size(name, skew, threads):
    """A skewed tile keeps the square tile's 2^(2t) units with input rows of
    2^(t - s) units and output rows of 2^(t + s); at the workloads' full
    sizes, sampled tiles replay to the oracle's map (range, exactly-once and
    destination checks on every unit of each sampled tile)."""
    w = wl.WORKLOADS[name]
    A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == w.n)
    t = 7 if w.elem_bytes == 4 else 6
    P = bm.Plan(w.n, A, c, w.elem_bytes, tile_log2=t, tile_skew=skew, tile_threads_log2=threads)
    assert P.info.passes == 1
    d = P.passes()[0]
    assert (d.t, d.in_row_log2, d.out_row_log2) == (t, t - skew, t + skew)
    assert d.threads_log2 == threads and P.describe()["tile_threads"] == 1 << threads
    assert P.describe()["tile_skew"] == skew and P.options()["tile_skew"] == skew
    checked = check_pass_sampled(d, *P.factors()[0], w.elem_bytes.bit_length() - 1,
                                 _sampled_blocks(1 << d.blk_bits, 77), oracle.map_indices)
    assert checked >= 55 * (1 << (2 * t))


def test_skew_argument_errors():
    n = 20
    A = wl.bit_reverse_matrix(n)
    for bad in (dict(tile_skew=9), dict(tile_skew=-9), dict(tile_log2=3, tile_skew=3)):
        with pytest.raises(bm.BmmcError):
            bm.Plan(n, A, 0, 4, **bad)
    # rows shorter than the kernel's 16-byte chunk are refused
    with pytest.raises(bm.BmmcError):
        bm.Plan(n, A, 0, 4, tile_log2=6, tile_skew=5)
    # the two-pass route of a general matrix takes rectangular tiles too (its
    # relabel then moves segments as long as the tile's input rows); a BPC
    # takes one tile pass whatever the route asks, skewed if asked
    G, c = _inv(n, 3)
    for skew in (1, -1, 2):
        P = bm.Plan(n, G, c, 4, tile_log2=6, tile_skew=skew, route=bm.ROUTE_TWO_PASS)
        assert P.info.passes == 2 and P.describe()["tile_skew"] == skew
        d = P.passes()[1]
        assert (d.in_row_log2, d.out_row_log2) == (6 - skew, 6 + skew)
    with pytest.raises(bm.BmmcError):
        bm.Plan(n, G, c, 4, tile_log2=6, tile_skew=6, route=bm.ROUTE_TWO_PASS)
    P = bm.Plan(n, A, 0, 4, tile_skew=1, route=bm.ROUTE_TWO_PASS)
    assert P.info.passes == 1 and P.describe()["tile_skew"] == 1


def test_tune_candidates_rebuild_distinct_plans():
    """bmmc_plan_tune_candidates lists options that rebuild distinct tables,
    the planner's own plan first, including rectangular tiles; a plan with no
    tile pass has none."""
    for name in ("c4", "c3", "c5"):
        w = wl.WORKLOADS[name]
        A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == w.n)
        P = bm.Plan(w.n, A, c, w.elem_bytes)
        cands = bm.bmmc_plan_tune_candidates(P.handle)
        assert P.tune_candidates() == cands
        assert 20 <= len(cands) <= 160
        digests = set()
        for k, o in enumerate(cands):
            Q = bm.Plan(w.n, A, c, w.elem_bytes, **o)
            assert Q.options() == o
            digests.add(b"".join(_desc_bytes(d) for d in Q.passes()))
            if k == 0:
                assert [_desc_bytes(d) for d in Q.passes()] == [_desc_bytes(d) for d in P.passes()]
        assert len(digests) == len(cands)
        assert {o["tile_skew"] for o in cands} >= {0, 1, -1, 2, -2}
        assert {o["tile_threads_log2"] for o in cands} == {8, 9}
        assert {o["split_stage"] for o in cands} == {0, 1}
        # buffer loads where the array holds at most 2^31 bytes (c4 holds 2^32)
        assert {o["buffer_loads"] for o in cands} == ({0} if name == "c4" else {0, 1})
        for o in cands:
            if o["buffer_loads"]:
                assert o["launch"] == bm.LAUNCH_ONE_TILE and o["split_stage"] == 0
                assert dict(o, buffer_loads=0) in cands
    R = bm.Plan(12, wl.identity_matrix(12), 5, 4)
    assert bm.bmmc_plan_tune_candidates(R.handle) == []


def test_thread_count_option_errors():
    A = wl.bit_reverse_matrix(20)
    with pytest.raises(bm.BmmcError):
        bm.Plan(20, A, 0, 4, tile_threads_log2=10)
    # the wide kernels exist for one tile per workgroup only, not the
    # iterated variant
    with pytest.raises(bm.BmmcError):
        bm.Plan(20, A, 0, 4, tile_log2=7, tile_threads_log2=9, launch=bm.LAUNCH_ONE_TILE,
                iters_log2=1)
    # tiles of at most 256 chunks use one thread per chunk whatever is asked
    P = bm.Plan(20, A, 0, 4, tile_log2=4, tile_threads_log2=9)
    assert P.passes()[0].threads_log2 == 2 * 4 - 2


# --------------------------------------------------------------------------
# Split staging: one-tile launches whose tiles pass LDS half at a time
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kw", [
    dict(launch=bm.LAUNCH_PERSISTENT), dict(launch=bm.LAUNCH_STREAMED),
    dict(launch=bm.LAUNCH_ONE_TILE, iters_log2=1)])
def test_split_stage_needs_one_tile_per_workgroup(kw):
    A, c = wl.random_bmmc(20, 5, lambda r: oracle.rank(r) == 20)
    with pytest.raises(bm.BmmcError) as e:
        bm.Plan(20, A, c, 4, split_stage=1, **kw)
    assert e.value.status == bm.ERR_INVALID_ARG


def test_split_stage_argument_errors():
    A, c = wl.random_bmmc(20, 5, lambda r: oracle.rank(r) == 20)
    for bad in (-1, 2):
        with pytest.raises(bm.BmmcError) as e:
            bm.Plan(20, A, c, 4, split_stage=bad)
        assert e.value.status == bm.ERR_INVALID_ARG
    # a tile of at most 256 chunks is one pass per thread: nothing to split
    with pytest.raises(bm.BmmcError) as e:
        bm.Plan(20, A, c, 4, split_stage=1, tile_log2=4)
    assert e.value.status == bm.ERR_INVALID_ARG


@pytest.mark.parametrize("kind,n,e,kw", [
    ("bitrev", 18, 4, dict(tile_log2=7)),
    ("bitrev", 18, 4, dict(tile_log2=7, tile_skew=1, tile_threads_log2=9)),
    ("general", 20, 4, {}),
    ("general", 19, 4, dict(tile_skew=1)),
    ("general", 18, 16, dict(tile_skew=2)),
    ("bpc", 18, 16, dict(tile_threads_log2=9)),
    ("transpose", 18, 4, dict(block_map=6)),
    ("general", 16, 2, dict(route=bm.ROUTE_TWO_PASS)),
    ("general", 17, 8, dict(cache_hint=1, block_map=9)),
])
def test_split_stage_plans_replay(kind, n, e, kw):
    """Split plans: a one-tile launch with half a tile of LDS whose kernel
    tables, replayed half by half on the host (every LDS slot of a half
    written and read once, in range), reproduce the oracle's permutation;
    the options rebuild the same tables."""
    A, c = _max_matrix(kind, n, 40 + n)
    P = bm.Plan(n, A, c, e, split_stage=1, **kw)
    tiled = [d for d in P.passes() if d.kernel == bm.KERNEL_TILED]
    assert tiled and all(d.split_stage == 1 and d.launch == bm.LAUNCH_ONE_TILE for d in tiled)
    for d in tiled:
        assert 2 * d.lds_bytes == (1 << d.unit_log2) << (2 * d.t)
    assert P.describe()["split_stage"] == 1
    x = wl.fill_random_bytes(n, e, 77)
    assert np.array_equal(run_plan_on_host(P, x), oracle.apply(A, c, x))
    o = P.options()
    assert o["split_stage"] == 1
    Q = bm.Plan(n, A, c, e, **o)
    assert [_desc_bytes(d) for d in Q.passes()] == [_desc_bytes(d) for d in P.passes()]


def test_split_stage_keeps_bank_costs_and_coalescing():
    """On the benchmark's large workloads the split tables keep the lanes'
    LDS banks of the whole-tile tables at the tuned shapes (the chosen
    functional leaves the lane bits' costs unchanged) and pass the replay's
    coalescing check at full size on sampled tiles."""
    for name, perm, kw in (("c4", 0, dict(tile_log2=7)),
                           ("c3", 0, dict(tile_log2=7, tile_skew=1, tile_threads_log2=9)),
                           ("c5", 10, dict(tile_log2=6, tile_skew=2)),
                           ("c2", 0, dict(tile_log2=7, tile_skew=1))):
        w = wl.WORKLOADS[name]
        A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == w.n, perm_index=perm)
        whole = bm.Plan(w.n, A, c, w.elem_bytes, launch=bm.LAUNCH_ONE_TILE, **kw)
        half = bm.Plan(w.n, A, c, w.elem_bytes, split_stage=1, **kw)
        d0, d1 = whole.passes()[0], half.passes()[0]
        U = 1 << d0.unit_log2
        CB = U << min(4 - d0.unit_log2, d0.t)
        for addrs, size in ((tiled_read_addresses, U), (tiled_write_addresses, CB)):
            for banks in (32, 64):
                assert bank_cycles(addrs(d1), size, banks) <= bank_cycles(addrs(d0), size, banks), name
        fa, fc = half.factors()[0]
        assert check_pass_sampled(d1, fa, fc, w.elem_bytes.bit_length() - 1,
                                  _sampled_blocks(1 << d1.blk_bits, 3), oracle.map_indices) > 0


def test_split_replay_catches_planted_mistakes():
    """The half-by-half replay rejects split tables run as one staging, whole
    tables run as two halves, and a pass bit moved out of the top position."""
    A, c = wl.random_bmmc(18, 3, lambda r: oracle.rank(r) == 18)
    from emulate import replay_pass
    P = bm.Plan(18, A, c, 4, split_stage=1, tile_log2=7)
    d = P.passes()[0]
    replay_pass(d)
    bad = bm.bmmc_pass_desc.from_buffer_copy(d)
    bad.split_stage = 0
    with pytest.raises(ReplayError):
        replay_pass(bad)
    W = bm.Plan(18, A, c, 4, launch=bm.LAUNCH_ONE_TILE, tile_log2=7).passes()[0]
    bad = bm.bmmc_pass_desc.from_buffer_copy(W)
    bad.split_stage = 1
    bad.lds_bytes //= 2
    with pytest.raises(ReplayError):
        replay_pass(bad)
    g = tiled_geometry(d.unit_log2, d.t, d.threads_log2)
    top = g["ntl"] + g["jl"] - 1
    bad = bm.bmmc_pass_desc.from_buffer_copy(d)
    for tab in (bad.ld_in, bad.ld_lds):
        tab[top], tab[top - 1] = tab[top - 1], tab[top]
    with pytest.raises(ReplayError):
        replay_pass(bad)


# --------------------------------------------------------------------------
# Buffer loads: one-tile launches that read the input by 32-bit offsets
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kw", [
    dict(launch=bm.LAUNCH_PERSISTENT), dict(launch=bm.LAUNCH_STREAMED),
    dict(launch=bm.LAUNCH_ONE_TILE, iters_log2=1), dict(split_stage=1)])
def test_buffer_loads_need_one_whole_tile_per_workgroup(kw):
    A, c = wl.random_bmmc(20, 5, lambda r: oracle.rank(r) == 20)
    with pytest.raises(bm.BmmcError) as e:
        bm.Plan(20, A, c, 4, buffer_loads=1, **kw)
    assert e.value.status == bm.ERR_INVALID_ARG


def test_buffer_loads_argument_errors():
    A = wl.bit_reverse_matrix(20)
    for bad in (-1, 2):
        with pytest.raises(bm.BmmcError) as e:
            bm.Plan(20, A, 0, 4, buffer_loads=bad)
        assert e.value.status == bm.ERR_INVALID_ARG
    # units of 1 and 2 bytes (bit reversal merges no element bits into a unit)
    for elem in (1, 2):
        with pytest.raises(bm.BmmcError) as e:
            bm.Plan(20, A, 0, elem, buffer_loads=1)
        assert e.value.status == bm.ERR_INVALID_ARG
    # 32-bit offsets: arrays of at most 2^31 bytes
    with pytest.raises(bm.BmmcError) as e:
        bm.Plan(30, wl.bit_reverse_matrix(30), 0, 4, buffer_loads=1)
    assert e.value.status == bm.ERR_INVALID_ARG
    with pytest.raises(bm.BmmcError) as e:
        bm.Plan(28, wl.bit_reverse_matrix(28), 0, 16, buffer_loads=1)
    assert e.value.status == bm.ERR_INVALID_ARG
    for n, elem in ((29, 4), (27, 16), (28, 8)):
        P = bm.Plan(n, wl.bit_reverse_matrix(n), 0, elem, buffer_loads=1)
        d = P.passes()[0]
        assert d.buffer_loads == 1 and d.launch == bm.LAUNCH_ONE_TILE
        assert d.nbits + d.unit_log2 == 31
    # the launch left to the planner becomes one tile per workgroup
    P = bm.Plan(20, A, 0, 4, buffer_loads=1)
    assert P.describe()["kernels"] == ["one_tile"] and P.describe()["buffer_loads"] == 1


@pytest.mark.parametrize("kind,n,e,kw", [
    ("bitrev", 18, 4, dict(tile_log2=7)),
    ("bitrev", 18, 4, dict(tile_log2=7, tile_skew=1, tile_threads_log2=9)),
    ("general", 20, 4, {}),
    ("general", 19, 8, dict(tile_skew=-1)),
    ("bpc", 18, 16, dict(tile_log2=5, tile_skew=2, tile_threads_log2=9)),
    ("transpose", 18, 4, dict(block_map=8)),
    ("general", 16, 4, dict(route=bm.ROUTE_TWO_PASS)),
    ("general", 17, 8, dict(cache_hint=1, block_map=9)),
])
def test_buffer_load_plans_replay(kind, n, e, kw):
    """A buffer-load plan has the tables of the global-load plan of the same
    options (only the load form differs), replays to the oracle's
    permutation on the host, and its options rebuild it."""
    A, c = _max_matrix(kind, n, 60 + n)
    P = bm.Plan(n, A, c, e, buffer_loads=1, **kw)
    G = bm.Plan(n, A, c, e, launch=bm.LAUNCH_ONE_TILE, **kw)
    tiled = [d for d in P.passes() if d.kernel == bm.KERNEL_TILED]
    assert tiled and all(d.buffer_loads == 1 for d in tiled)
    plain = []
    for d in P.passes():
        q = bm.bmmc_pass_desc.from_buffer_copy(d)
        q.buffer_loads = 0
        plain.append(_desc_bytes(q))
    assert plain == [_desc_bytes(d) for d in G.passes()]
    x = wl.fill_random_bytes(n, e, 78)
    assert np.array_equal(run_plan_on_host(P, x), oracle.apply(A, c, x))
    o = P.options()
    assert o["buffer_loads"] == 1
    Q = bm.Plan(n, A, c, e, **o)
    assert [_desc_bytes(d) for d in Q.passes()] == [_desc_bytes(d) for d in P.passes()]


def test_buffer_load_replay_rejects_bad_descriptors():
    """The replay refuses buffer loads on a launch or an array they do not
    serve."""
    from emulate import replay_pass
    A, c = wl.random_bmmc(18, 3, lambda r: oracle.rank(r) == 18)
    d = bm.Plan(18, A, c, 4, buffer_loads=1).passes()[0]
    replay_pass(d)
    for field, value in (("buffer_loads", 2), ("iters_log2", 1), ("unit_log2", 1),
                         ("nbits", 30)):
        bad = bm.bmmc_pass_desc.from_buffer_copy(d)
        setattr(bad, field, value)
        with pytest.raises(ReplayError):
            replay_pass(bad)
    P = bm.Plan(18, A, c, 4, launch=bm.LAUNCH_PERSISTENT)
    bad = bm.bmmc_pass_desc.from_buffer_copy(P.passes()[0])
    bad.buffer_loads = 1
    with pytest.raises(ReplayError):
        replay_pass(bad)


@pytest.mark.parametrize("fixed", [
    dict(launch=bm.LAUNCH_STREAMED), dict(tile_skew=1), dict(tile_threads_log2=9),
    dict(split_stage=1), dict(block_map=6), dict(route=bm.ROUTE_TWO_PASS), dict(tile_log2=6),
    dict(buffer_loads=1)])
def test_tune_candidates_keep_what_the_caller_fixed(fixed):
    """Every candidate keeps an option the caller set at plan creation; the
    options left open still vary."""
    n = 28
    A, c = wl.workload_matrix("c3")
    if "route" in fixed:  # a general matrix, so that the two-pass route applies
        n = 24
        A, c = wl.random_bmmc(n, 24, lambda r: oracle.rank(r) == n)
    P = bm.Plan(n, A, c, 4, **fixed)
    cands = P.tune_candidates()
    assert cands
    for k, v in fixed.items():
        if k == "route":
            # two passes each, square and rectangular tiles
            assert {o["route"] for o in cands} == {v}
            assert all(bm.Plan(n, A, c, 4, **o).info.passes == 2 for o in cands)
            assert {o["tile_skew"] for o in cands} >= {0, 1, -1}
        else:
            assert {o[k] for o in cands} == {v}, k
    if "block_map" not in fixed:
        assert len({o["block_map"] for o in cands}) >= 4
    if "split_stage" in fixed:
        assert {o["launch"] for o in cands} == {bm.LAUNCH_ONE_TILE}
    if fixed.get("launch") == bm.LAUNCH_STREAMED:
        assert {o["split_stage"] for o in cands} == {0}
        assert {o["buffer_loads"] for o in cands} == {0}
    if "buffer_loads" in fixed:
        assert {o["launch"] for o in cands} == {bm.LAUNCH_ONE_TILE}
        assert {o["split_stage"] for o in cands} == {0}
