"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison is bit-exact (bytes).  Outputs are pre-filled with a
sentinel so that a missed write cannot pass.  Small cases cover every kind,
route, element size, tile side and iteration count, including the edge cases
n = 1 and n = 2t; the five workloads run at full size with the launch
configuration the benchmark times, checked in full where the host can hold
the oracle's output and on sampled indices beyond that.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import bmmc_affine_index_amd as bm
from bmmc_affine_index_amd import workloads as wl

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5
HOST_THREADS = max(1, min(16, os.cpu_count() or 1))


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(A, c, x, **plan_kw):
    """Permute host array x on the GPU; returns (host result, plan)."""
    torch = _torch()
    n = len(A)
    raw = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
    elem = raw.size >> n
    P = bm.Plan(n, A, c, elem, **plan_kw)
    d_in = torch.from_numpy(raw.copy()).to("cuda:0")
    d_out = torch.full_like(d_in, SENTINEL)
    P(d_in, d_out)
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(x.dtype).reshape(x.shape)
    return got, P


def _inv(n, seed):
    return wl.random_bmmc(n, seed, lambda r: oracle.rank(r) == n)


def _matrix(kind, n, seed):
    if kind == "bitrev":
        return wl.bit_reverse_matrix(n), 0
    if kind == "transpose":
        return wl.transpose_matrix(n // 2, n - n // 2), 0
    if kind == "bpc":
        return wl.random_bpc(n, seed)
    if kind == "complement":
        return wl.identity_matrix(n), ((1 << n) - 1) & (0x5A5A5A5A5 ^ seed)
    if kind == "identity":
        return wl.identity_matrix(n), 0
    return _inv(n, seed)


# --------------------------------------------------------------------------
# small cases: every route and element size
# --------------------------------------------------------------------------

SMALL = []
for e in (1, 2, 4, 8, 16):
    for n in (1, 2, 3, 5, 8, 11, 12, 14, 17):
        for kind in ("bitrev", "bpc", "general", "complement"):
            SMALL.append((kind, n, e, {}))
    for kind in ("transpose", "identity"):
        SMALL.append((kind, 16, e, {}))
    SMALL.append(("general", 16, e, dict(route=bm.ROUTE_TWO_PASS)))
    SMALL.append(("general", 13, e, dict(route=bm.ROUTE_NAIVE)))
for t in (1, 2, 3, 4, 5, 6, 7):
    SMALL.append(("general", 16, 4, dict(tile_log2=t)))
    SMALL.append(("bpc", 16, 4, dict(tile_log2=t)))
for it in (1, 2, 3):
    SMALL.append(("general", 18, 4, dict(iters_log2=it)))
    SMALL.append(("bitrev", 18, 4, dict(iters_log2=it)))
    SMALL.append(("bpc", 18, 16, dict(iters_log2=it)))
SMALL.append(("general", 15, 4, dict(no_swizzle=1)))
for e in (1, 2, 4, 8, 16):
    for kind in ("general", "bpc", "bitrev"):
        SMALL.append((kind, 17, e, dict(launch=bm.LAUNCH_STREAMED)))
        SMALL.append((kind, 17, e, dict(launch=bm.LAUNCH_STREAMED, grid_log2=2)))
        SMALL.append((kind, 17, e, dict(launch=bm.LAUNCH_STREAMED, grid_log2=3,
                                        walk=bm.WALK_INTERLEAVED)))
        for dp in (1, 2):
            for g in (0, 5, 6):  # g = 5, 6: walks of 2 and 1 tiles (odd/short counts)
                SMALL.append((kind, 16, e, dict(launch=bm.LAUNCH_STREAMED, depth=dp,
                                                grid_log2=g)))
for hint in (1, 2):
    for e in (1, 4, 8, 16):
        SMALL.append(("general", 17, e, dict(cache_hint=hint)))
        SMALL.append(("bitrev", 16, e, dict(cache_hint=hint, launch=bm.LAUNCH_ONE_TILE)))
        SMALL.append(("transpose", 18, e, dict(cache_hint=hint, launch=bm.LAUNCH_STREAMED)))
for bmap in (2, 3, 4, 5, 99):
    SMALL.append(("general", 17, 4, dict(block_map=bmap)))
    SMALL.append(("bpc", 17, 16, dict(block_map=bmap, launch=bm.LAUNCH_ONE_TILE)))
for bmap in (3, 5, 6, 7):
    SMALL.append(("bitrev", 18, 4, dict(block_map=bmap, launch=bm.LAUNCH_PERSISTENT, grid_log2=3)))
    SMALL.append(("general", 18, 8, dict(block_map=bmap, launch=bm.LAUNCH_STREAMED,
                                         walk=bm.WALK_INTERLEAVED, grid_log2=2)))
for e in (1, 4, 16):
    for kind in ("general", "bpc"):
        SMALL.append((kind, 16, e, dict(launch=bm.LAUNCH_ONE_TILE)))
        for g in (1, 3, 6):
            SMALL.append((kind, 17, e, dict(launch=bm.LAUNCH_PERSISTENT, grid_log2=g)))
            SMALL.append((kind, 17, e, dict(launch=bm.LAUNCH_PERSISTENT, grid_log2=g,
                                            walk=bm.WALK_INTERLEAVED)))
SMALL.append(("bitrev", 12, 4, dict(tile_log2=6)))  # n = 2t: a single tile
SMALL.append(("general", 12, 4, dict(tile_log2=6)))


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s-n%d-e%d-%s" % (
    c[0], c[1], c[2], "-".join("%s%s" % kv for kv in sorted(c[3].items()))))
def test_small_parity(case):
    kind, n, e, kw = case
    A, c = _matrix(kind, n, 7000 + 37 * n + e)
    x = wl.fill_random_bytes(n, e, seed=n * 131 + e)
    got, P = _run(A, c, x, **kw)
    want = oracle.apply(A, c, x)
    assert np.array_equal(got, want), P.describe()


def _block_permutation(n, seg_log2, seed):
    """A BMMC that moves whole segments of 2^seg_log2 elements: the identity on
    the low bits, a random invertible matrix on the segment index."""
    Q, _ = _inv(n - seg_log2, seed)
    return np.array([1 << r for r in range(seg_log2)] + [int(q) << seg_log2 for q in Q],
                    dtype=np.uint64)


# Chunk gathers on both sides of the size up to which a workgroup takes its
# source base from scalar loads (2^20 chunks), and below one workgroup.
CHUNK_BOUNDARY = [(16, 7, 5), (16, 9, 6), (16, 20, 6), (16, 21, 6), (4, 22, 8), (4, 23, 8),
                  (1, 24, 10), (1, 25, 10), (8, 20, 7), (2, 23, 9)]


@pytest.mark.parametrize("case", CHUNK_BOUNDARY, ids=lambda c: "e%d-n%d-seg%d" % c)
def test_chunk_gather_size_boundary(case):
    e, n, sl = case
    A = _block_permutation(n, sl, 40 + n)
    c = (5 << sl) & ((1 << n) - 1)
    x = wl.fill_random_bytes(n, e, seed=900 + n)
    _note("chunk gather e=%d n=%d seg=%d" % case)
    got, P = _run(A, c, x)
    assert P.describe()["kernels"] == ["chunk"], P.describe()
    assert np.array_equal(got, oracle.apply(A, c, x)), P.describe()


@pytest.mark.parametrize("n", [22, 23])
def test_two_pass_relabel_size_boundary(n):
    """The two-pass route's segment relabel just inside and just past 2^20
    chunks."""
    A, c = _inv(n, 3)
    x = wl.fill_index_int32(n)
    got, P = _run(A, c, x, route=bm.ROUTE_TWO_PASS)
    assert P.info.passes == 2
    assert np.array_equal(got, oracle.apply(A, c, x)), P.describe()


@pytest.mark.parametrize("seed", range(12))
def test_random_general_sweep(seed):
    """Random sizes and matrices over both general routes."""
    rng = np.random.Generator(np.random.PCG64(99 + seed))
    n = int(rng.integers(4, 21))
    e = int(rng.choice([1, 2, 4, 8, 16]))
    A, c = _inv(n, 8000 + seed)
    x = wl.fill_random_bytes(n, e, seed=seed)
    want = oracle.apply(A, c, x)
    for route in (bm.ROUTE_AUTO, bm.ROUTE_TWO_PASS):
        got, P = _run(A, c, x, route=route)
        assert np.array_equal(got, want), P.describe()


def test_copy_ceiling_kernel():
    torch = _torch()
    # every launch shape (one-shot up to 8 MiB and above 64 MiB, grid-stride
    # in (8, 16] and (32, 64] MiB, one-shot with four vectors per lane in
    # (16, 32] MiB), their edges, and ragged byte tails; each buffer has 64
    # spare bytes that must keep the sentinel
    for nbytes in (0, 1, 15, 16, 4096 + 7, (1 << 20) + 48, 3 << 20, 4 << 20, (4 << 20) + 16,
                   (6 << 20) + 3, 8 << 20, (8 << 20) + 16, 16 << 20, (16 << 20) + 16,
                   (17 << 20) + 5, 32 << 20, (32 << 20) + 16, 64 << 20, (64 << 20) + 16,
                   (200 << 20) + 9):
        src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device="cuda:0")
        dst = torch.full_like(src, SENTINEL)
        bm.copy(src, dst, nbytes)
        torch.cuda.synchronize()
        assert torch.equal(src[:nbytes], dst[:nbytes]), nbytes
        assert int(dst[nbytes:].eq(SENTINEL).all()) == 1, nbytes


def test_two_pass_plan_reused_and_streams():
    """A two-pass plan reuses its scratch across calls and runs on a side stream."""
    torch = _torch()
    n = 18
    A, c = _inv(n, 4242)
    P = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS)
    s = torch.cuda.Stream()
    for k in range(3):
        x = wl.fill_random_bytes(n, 4, seed=k).view(np.uint32).reshape(-1)
        d_in = torch.from_numpy(x.view(np.int32).copy()).to("cuda:0")
        d_out = torch.full_like(d_in, -1)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            P(d_in, d_out, stream=s)
        s.synchronize()
        assert np.array_equal(d_out.cpu().numpy().view(np.uint32), oracle.apply(A, c, x))


def test_failed_scratch_allocation_then_recovery():
    """A two-pass plan whose scratch allocation fails (injected from the host)
    returns ERR_OUT_OF_MEMORY and writes nothing; the next call allocates and
    matches the oracle."""
    torch = _torch()
    n = 18
    A, c = _inv(n, 4343)
    P = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS)
    x = wl.fill_random_bytes(n, 4, seed=43).view(np.uint32).reshape(-1)
    d_in = torch.from_numpy(x.view(np.int32).copy()).to("cuda:0")
    d_out = torch.full_like(d_in, -1)
    try:
        assert bm.bmmc_testing_fail_scratch_allocs(1) == bm.OK
        assert bm.bmmc_execute(P.handle, d_in, d_out) == bm.ERR_OUT_OF_MEMORY
    finally:
        bm.bmmc_testing_fail_scratch_allocs(0)
    torch.cuda.synchronize()
    assert bool((d_out == -1).all())
    assert bm.bmmc_execute(P.handle, d_in, d_out) == bm.OK
    torch.cuda.synchronize()
    assert np.array_equal(d_out.cpu().numpy().view(np.uint32), oracle.apply(A, c, x))


@pytest.mark.parametrize("kw", [dict(), dict(launch=bm.LAUNCH_ONE_TILE),
                                dict(launch=bm.LAUNCH_PERSISTENT), dict(launch=bm.LAUNCH_STREAMED),
                                dict(route=bm.ROUTE_TWO_PASS), dict(route=bm.ROUTE_NAIVE)],
                         ids=["auto", "one_tile", "persistent", "streamed", "two_pass", "naive"])
def test_graph_capture_replays(kw):
    """Executes captured in a HIP graph (as the benchmark times them) give the
    oracle's result on every replay, with eager work and synchronisation
    between the replays: the outputs are refilled eagerly before each one."""
    torch = _torch()
    n, e = 18, 4
    A, c = _inv(n, 6060)
    xs = [wl.fill_random_bytes(n, e, seed=700 + k) for k in range(3)]
    wants = [oracle.apply(A, c, x).view(np.uint8).reshape(-1) for x in xs]
    d_ins = [torch.from_numpy(np.ascontiguousarray(x).view(np.uint8).reshape(-1).copy())
             .to("cuda:0") for x in xs]
    d_outs = [torch.empty_like(d) for d in d_ins]
    P = bm.Plan(n, A, c, e, **kw)
    P(d_ins[0], d_outs[0])  # first call allocates a two-pass plan's scratch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        h = int(torch.cuda.current_stream().cuda_stream)
        for d_in, d_out in zip(d_ins, d_outs):
            assert bm.bmmc_execute(P.handle, d_in, d_out, h) == bm.OK
        assert bm.bmmc_copy(d_ins[0], d_outs[2], 4096, h) == bm.OK  # the copy kernel too
    wants[2] = wants[2].copy()
    wants[2][:4096] = np.ascontiguousarray(xs[0]).view(np.uint8).reshape(-1)[:4096]
    for rep in range(3):
        for d_out in d_outs:
            d_out.fill_(SENTINEL)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (d_out, want) in enumerate(zip(d_outs, wants)):
            assert np.array_equal(d_out.cpu().numpy(), want), (rep, k, P.describe())


def test_execute_rejects_alias_on_device():
    torch = _torch()
    P = bm.Plan(12, wl.bit_reverse_matrix(12), 0, 4)
    buf = torch.zeros(2 << 12, dtype=torch.int32, device="cuda:0")
    assert bm.bmmc_execute(P.handle, buf, buf[100:], None) == bm.ERR_ALIAS


TUNE_CASES = [("general", 17, 4, {}), ("bpc", 18, 16, {}), ("bitrev", 16, 1, {}),
              ("transpose", 18, 8, {}), ("general", 15, 2, dict(route=bm.ROUTE_TWO_PASS)),
              ("general", 17, 4, dict(launch=bm.LAUNCH_ONE_TILE)),
              ("bpc", 17, 4, dict(block_map=7)), ("general", 12, 4, dict(iters_log2=1)),
              ("complement", 14, 4, {}), ("identity", 14, 4, {}),
              ("transpose", 16, 4, dict(tile_log2=5)), ("bitrev", 18, 2, {})]


@pytest.mark.parametrize("case", TUNE_CASES, ids=lambda c: "%s-n%d-e%d-%s" % (
    c[0], c[1], c[2], "-".join("%s%s" % kv for kv in sorted(c[3].items()))))
def test_tune_keeps_results_and_fixed_options(case):
    torch = _torch()
    kind, n, e, kw = case
    A, c = _matrix(kind, n, 9100 + n + e)
    x = wl.fill_random_bytes(n, e, seed=17 * n + e)
    want = oracle.apply(A, c, x)
    P = bm.Plan(n, A, c, e, **kw)
    before = [(d.kernel, d.launch, d.block_map) for d in P.passes()]
    raw = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
    d_in = torch.from_numpy(raw.copy()).to("cuda:0")
    d_out = torch.full_like(d_in, SENTINEL)
    P.tune(d_in, d_out, reps=1)
    torch.cuda.synchronize()
    assert np.array_equal(d_out.cpu().numpy().view(x.dtype).reshape(x.shape), want)
    for rep in range(2):
        d_out.fill_(SENTINEL)
        P(d_in, d_out)
        torch.cuda.synchronize()
        got = d_out.cpu().numpy().view(x.dtype).reshape(x.shape)
        assert np.array_equal(got, want), (rep, P.describe())
    after = P.passes()
    assert [d.kernel for d in after] == [b[0] for b in before]
    if "tile_log2" in kw:
        assert P.info.tile_log2 == kw["tile_log2"]
    for d in after:
        if d.kernel == bm.KERNEL_TILED:
            if "launch" in kw:
                assert d.launch == kw["launch"]
            if "block_map" in kw:
                assert d.block_map == kw["block_map"]
            else:
                assert d.block_map in (1, 3, 5, 6, 8, 9)
        else:
            assert (d.kernel, d.launch, d.block_map) in before


@pytest.mark.parametrize("kind,n,e", [("general", 20, 4), ("bpc", 20, 16), ("bitrev", 22, 4)])
def test_tuned_options_rebuild_the_tuned_plan(kind, n, e):
    """After tuning, the plan's options rebuild the tuned tables exactly (no
    timing), and the rebuilt plan gives the oracle's result."""
    import ctypes
    torch = _torch()
    A, c = _matrix(kind, n, 8100 + n)
    x = wl.fill_random_bytes(n, e, seed=n + e)
    raw = np.ascontiguousarray(x).view(np.uint8).reshape(-1)
    d_in = torch.from_numpy(raw.copy()).to("cuda:0")
    d_out = torch.full_like(d_in, SENTINEL)
    P = bm.Plan(n, A, c, e)
    P.tune(d_in, d_out, reps=2)
    Q = bm.Plan(n, A, c, e, **P.options())
    for dp, dq in zip(P.passes(), Q.passes()):
        assert (ctypes.string_at(ctypes.addressof(dp), ctypes.sizeof(dp)) ==
                ctypes.string_at(ctypes.addressof(dq), ctypes.sizeof(dq)))
    d_out.fill_(SENTINEL)
    Q(d_in, d_out)
    torch.cuda.synchronize()
    assert np.array_equal(d_out.cpu().numpy().view(x.dtype).reshape(x.shape),
                          oracle.apply(A, c, x)), Q.describe()


@pytest.mark.parametrize("route", [bm.ROUTE_AUTO, bm.ROUTE_TWO_PASS])
def test_tune_over_rotating_pairs(route):
    """bmmc_plan_tune_pairs: outs[0] holds the permutation of ins[0]; every
    other output holds its own input's permutation or is untouched."""
    torch = _torch()
    n, e = 16, 4
    A, c = _inv(n, 5150)
    xs = [wl.fill_random_bytes(n, e, seed=300 + k) for k in range(5)]
    d_ins = [torch.from_numpy(np.ascontiguousarray(x).view(np.uint8).reshape(-1).copy())
             .to("cuda:0") for x in xs]
    d_outs = [torch.full_like(d, SENTINEL) for d in d_ins]
    P = bm.Plan(n, A, c, e, route=route)
    P.tune(pairs=list(zip(d_ins, d_outs)), reps=2)
    torch.cuda.synchronize()
    for k, (x, d) in enumerate(zip(xs, d_outs)):
        got = d.cpu().numpy()
        want = oracle.apply(A, c, x).view(np.uint8).reshape(-1)
        untouched = bool(np.all(got == SENTINEL))
        assert np.array_equal(got, want) or (k > 0 and untouched), k
    for x, d_in, d_out in zip(xs, d_ins, d_outs):
        d_out.fill_(SENTINEL)
        P(d_in, d_out)
        torch.cuda.synchronize()
        assert np.array_equal(d_out.cpu().numpy(), oracle.apply(A, c, x).view(np.uint8).reshape(-1))


# --------------------------------------------------------------------------
# the five workloads at full size
# --------------------------------------------------------------------------

def _device_run(name, A, c, x, tune=False, **plan_kw):
    """Run a workload's plan; with tune=True the plan is first tuned on the
    same buffers (as the benchmark does), then run again into a fresh
    sentinel-filled output."""
    torch = _torch()
    n = wl.WORKLOADS[name].n
    raw = x.reshape(-1).view(np.uint8)
    P = bm.Plan(n, A, c, raw.size >> n, **plan_kw)
    d_in = torch.from_numpy(raw).to("cuda:0")
    d_out = torch.full_like(d_in, SENTINEL)
    if tune:
        P.tune(d_in, d_out)
        torch.cuda.synchronize()
        _note("%s tuned: %s" % (name, P.describe()))
        d_out.fill_(SENTINEL)
    P(d_in, d_out)
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(x.dtype).reshape(x.shape)
    del d_in, d_out
    torch.cuda.empty_cache()
    return got, P


def _lib_accepts(n):
    def accept(rows):
        h = bm.bmmc_plan_create(n, rows, 0, 4)
        if h:
            bm.bmmc_plan_destroy(h)
        return bool(h)
    return accept


def _sample_idx(n, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = rng.integers(0, 1 << n, size=count, dtype=np.uint64)
    # the ends of the array and the segment edges are always included
    edges = np.array([0, 1, (1 << n) - 1, (1 << n) - 2, 63, 64, 4095, 4096], dtype=np.uint64)
    return np.concatenate([edges[edges < (1 << n)], idx])


@pytest.mark.parametrize("name", ["c1a", "c1b", "c2"])
def test_workload_full_check(name):
    n = wl.WORKLOADS[name].n
    A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == n)
    # the oracle's choice of the random matrix is the library's choice too
    if name == "c1a":
        assert np.array_equal(A, wl.workload_matrix(name, accept=_lib_accepts(n))[0])
    x = wl.workload_data(name)
    want = oracle.apply(A, c, x, threads=HOST_THREADS)
    routes = [{}, dict(tune=True), dict(buffer_loads=1)] + (
        [dict(route=bm.ROUTE_TWO_PASS), dict(route=bm.ROUTE_TWO_PASS, buffer_loads=1)]
        if name == "c1a" else [])
    for kw in routes:
        _note("%s %s" % (name, kw))
        got, P = _device_run(name, A, c, x, **kw)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), P.describe()
    if name == "c2":
        # the transpose of the 4096 x 4096 fp32 matrix, as two loops would give it
        assert np.array_equal(got.view(np.uint32),
                              x.reshape(4096, 4096).T.reshape(-1).view(np.uint32))


def test_workload_c3_bitrev28_full():
    name = "c3"
    A, c = wl.workload_matrix(name)
    x = wl.workload_data(name)
    _note("c3: oracle")
    want = oracle.apply(A, c, x, threads=HOST_THREADS)
    for tune in (False, True):
        _note("c3: gpu tune=%s" % tune)
        got, P = _device_run(name, A, c, x, tune=tune)
        assert P.info.passes == 1 and P.info.kind == bm.KIND_BPC
        assert np.array_equal(got, want), P.describe()
        del got
    # staged in LDS half at a time, with the shapes the tuning tries
    for kw in (dict(tile_log2=7), dict(tile_log2=7, tile_skew=1, tile_threads_log2=9),
               dict(tile_log2=7, tile_skew=2)):
        _note("c3: gpu split %s" % kw)
        got, P = _device_run(name, A, c, x, split_stage=1, **kw)
        assert P.describe()["split_stage"] == 1
        assert np.array_equal(got, want), P.describe()
        del got
    # the input read with buffer loads
    for kw in (dict(), dict(tile_log2=7, tile_skew=1, tile_threads_log2=9),
               dict(tile_log2=6, tile_skew=-1, block_map=8)):
        _note("c3: gpu buffer loads %s" % kw)
        got, P = _device_run(name, A, c, x, buffer_loads=1, **kw)
        assert P.describe()["buffer_loads"] == 1
        assert np.array_equal(got, want), P.describe()
        del got


def test_workload_c4_general30():
    name = "c4"
    n = 30
    A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == n)
    x = wl.workload_data(name)
    _note("c4: oracle")
    want = oracle.apply(A, c, x, threads=HOST_THREADS)
    for kw in ({}, dict(tune=True), dict(route=bm.ROUTE_TWO_PASS),
               dict(route=bm.ROUTE_TWO_PASS, tile_log2=7, tile_skew=1, tile_threads_log2=9),
               dict(route=bm.ROUTE_TWO_PASS, tile_log2=6, tile_skew=-2)):
        _note("c4 %s" % kw)
        got, P = _device_run(name, A, c, x, **kw)
        assert P.info.kind == bm.KIND_GENERAL
        bad, first = oracle.check_sampled(A, c, x, got, _sample_idx(n, 1 << 20, 30))
        assert bad == 0, (first, P.describe())
        assert np.array_equal(got, want), P.describe()
        del got


def test_workload_c4_every_tuning_candidate():
    """Every plan bmmc_plan_tune would time (bmmc_plan_tune_candidates: tile
    sides, shapes, thread counts, launches and orders) at the full n = 30
    size, on sampled indices."""
    torch = _torch()
    name = "c4"
    n = 30
    A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == n)
    x = wl.workload_data(name)
    d_in = torch.from_numpy(x.reshape(-1).view(np.uint8)).to("cuda:0")
    d_out = torch.empty_like(d_in)
    idx = _sample_idx(n, 1 << 18, 31)
    # the oracle maps the sampled input indices once; each candidate's output
    # elements at those positions are gathered on the device (a 4 GiB copy to
    # the host per candidate would take most of the test's time)
    pos = torch.from_numpy(oracle.map_indices(A, c, idx).astype(np.int64)).to("cuda:0")
    want = x.reshape(-1)[idx.astype(np.int64)]
    cands = bm.Plan(n, A, c, 4).tune_candidates()
    assert len(cands) >= 40
    for k, opts in enumerate(cands):
        _note("c4 candidate %d %s" % (k, opts))
        P = bm.Plan(n, A, c, 4, **opts)
        d_out.fill_(SENTINEL)
        P(d_in, d_out)
        got = d_out.view(torch.int32).index_select(0, pos).cpu().numpy().view(x.dtype)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (k, opts, int(idx[bad[0]]), P.describe())


def test_workload_c4_every_two_pass_candidate():
    """Every plan the tuning of the pages' two-pass route would time (square
    and rectangular tiles, thread counts, launches and orders) at the full
    n = 30 size, on sampled indices gathered on the device."""
    torch = _torch()
    name = "c4"
    n = 30
    A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == n)
    x = wl.workload_data(name)
    d_in = torch.from_numpy(x.reshape(-1).view(np.uint8)).to("cuda:0")
    d_out = torch.empty_like(d_in)
    idx = _sample_idx(n, 1 << 18, 32)
    pos = torch.from_numpy(oracle.map_indices(A, c, idx).astype(np.int64)).to("cuda:0")
    want = x.reshape(-1)[idx.astype(np.int64)]
    cands = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS).tune_candidates()
    assert {o["tile_skew"] for o in cands} >= {0, 1, -1}
    for k, opts in enumerate(cands):
        _note("c4 two-pass candidate %d %s" % (k, opts))
        P = bm.Plan(n, A, c, 4, **opts)
        assert P.info.passes == 2
        d_out.fill_(SENTINEL)
        P(d_in, d_out)
        got = d_out.view(torch.int32).index_select(0, pos).cpu().numpy().view(x.dtype)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (k, opts, int(idx[bad[0]]), P.describe())


def test_workload_c1a_every_two_pass_candidate():
    """Every two-pass tuning candidate of c1a (n = 20), over the whole array."""
    torch = _torch()
    name = "c1a"
    n = 20
    A, c = wl.workload_matrix(name, accept=lambda r: oracle.rank(r) == n)
    x = wl.workload_data(name)
    want = oracle.apply(A, c, x, threads=HOST_THREADS)
    d_in = torch.from_numpy(x.reshape(-1).view(np.uint8)).to("cuda:0")
    d_out = torch.empty_like(d_in)
    cands = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS).tune_candidates()
    assert any(o["buffer_loads"] for o in cands) and any(o["tile_skew"] for o in cands)
    for k, opts in enumerate(cands):
        _note("c1a two-pass candidate %d %s" % (k, opts))
        P = bm.Plan(n, A, c, 4, **opts)
        d_out.fill_(SENTINEL)
        P(d_in, d_out)
        got = d_out.cpu().numpy().view(x.dtype).reshape(x.shape)
        assert np.array_equal(got, want), (k, opts, P.describe())


def test_workload_c5_buffer_loads():
    """c5's slowest permutation (10) with the input read by buffer loads:
    the whole 2 GiB array (the largest the form allows) against the oracle
    for two shapes, and every buffer-load plan the tuning would time on
    sampled indices."""
    torch = _torch()
    name = "c5"
    n = 27
    x = wl.workload_data(name)
    A, c = wl.workload_matrix(name, perm_index=10)
    d_in = torch.from_numpy(x.reshape(-1).view(np.uint8)).to("cuda:0")
    d_out = torch.empty_like(d_in)
    want = oracle.apply(A, c, x, threads=HOST_THREADS).view(np.uint32).reshape(-1)
    for kw in (dict(tile_log2=5, tile_skew=2, tile_threads_log2=9), dict()):
        _note("c5 perm 10 buffer loads %s" % kw)
        P = bm.Plan(n, A, c, 16, buffer_loads=1, **kw)
        d_out.fill_(SENTINEL)
        P(d_in, d_out)
        torch.cuda.synchronize()
        assert np.array_equal(d_out.cpu().numpy().view(np.uint32), want), P.describe()
    del want
    idx = _sample_idx(n, 1 << 18, 32)
    pos = torch.from_numpy(oracle.map_indices(A, c, idx).astype(np.int64)).to("cuda:0")
    exp = torch.from_numpy(x.reshape(1 << n, 4)[idx.astype(np.int64)].view(np.int32)).to("cuda:0")
    cands = [o for o in bm.Plan(n, A, c, 16).tune_candidates() if o["buffer_loads"]]
    assert len(cands) >= 20
    for k, opts in enumerate(cands):
        _note("c5 perm 10 buffer-load candidate %d %s" % (k, opts))
        P = bm.Plan(n, A, c, 16, **opts)
        d_out.fill_(SENTINEL)
        P(d_in, d_out)
        got = d_out.view(torch.int32).view(1 << n, 4).index_select(0, pos)
        assert bool((got == exp).all()), (k, opts, P.describe())
    del d_in, d_out


_C5_DATA = {}


@pytest.mark.parametrize("k", range(32))
def test_workload_c5_random_bpc_records(k):
    """Each of the 32 seeded permutations, tuned as the benchmark tunes it,
    against the oracle over the whole 2 GiB array."""
    torch = _torch()
    name = "c5"
    n = 27
    if "x" not in _C5_DATA:
        _C5_DATA["x"] = wl.workload_data(name)
    x = _C5_DATA["x"]
    d_in = torch.from_numpy(x.reshape(-1).view(np.uint8)).to("cuda:0")
    d_out = torch.empty_like(d_in)
    A, c = wl.workload_matrix(name, perm_index=k)
    _note("c5 perm %d" % k)
    P = bm.Plan(n, A, c, 16)
    assert P.info.passes == 1 and P.info.kind == bm.KIND_BPC
    P.tune(d_in, d_out)  # the benchmark tunes each permutation's plan
    d_out.fill_(SENTINEL)
    P(d_in, d_out)
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(np.uint32)
    del d_in, d_out
    want = oracle.apply(A, c, x, threads=HOST_THREADS).view(np.uint32).reshape(-1)
    assert np.array_equal(got, want), (k, P.describe())
    if k == 31:
        _C5_DATA.clear()


# --------------------------------------------------------------------------
# the largest arrays the ABI accepts, checked on sampled indices on the device
# --------------------------------------------------------------------------

GPU_MAX_CASES = [  # (n, elem_bytes, kind, plan options, tune)
    (32, 1, "general", {}, False),                        # 4 GiB per array
    (32, 1, "general", dict(route=bm.ROUTE_TWO_PASS), False),
    (32, 2, "transpose", {}, False),                      # 8 GiB
    (31, 8, "bpc", {}, True),                             # 16 GiB
    (32, 16, "bitrev", {}, False),                        # 64 GiB = 2^36 bytes
    (32, 16, "general", {}, True),
    # 2^28 workgroups of 16 threads: more work-items than one launch may
    # hold, so the pass is split into several launches
    (32, 16, "general", dict(tile_log2=2, launch=bm.LAUNCH_ONE_TILE), False),
    # the naive pass: 2^24 one-byte groups of 256 lanes, also split in two launches
    (32, 1, "general", dict(route=bm.ROUTE_NAIVE), False),
    (32, 4, "reverse", {}, False),                        # complement only: chunk kernel
    # tiles staged in LDS half at a time
    (32, 4, "bitrev", dict(split_stage=1, tile_log2=7), False),          # 16 GiB
    (31, 8, "bpc", dict(split_stage=1, tile_threads_log2=9), False),     # 16 GiB
    (32, 16, "general", dict(split_stage=1, tile_skew=1), False),        # 64 GiB
    # the input read with buffer loads, at the 2^31 bytes they allow
    (29, 4, "general", dict(buffer_loads=1), False),
    (28, 8, "bitrev", dict(buffer_loads=1, tile_skew=1), False),
    (27, 16, "bpc", dict(buffer_loads=1, tile_log2=5, tile_skew=2, tile_threads_log2=9),
     False),
    (29, 4, "general", {}, True),   # tuned: the buffer-load candidates included
]


def _max_matrix(kind, n, seed):
    if kind == "reverse":
        return wl.identity_matrix(n), (1 << n) - 1
    if kind == "bitrev":
        return wl.bit_reverse_matrix(n), 0
    if kind == "transpose":
        return wl.transpose_matrix(n // 2, n - n // 2), 0
    if kind == "bpc":
        return wl.random_bpc(n, seed)
    return _inv(n, seed)


@pytest.mark.parametrize("case", GPU_MAX_CASES, ids=lambda c: "n%d-e%d-%s-%s%s" % (
    c[0], c[1], c[2], "-".join("%s%s" % kv for kv in sorted(c[3].items())),
    "-tuned" if c[4] else ""))
def test_maximum_sizes_sampled(case):
    """Arrays of up to 2^36 bytes (the ABI's limit): random bytes filled on the
    device, one execute (after tuning for the tuned cases, whose tuning also
    writes the output), then 2^20 sampled source indices plus the ends of the
    array, mapped by the oracle on the host, compared element by element on
    the device (out[map(i)] == in[i])."""
    torch = _torch()
    n, e, kind, kw, tune = case
    nbytes = e << n
    scratch = nbytes if kw.get("route") == bm.ROUTE_TWO_PASS else 0
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 2 * nbytes + scratch + (4 << 30):
        pytest.skip("needs %d GiB of free device memory, %d GiB free"
                    % ((2 * nbytes + scratch) >> 30, free >> 30))
    A, c = _max_matrix(kind, n, 4100 + n + e)
    _note("max n=%d e=%d %s %s: allocate and fill %d GiB" % (n, e, kind, kw, nbytes >> 30))
    d_in = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(n * 131 + e)
    step = 1 << 30
    for off in range(0, nbytes, step):
        d_in[off:off + step].random_(0, 256, generator=gen)
    d_out = torch.full_like(d_in, SENTINEL)
    P = bm.Plan(n, A, c, e, **kw)
    _note("max: plan %s" % P.describe())
    if tune:
        P.tune(d_in, d_out, reps=1)
        torch.cuda.synchronize()
        _note("max: tuned %s" % P.describe())
        d_out.fill_(SENTINEL)
    P(d_in, d_out)
    torch.cuda.synchronize()
    _note("max: check")
    N = 1 << n
    rng = np.random.Generator(np.random.PCG64(n + e))
    idx = np.concatenate([np.array([0, 1, N - 2, N - 1, N // 2], dtype=np.uint64),
                          rng.integers(0, N, size=1 << 20, dtype=np.uint64)])
    dst = oracle.map_indices(A, c, idx)
    src_t = torch.from_numpy(idx.astype(np.int64)).to("cuda:0")
    dst_t = torch.from_numpy(dst.astype(np.int64)).to("cuda:0")
    vin, vout = d_in.view(N, e), d_out.view(N, e)
    same = (vin.index_select(0, src_t) == vout.index_select(0, dst_t)).all(dim=1)
    bad = int((~same).sum())
    assert bad == 0, (bad, P.describe())
    # the copy ceiling at the same size
    d_out.fill_(SENTINEL)
    assert bm.bmmc_copy(d_in, d_out, nbytes, None) == bm.OK
    torch.cuda.synchronize()
    assert bool((vin.index_select(0, src_t) == vout.index_select(0, src_t)).all())
    del d_in, d_out, vin, vout
    torch.cuda.empty_cache()
