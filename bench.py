"""Benchmark: effective bandwidth of a BMMC permutation on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

A step is one bmmc_execute of the planned permutation over the whole array
(input resident in HBM).  Effective bandwidth = (bytes read + bytes written)
/ time, with each element read once and written once ("A kernel that is
correct": effective bandwidth; 2 x 4096^2 x 4 bytes for the transpose), GB =
1e9.  The copy ceiling (bmmc_copy of the same bytes, same buffers, same
protocol) is timed in the same run.

Residency: by default the K steps rotate over enough input/output buffer
pairs that the working set is at least 1 GiB, four times the 256 MB Infinity
Cache, so every step streams from and to HBM; --warm reuses one pair (the
pages' protocol of repeating one launch), which lets small arrays sit in the
cache.

Prints ONE JSON line.  The CPU baseline is the oracle (oracle/), timed on a
bounded sample on the host cores, for context only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bmmc_affine_index_amd as bm  # noqa: E402
from bmmc_affine_index_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 1000 * 1000
WORKLOAD_NAMES = {
    "c1a": "bmmc_random_n20_int32",
    "c1b": "bitreverse_n20_int32",
    "c2": "transpose4096x4096_fp32_n24",
    "c3": "bitreverse_n28_int32",
    "c4": "bmmc_random_n30_int32",
    "c5": "random_bpc_n27_16B_records",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_%s.txt")


def kernel_source_digest() -> str:
    """Digest of the device code: the kernels and what they include."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bmmc_affine_index_amd", "csrc")
    for rel in sorted(["launch.h", "kernels/tiled.hip", "kernels/tiled_cfg.h", "kernels/chunk.hip",
                       "kernels/copy.hip", "kernels/common.h"]):
        with open(os.path.join(csrc, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def plan_tables_digest(plan) -> str:
    """Digest of the kernel tables of every pass of a plan: with the device
    code, they decide every address the kernels touch."""
    h = hashlib.sha256()
    for d in plan.passes():
        h.update(bytes(d))
    return h.hexdigest()[:16]


def read_traffic(workload: str, plan_options: dict, tables_digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when there is none, or it holds no entry taken with this device code,
    this plan (launch style, tile side, tile order ...) and these kernel
    tables.  A summary holds one entry per plan counted, each opened by a line
    "[entry]" and made of key=value lines; '#' lines are comments."""
    path = TRAFFIC_FILE % workload
    if not os.path.exists(path):
        return None
    entries, kv = [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line == "[entry]":
                kv = {}
                entries.append(kv)
            elif kv is not None and "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    digest = kernel_source_digest()
    for kv in entries:
        if kv.get("kernel_source_digest") != digest or kv.get("plan_tables_digest") != tables_digest:
            continue
        try:
            if json.loads(kv.get("plan_options", "null")) != plan_options:
                continue
            return float(kv["hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            continue
    return None


def lib_accepts(n: int):
    def accept(rows):
        h = bm.bmmc_plan_create(n, rows, 0, 4)
        if h:
            bm.bmmc_plan_destroy(h)
        return bool(h)
    return accept


def time_replays(torch, fn, bufs, steps, warmup, stream, replays=5, graph=True):
    """Warm up, then time `replays` regions of exactly `steps` calls
    fn(in, out, stream_handle) each, with events on `stream` and a
    synchronisation on both sides of every region; returns the milliseconds
    per step of each region.  graph=True captures the `steps` calls once into
    a HIP graph and each region replays it, so the host's per-call cost
    (ctypes, argument checks, the launch itself) stays out of the measurement
    of arrays whose steps take microseconds."""
    h = int(stream.cuda_stream)
    for k in range(warmup):
        fn(*bufs[k % len(bufs)], h)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    if graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            hc = int(torch.cuda.current_stream().cuda_stream)
            for k in range(steps):
                fn(*bufs[k % len(bufs)], hc)
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        for _ in range(replays):
            start.record(stream)
            g.replay()
            stop.record(stream)
            torch.cuda.synchronize()
            out.append(start.elapsed_time(stop) / steps)
        del g
    else:
        for _ in range(replays):
            start.record(stream)
            for k in range(steps):
                fn(*bufs[k % len(bufs)], h)
            stop.record(stream)
            torch.cuda.synchronize()
            out.append(start.elapsed_time(stop) / steps)
    return out


def replay_stats(ms_list, algo_bytes):
    """Median, min and max over timed regions, as ms per step and GB/s."""
    v = sorted(ms_list)
    med = v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    gbs = lambda ms: algo_bytes / (ms * 1e-3) / 1e9  # noqa: E731
    return {"ms_per_step": med, "ms_min": v[0], "ms_max": v[-1],
            "ms_mean": sum(v) / len(v), "gbs": gbs(med), "gbs_min": gbs(v[-1]),
            "gbs_max": gbs(v[0]), "replays": len(v)}


def per_launch_ms(torch, fn, bufs, reps, stream):
    """Median/min/max of individually event-timed launches."""
    h = int(stream.cuda_stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for k, (a, b) in enumerate(ev):
        a.record(stream)
        fn(*bufs[k % len(bufs)], h)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms[len(ms) // 2], ms[0], ms[-1]


def oracle_threads() -> int:
    """Host threads for the oracle: the cores this process may run on (its
    CPU affinity), or OMP_NUM_THREADS where the host sets the process's CPU
    share that way."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def sampled_parity(torch, A, c, x, out, samples=1 << 20, seed=1):
    """Check out[A.i XOR c] = x[i] on `samples` seeded input indices plus the
    first and last: the oracle maps each sampled index, the device gathers
    those output elements, and the host compares them with the input's.
    Returns (mismatches, checked)."""
    import oracle
    n = len(A)
    N = 1 << n
    elem = x.nbytes >> n
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = np.concatenate([np.array([0, N - 1], dtype=np.uint64),
                          rng.integers(0, N, size=samples, dtype=np.uint64)])
    pos = oracle.map_indices(A, c, idx)
    rows = out.view(torch.uint8).reshape(N, elem)
    got = rows.index_select(0, torch.from_numpy(pos.astype(np.int64)).to(out.device)).cpu().numpy()
    want = np.ascontiguousarray(x).reshape(-1).view(np.uint8).reshape(N, elem)[idx.astype(np.int64)]
    bad = int(np.count_nonzero(np.any(got != want, axis=1)))
    return bad, int(idx.size)


def full_parity(A, c, x, got_host):
    """The whole output against the oracle's; True when every byte agrees."""
    import oracle
    want = oracle.apply(A, c, x, threads=oracle_threads())
    return np.array_equal(np.ascontiguousarray(got_host).view(np.uint8).reshape(-1),
                          want.view(np.uint8).reshape(-1))


def cpu_baseline(A, c, x, budget_s: float):
    """The oracle, as it stands, on the host cores: repeated full-array
    scatters (or index ranges for big arrays) for about budget_s seconds."""
    import oracle
    threads = oracle_threads()
    n = len(A)
    N = 1 << n
    elem = x.nbytes >> n
    out = np.empty_like(x)
    # one slice of at most 2^24 indices per call keeps each call short
    span = min(N, 1 << 24)
    done = 0
    t0 = time.perf_counter()
    while True:
        lo = (done * span) % N
        oracle.apply_range(A, c, x, out, lo, lo + span, threads=threads)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 100000:
            break
    moved = 2.0 * done * span * elem
    # the same calls on one thread, for about a fifth of the budget
    one, t1 = 0, time.perf_counter()
    while True:
        lo = (one * span) % N
        oracle.apply_range(A, c, x, out, lo, lo + span, threads=1)
        one += 1
        el1 = time.perf_counter() - t1
        if el1 >= budget_s / 5 or one >= 100000:
            break
    return {"value": round(moved / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d oracle calls of 2^%d consecutive input indices each (%.1f s, "
                      "%d threads), same matrix and data" % (done, span.bit_length() - 1, el,
                                                             threads),
            "single_thread_value": round(2.0 * one * span * elem / el1 / 1e9, 4),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


ABLATION_VARIANTS = [
    # name, plan options; the paper's Figure 9 columns, then this library's default
    ("naive", dict(route=bm.ROUTE_NAIVE)),
    # (the paper's kernels take the tiles in their natural order: block_map 1)
    ("tile", dict(launch=bm.LAUNCH_ONE_TILE, no_swizzle=True, block_map=1)),
    ("tile+banks", dict(launch=bm.LAUNCH_ONE_TILE, block_map=1)),
    ("tile+banks+iters", dict(launch=bm.LAUNCH_ONE_TILE, iters_log2=2, block_map=1)),
    ("planner, untuned", dict()),
    ("tuned (default)", dict(tune=True)),
]


def run_ablation(args, torch):
    """The paper's Figure 9 (speedup of each optimisation over the naive kernel
    for random BPC, bit-reversal and random BMMC) and Figure 11 (the same
    against the array size), on 32-bit elements.  Random BMMCs are run both
    as the pages' two tiled passes and as the fused single pass."""
    import oracle
    stream = torch.cuda.current_stream()
    s_handle = int(stream.cuda_stream)
    # about 0.1 s of copies first, so that the first size is not timed while
    # the GPU's clocks are still rising
    wbuf = torch.empty(2 << 28, dtype=torch.uint8, device="cuda:0")
    for _ in range(60):
        if bm.bmmc_copy(wbuf[: 1 << 28], wbuf[1 << 28:], 1 << 28, s_handle) != bm.OK:
            raise bm.BmmcError(bm.ERR_HIP, "bmmc_copy")
    torch.cuda.synchronize()
    del wbuf
    for n in [int(v) for v in args.sizes.split(",")]:
        elem = 4
        nbytes = elem << n
        x = wl.fill_random_bytes(n, elem, 1000 + n)
        raw = torch.from_numpy(x.reshape(-1)).to("cuda:0")
        pairs = max(1, -(-(1 << 30) // (2 * nbytes)))
        ins = [raw] + [raw.clone() for _ in range(pairs - 1)]
        outs = [torch.empty_like(raw) for _ in range(pairs)]
        bufs = list(zip(ins, outs))
        steps = max(10, min(args.steps, int(2e9 // (2 * nbytes)) or 10))

        def copy(i, o, h):
            st = bm.bmmc_copy(i, o, nbytes, h)
            if st != bm.OK:
                raise bm.BmmcError(st, "bmmc_copy")
        # the ceiling: the faster of two timings
        ms_copy = replay_stats(time_replays(torch, copy, bufs, steps, 3, stream, 3,
                                            graph=not args.no_graph), 2.0 * nbytes)["ms_per_step"]
        copy_gbs = 2.0 * nbytes / (ms_copy * 1e-3) / 1e9
        kinds = [("random_bpc", wl.random_bpc(n, 7)), ("bit_reverse", (wl.bit_reverse_matrix(n), 0)),
                 ("random_bmmc", wl.random_bmmc(n, 7, lib_accepts(n)))]
        for kind, (A, c) in kinds:
            variants = list(ABLATION_VARIANTS)
            if kind == "random_bmmc":
                variants = [variants[0]] + [
                    (nm + " two-pass", dict(kw, route=bm.ROUTE_TWO_PASS)) for nm, kw in variants[1:4]
                ] + [("persistent two-pass", dict(route=bm.ROUTE_TWO_PASS))] + variants[4:]
            base = None
            for vname, kw in variants:
                kw = dict(kw)
                tune = kw.pop("tune", False)
                plan = bm.Plan(n, A, c, elem, **kw)
                if tune:
                    plan.tune(pairs=bufs, stream=s_handle)

                def step(i, o, h, plan=plan):
                    st = bm.bmmc_execute(plan.handle, i, o, h)
                    if st != bm.OK:
                        raise bm.BmmcError(st, "bmmc_execute")
                # median of three timed regions: one region alone can catch a
                # hiccup of the box (a 16 MiB cell once timed 2.4x its median)
                ms = replay_stats(time_replays(torch, step, bufs, steps, 3, stream, 3,
                                               graph=not args.no_graph), 2.0 * nbytes)["ms_per_step"]
                gbs = 2.0 * nbytes / (ms * 1e-3) / 1e9
                base = base or gbs
                step(*bufs[0], s_handle)
                torch.cuda.synchronize()
                got = outs[0].cpu().numpy().reshape(x.shape)
                if n <= 24:
                    ok = np.array_equal(got, oracle.apply(A, c, x, threads=16))
                else:
                    idx = np.random.Generator(np.random.PCG64(n)).integers(
                        0, 1 << n, size=1 << 18, dtype=np.uint64)
                    ok = oracle.check_sampled(A, c, x, got, idx)[0] == 0
                print(json.dumps({"ablation": True, "kind": kind, "n": n, "elem_bytes": elem,
                                  "variant": vname, "gbs": round(gbs, 1),
                                  "frac_of_copy": round(gbs / copy_gbs, 4),
                                  "speedup_vs_naive": round(gbs / base, 3),
                                  "ms": round(ms, 5), "copy_gbs": round(copy_gbs, 1),
                                  "passes": plan.info.passes, "plan": plan.describe(),
                                  "parity": "bit-exact" if ok else "MISMATCH"}), flush=True)
                if not ok:
                    sys.exit(3)
        del ins, outs, bufs, raw
        torch.cuda.empty_cache()


# The configurations measured beside the headline, in the order they run:
# (key, workload, route).  c4's two-pass route reuses the headline's buffers.
CONFIG_CASES = [
    ("c4_two_pass", "c4", bm.ROUTE_TWO_PASS),
    ("c1a_fused", "c1a", bm.ROUTE_AUTO),
    ("c1a_two_pass", "c1a", bm.ROUTE_TWO_PASS),
    ("c1b", "c1b", bm.ROUTE_AUTO),
    ("c2", "c2", bm.ROUTE_AUTO),
    ("c3", "c3", bm.ROUTE_AUTO),
    ("c5", "c5", bm.ROUTE_AUTO),
]
C5_PERMS = 32


def log(msg):
    print("bench.py: " + msg, file=sys.stderr, flush=True)


class Runner:
    """Buffers, timing and parity checks shared by the headline and the
    configurations; the copy ceiling is timed once per array size."""

    def __init__(self, torch, args):
        self.torch, self.args = torch, args
        self.stream = torch.cuda.current_stream()
        self.h = int(self.stream.cuda_stream)
        self.graph = not args.no_graph
        self.copies = {}

    def buffers(self, x, nbytes):
        """Rotating (input, output) pairs with at least 1 GiB of working set
        (four times the 256 MB Infinity Cache), or one pair with --warm."""
        torch = self.torch
        pairs = 1 if self.args.warm else max(1, -(-(1 << 30) // (2 * nbytes)))
        raw = torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.uint8)).to("cuda:0")
        ins = [raw] + [raw.clone() for _ in range(pairs - 1)]
        outs = [torch.empty_like(raw) for _ in range(pairs)]
        return list(zip(ins, outs))

    def steps_for(self, nbytes, headline):
        """The headline times exactly --steps steps per region; the other
        configurations take more steps on small arrays, so that a region
        lasts about 2 ms (1000 steps at most)."""
        if headline:
            return self.args.steps
        return max(self.args.steps, min(1000, int(2e-3 * 5e12 / (2.0 * nbytes))))

    def time_plan(self, plan, bufs, nbytes, steps):
        def step(i, o, h):
            st = bm.bmmc_execute(plan.handle, i, o, h)
            if st != bm.OK:
                raise bm.BmmcError(st, "bmmc_execute")
        ms = time_replays(self.torch, step, bufs, steps, self.args.warmup, self.stream,
                          self.args.replays, graph=self.graph)
        return replay_stats(ms, 2.0 * nbytes)

    def copy_ceiling(self, bufs, nbytes, steps):
        key = (nbytes, steps)
        if key not in self.copies:
            def copy(i, o, h):
                st = bm.bmmc_copy(i, o, nbytes, h)
                if st != bm.OK:
                    raise bm.BmmcError(st, "bmmc_copy")
            ms = time_replays(self.torch, copy, bufs, steps, self.args.warmup, self.stream,
                              self.args.replays, graph=self.graph)
            self.copies[key] = replay_stats(ms, 2.0 * nbytes)
        return self.copies[key]

    def parity(self, plan, A, c, x, bufs):
        """Run the plan once more on the first pair and check it against the
        oracle: the whole array up to n = 24, 2^20 + 2 sampled elements
        (gathered on the device) above.  Returns (ok, text)."""
        torch = self.torch
        i0, o0 = bufs[0]
        o0.fill_(0xA5)
        plan(i0, o0, self.h)
        torch.cuda.synchronize()
        n = len(A)
        if self.args.no_check:
            return True, "skipped"
        if n <= 24:
            ok = full_parity(A, c, x, o0.cpu().numpy())
            return ok, ("bit-exact vs oracle (all %d elements)" % (1 << n) if ok else "MISMATCH")
        bad, checked = sampled_parity(torch, A, c, x, o0)
        return bad == 0, ("bit-exact vs oracle (%d sampled elements)" % checked if bad == 0
                          else "MISMATCH (%d of %d samples)" % (bad, checked))


def plan_brief(plan):
    d = plan.describe()
    return {"route": d["route"], "passes": d["passes"], "kernels": d["kernels"],
            "tile_log2": d["tile_log2"], "tile_skew": d["tile_skew"],
            "tile_threads": d["tile_threads"], "split_stage": d["split_stage"],
            "buffer_loads": d["buffer_loads"], "block_map": d["block_map"],
            "unit_bytes": d["unit_bytes"]}


def plan_label(d):
    """One line naming a tile plan's launch and shape (or a plan's kernels,
    when it has no tile pass), from Plan.describe()."""
    if d.get("tile_skew") is None:
        return "+".join(d["kernels"])
    return "%s t=%s skew %s%s%s%s order %s" % (
        d["kernels"][-1], d["tile_log2"], d["tile_skew"],
        " threads %d" % d["tile_threads"] if d.get("tile_threads") not in (None, 256) else "",
        " split" if d.get("split_stage") else "",
        " buffer loads" if d.get("buffer_loads") else "", d["block_map"])


def measure_case(run, name, route, x=None, bufs=None, A=None, c=None):
    """One configuration at its own size: plan, tune over the rotating pairs,
    time, and check; returns its entry of the configs object."""
    w = wl.WORKLOADS[name]
    n, elem = w.n, w.elem_bytes
    nbytes = elem << n
    if A is None:
        A, c = wl.workload_matrix(name, accept=lib_accepts(n))
    if x is None:
        x = wl.workload_data(name)
    if bufs is None:
        bufs = run.buffers(x, nbytes)
    plan = bm.Plan(n, A, c, elem, route=route)
    t0 = time.perf_counter()
    if not run.args.no_tune:
        plan.tune(pairs=bufs, stream=run.h)
    tune_ms = (time.perf_counter() - t0) * 1e3
    steps = run.steps_for(nbytes, headline=False)
    r = run.time_plan(plan, bufs, nbytes, steps)
    cp = run.copy_ceiling(bufs, nbytes, steps)
    ok, parity = run.parity(plan, A, c, x, bufs)
    e = {"workload": WORKLOAD_NAMES[name], "n": n, "elem_bytes": elem,
         "gbs": round(r["gbs"], 2), "gbs_min": round(r["gbs_min"], 2),
         "gbs_max": round(r["gbs_max"], 2), "ms_per_step": round(r["ms_per_step"], 6),
         "frac_of_copy": round(r["gbs"] / cp["gbs"], 4),
         "frac_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4),
         "copy_gbs": round(cp["gbs"], 2), "steps": steps, "replays": r["replays"],
         "plan": plan_brief(plan), "plan_options": plan.options(),
         "tune_ms": round(tune_ms, 1), "parity": parity}
    if plan.info.passes > 1:
        e["transfer_gbs"] = round(plan.info.passes * r["gbs"], 2)
    else:
        # HBM bytes per launch from the committed counter summary of this
        # plan, when there is one for this device code and these tables
        e["traffic"] = read_traffic(name, plan.options(), plan_tables_digest(plan))
    return e, ok


def measure_c5(run):
    """c5's protocol: each of the 32 seeded bit permutations planned, tuned,
    timed and checked on the same buffers; min / median / max."""
    w = wl.WORKLOADS["c5"]
    n, elem = w.n, w.elem_bytes
    nbytes = elem << n
    x = wl.workload_data("c5")
    bufs = run.buffers(x, nbytes)
    steps = run.steps_for(nbytes, headline=False)
    cp = run.copy_ceiling(bufs, nbytes, steps)
    vals, okays, plans, options = [], 0, [], []
    for k in range(C5_PERMS):
        A, c = wl.workload_matrix("c5", perm_index=k)
        plan = bm.Plan(n, A, c, elem)
        if not run.args.no_tune:
            plan.tune(pairs=bufs, stream=run.h)
        r = run.time_plan(plan, bufs, nbytes, steps)
        ok, parity = run.parity(plan, A, c, x, bufs)
        okays += ok
        vals.append(r["gbs"])
        plans.append(plan_label(plan.describe()))
        options.append(plan.options())
        log("c5 perm %d: %.1f GB/s (%.3f of copy) %s, %s" % (k, r["gbs"], r["gbs"] / cp["gbs"],
                                                          plans[-1], parity))
    order = sorted(range(len(vals)), key=lambda i: vals[i])
    med = 0.5 * (vals[order[len(vals) // 2 - 1]] + vals[order[len(vals) // 2]])
    e = {"workload": WORKLOAD_NAMES["c5"], "n": n, "elem_bytes": elem, "perms": len(vals),
         "min_gbs": round(vals[order[0]], 2), "median_gbs": round(med, 2),
         "max_gbs": round(vals[order[-1]], 2),
         "min_frac_of_copy": round(vals[order[0]] / cp["gbs"], 4),
         "median_frac_of_copy": round(med / cp["gbs"], 4),
         "max_frac_of_copy": round(vals[order[-1]] / cp["gbs"], 4),
         "median_frac_of_hbm_peak": round(med / HBM_PEAK_GBS, 4),
         "min_perm": order[0], "max_perm": order[-1], "copy_gbs": round(cp["gbs"], 2),
         "steps": steps, "replays": run.args.replays,
         "per_perm_gbs": [round(v, 1) for v in vals], "per_perm_plan": plans,
         "per_perm_options": options,
         "parity": ("bit-exact vs oracle on %d of %d permutations (2^20 + 2 sampled "
                    "elements each)" % (okays, len(vals)))}
    return e, okays == len(vals)


# Tensor front-end workloads: float32 tensors of 2^28 elements (1 GiB), the
# dimension permutations and flips of the Futhark page's LMAD layouts, as
# transformer-style shapes.
FRONTEND_CASES = [
    # (name, shape, perm, flip)
    ("batched_transpose", (64, 64, 256, 256), (0, 1, 3, 2), ()),
    ("heads_to_front", (16, 2048, 32, 256), (0, 2, 1, 3), ()),
    ("reverse_dims", (256, 256, 64, 64), (3, 2, 1, 0), ()),
    ("transpose_flip", (16384, 16384), (1, 0), (1,)),
]


def run_frontend(args, torch):
    """The tensor front-end (permute_dims, parm) on 1 GiB float32 tensors:
    each call as a user makes it (eager; the front-end plans on the first
    call and keeps the plan), against torch's own strided copy of the same
    view and bmmc_copy of the same bytes, all timed with events on the
    current stream; every output is compared with torch's.  parm's permutation by its matrix is timed alone
    as well and checked against the oracle on sampled elements.  One JSON
    line (not the headline)."""
    stream = torch.cuda.current_stream()
    h = int(stream.cuda_stream)
    n = 28
    nbytes = 4 << n
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(2024)
    src = torch.rand(1 << n, device="cuda:0", generator=gen)
    dst = torch.empty_like(src)
    steps = max(5, args.steps)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(args.replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b) / steps)
        return replay_stats(ms, 2.0 * nbytes)

    def copy():
        if bm.bmmc_copy(src, dst, nbytes, h) != bm.OK:
            raise bm.BmmcError(bm.ERR_HIP, "bmmc_copy")
    cp = timed(copy)["gbs"]
    entries = []
    ok_all = True
    for name, shape, perm, flip in FRONTEND_CASES:
        t = src.view(shape)
        view = t.flip(list(flip)) if flip else t
        view = view.permute(*perm)
        ours = timed(lambda: bm.permute_dims(t, perm, flip))
        tuned = timed(lambda: bm.permute_dims(t, perm, flip, tune=True))
        theirs = timed(lambda: dst.view(view.shape).copy_(view))
        got = bm.permute_dims(t, perm, flip)
        want = view.contiguous()
        ok = bool(torch.equal(got, want))
        got = bm.permute_dims(t, perm, flip, tune=True)
        ok &= bool(torch.equal(got, want))
        ok_all &= ok
        A, c, nb = bm.bmmc_tensor_permute_matrix([s.bit_length() - 1 for s in shape],
                                                 list(perm), sum(1 << d for d in flip))
        plan = bm.Plan(nb, A, c, (4 << n) >> nb)
        entries.append({"op": "permute_dims", "case": name, "shape": list(shape),
                        "perm": list(perm), "flip": list(flip), "dtype": "float32",
                        "gbs": round(ours["gbs"], 2), "frac_of_copy": round(ours["gbs"] / cp, 4),
                        "tuned_gbs": round(tuned["gbs"], 2),
                        "tuned_frac_of_copy": round(tuned["gbs"] / cp, 4),
                        "torch_gbs": round(theirs["gbs"], 2),
                        "vs_torch": round(ours["gbs"] / theirs["gbs"], 3),
                        "plan": plan_label(plan.describe()),
                        "parity": "bit-exact vs torch" if ok else "MISMATCH vs torch"})
        log("frontend %s: %.1f GB/s (%.3f of copy; tuned %.3f), torch %.1f GB/s, %s" % (
            name, ours["gbs"], ours["gbs"] / cp, tuned["gbs"] / cp, theirs["gbs"],
            entries[-1]["parity"]))
        del got, want
    # parm: the permutation by its matrix alone (tuned, as the library's
    # pass), then the whole call with f the identity
    mask = 0b1011 | (1 << 20)
    A = bm.bmmc_parm_matrix(n, mask)
    plan = bm.Plan(n, A, 0, 4)
    plan.tune(src, dst, stream=h)
    r = timed(lambda: plan(src, dst, h))
    x_host = src.cpu().numpy()
    plan(src, dst, h)
    torch.cuda.synchronize()
    bad, checked = sampled_parity(torch, A, 0, x_host, dst)
    ok_all &= bad == 0
    whole = timed(lambda: bm.parm(src, mask, lambda y: y))
    entries.append({"op": "parm", "n": n, "mask": mask, "dtype": "float32",
                    "gbs": round(r["gbs"], 2), "frac_of_copy": round(r["gbs"] / cp, 4),
                    "plan": plan_label(plan.describe()),
                    "parm_call_ms": round(whole["ms_per_step"], 4),
                    "parm_call_vs_copies": round(whole["ms_per_step"] / (2.0 * nbytes / (cp * 1e9) * 1e3), 3),
                    "parity": "bit-exact vs oracle (%d sampled elements)" % checked if not bad
                              else "MISMATCH vs oracle (%d of %d)" % (bad, checked)})
    log("frontend parm permutation: %.1f GB/s (%.3f of copy), %s; whole call %.3f ms" % (
        r["gbs"], r["gbs"] / cp, entries[-1]["parity"], whole["ms_per_step"]))
    print(json.dumps({"metric": "frontend", "unit": "GB/s", "copy_gbs": round(cp, 2),
                      "steps": steps, "replays": args.replays, "entries": entries}))
    sys.stdout.flush()
    if not ok_all:
        sys.exit(3)


def run_candidates(torch, args, run, plan, n, A, c, elem, x, bufs, workload_name):
    """Every plan bmmc_plan_tune_pairs would time, in its order: one
    bmmc_copy of the array, then --steps executions of the candidate, on the
    stream, one candidate after the other.  In a counter run, each candidate's
    dispatches are those between two copies.  Prints the candidates' options
    and table digests as one JSON line; the last execution of each is checked
    against the oracle on sampled elements."""
    nbytes = elem << n
    i0, o0 = bufs[0]
    out = []
    ok_all = True
    for k, opts in enumerate(bm.bmmc_plan_tune_candidates(plan.handle)):
        q = bm.Plan(n, A, c, elem, **opts)
        st = bm.bmmc_copy(i0, o0, nbytes, run.h)
        if st != bm.OK:
            raise bm.BmmcError(st, "bmmc_copy")
        for _ in range(args.steps):
            q(i0, o0, run.h)
        torch.cuda.synchronize()
        ok, parity = run.parity(q, A, c, x, bufs)
        ok_all &= ok
        out.append({"index": k, "plan_options": q.options(),
                    "plan_tables_digest": plan_tables_digest(q),
                    "kernels": q.describe()["kernels"], "parity": parity})
        log("candidate %d: %s %s" % (k, json.dumps(q.options(), sort_keys=True), parity))
    print(json.dumps({"workload": workload_name, "kernel_source_digest": kernel_source_digest(),
                      "bytes": int(nbytes), "runs_per_candidate": args.steps,
                      "candidates": out}))
    sys.stdout.flush()
    if not ok_all:
        sys.exit(3)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed steps per timed region of the headline (the other "
                         "configurations take more on small arrays)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replays", type=int, default=5,
                    help="timed regions per measurement; the median is reported, with min and max")
    ap.add_argument("--workload", default="c4", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--configs", default="auto", choices=["auto", "all", "none"],
                    help="also measure every other configuration (auto: only with the "
                         "default headline)")
    ap.add_argument("--kind", default=None,
                    choices=["bitrev", "transpose", "bpc", "bmmc", "blockperm", "reverse"],
                    help="custom workload instead of --workload: the matrix kind "
                         "(blockperm: identity on the low --seg-log2 bits, random on the rest)")
    ap.add_argument("--seg-log2", type=int, default=10, help="blockperm: block size, log2 elements")
    ap.add_argument("--n", type=int, default=24, help="custom workload: index bits")
    ap.add_argument("--elem", type=int, default=4, help="custom workload: element bytes")
    ap.add_argument("--seed", type=int, default=1, help="custom workload: matrix seed")
    ap.add_argument("--perm", type=int, default=0, help="c5: permutation index 0..31")
    ap.add_argument("--perms", type=int, default=0,
                    help="c5 as --workload: time permutations 0..PERMS-1 and report "
                         "min/median/max")
    ap.add_argument("--route", default="auto", choices=["auto", "naive", "two_pass", "fused"])
    ap.add_argument("--tile-log2", type=int, default=0)
    ap.add_argument("--iters-log2", type=int, default=0)
    ap.add_argument("--no-swizzle", action="store_true")
    ap.add_argument("--launch", default="auto",
                    choices=["auto", "one_tile", "persistent", "streamed"])
    ap.add_argument("--grid-log2", type=int, default=0)
    ap.add_argument("--walk", default="auto", choices=["auto", "ranges", "interleaved"])
    ap.add_argument("--block-map", type=int, default=0)
    ap.add_argument("--depth", type=int, default=0)
    ap.add_argument("--cache-hint", type=int, default=0)
    ap.add_argument("--plan-options", default=None,
                    help="JSON object of plan options, as printed in config.plan_options: "
                         "build exactly that plan and skip the tuning")
    ap.add_argument("--warm", action="store_true", help="reuse one buffer pair")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager calls from Python instead of replaying a HIP graph of them")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip bmmc_plan_tune (the planner's untimed choice of tile order)")
    ap.add_argument("--ablation", action="store_true",
                    help="the paper's Figure 9/11 variants over kinds and sizes, "
                         "one JSON line each (not the headline line)")
    ap.add_argument("--sizes", default="20,24,28", help="ablation: comma-separated n")
    ap.add_argument("--frontend", action="store_true",
                    help="the tensor front-end (permute_dims on 1 GiB float32 tensors, parm) "
                         "against torch's strided copy, as one JSON line (not the headline)")
    ap.add_argument("--candidates", action="store_true",
                    help="run every plan the tuning would time for the workload, each "
                         "--steps times after one bmmc_copy of the array (a separator for "
                         "counter runs), and print them as one JSON line (not timed)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU only (no sharding or collectives); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.replays < 1:
        print("bench.py: --steps and --replays must be positive", file=sys.stderr)
        sys.exit(2)
    explicit_workload = "--workload" in sys.argv[1:] or any(
        a.startswith("--workload=") for a in sys.argv[1:])
    with_configs = args.configs == "all" or (
        args.configs == "auto" and not (args.kind or args.plan_options or explicit_workload
                                        or args.perms or args.warm))

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    bm.lib()  # fails loudly when the HIP library is missing

    if args.ablation:
        run_ablation(args, torch)
        return
    if args.frontend:
        run_frontend(args, torch)
        return

    name = args.workload
    if args.kind:
        n, elem = args.n, args.elem
        if args.kind == "bitrev":
            A, c = wl.bit_reverse_matrix(n), 0
        elif args.kind == "transpose":
            A, c = wl.transpose_matrix(n // 2, n - n // 2), 0
        elif args.kind == "bpc":
            A, c = wl.random_bpc(n, args.seed)
        elif args.kind == "reverse":
            # the whole array reversed: A = I with every complement bit set
            A, c = wl.identity_matrix(n), (1 << n) - 1
        elif args.kind == "blockperm":
            sl = args.seg_log2
            Q, _ = wl.random_bmmc(n - sl, args.seed, lib_accepts(n - sl))
            A = np.array([1 << r for r in range(sl)] + [int(q) << sl for q in Q], dtype=np.uint64)
            c = 0
        else:
            A, c = wl.random_bmmc(n, args.seed, lib_accepts(n))
        x = wl.fill_random_bytes(n, elem, args.seed)
        workload_name = "%s_n%d_%dB" % (args.kind, n, elem) + (
            "_seg%d" % args.seg_log2 if args.kind == "blockperm" else "")
    else:
        w = wl.WORKLOADS[name]
        n, elem = w.n, w.elem_bytes
        A, c = wl.workload_matrix(name, accept=lib_accepts(n), perm_index=args.perm)
        x = wl.workload_data(name)
        workload_name = WORKLOAD_NAMES[name] + ("_perm%d" % args.perm if name == "c5" else "")
    nbytes = elem << n
    route = {"auto": bm.ROUTE_AUTO, "naive": bm.ROUTE_NAIVE, "two_pass": bm.ROUTE_TWO_PASS,
             "fused": bm.ROUTE_FUSED}[args.route]
    launch = {"auto": bm.LAUNCH_AUTO, "one_tile": bm.LAUNCH_ONE_TILE,
              "persistent": bm.LAUNCH_PERSISTENT, "streamed": bm.LAUNCH_STREAMED}[args.launch]
    plan_kw = dict(route=route, tile_log2=args.tile_log2, no_swizzle=args.no_swizzle,
                   iters_log2=args.iters_log2, launch=launch, grid_log2=args.grid_log2,
                   walk={"auto": 0, "ranges": 1, "interleaved": 2}[args.walk],
                   block_map=args.block_map, depth=args.depth, cache_hint=args.cache_hint)

    t0 = time.perf_counter()
    if args.plan_options:
        plan = bm.Plan(n, A, c, elem, **json.loads(args.plan_options))
        args.no_tune = True
    else:
        plan = bm.Plan(n, A, c, elem, **plan_kw)
    plan_us = (time.perf_counter() - t0) * 1e6
    if name == "c4" and not args.kind and route == bm.ROUTE_TWO_PASS:
        assert plan.info.passes == 2

    run = Runner(torch, args)
    log("headline %s: %s" % (workload_name, plan.describe()["kernels"]))
    bufs = run.buffers(x, nbytes)
    if args.candidates:
        run_candidates(torch, args, run, plan, n, A, c, elem, x, bufs, workload_name)
        return

    # bmmc_plan_tune_pairs: time the candidate tile orders over the same
    # rotating buffer pairs and keep the fastest (outside the timed region,
    # like plan creation)
    tune_ms = None
    if not args.no_tune:
        t0 = time.perf_counter()
        plan.tune(pairs=bufs, stream=run.h)
        tune_ms = (time.perf_counter() - t0) * 1e3

    def step(i, o, h):
        st = bm.bmmc_execute(plan.handle, i, o, h)
        if st != bm.OK:
            raise bm.BmmcError(st, "bmmc_execute")

    r = run.time_plan(plan, bufs, nbytes, args.steps)
    cp = run.copy_ceiling(bufs, nbytes, args.steps)
    med, mn, mx = per_launch_ms(torch, step, bufs, 20, run.stream)
    algo_bytes = 2.0 * nbytes
    value = r["gbs"]
    copy_gbs = cp["gbs"]
    log("headline: %.1f GB/s (%.3f of copy)" % (value, value / copy_gbs))

    perm_stats = None
    if args.perms and name == "c5" and not args.kind:
        # the workload's protocol: every permutation planned, tuned, timed and
        # checked the same way on the same buffers; min / median / max
        vals, okays = [], 0
        for k in range(args.perms):
            Ak, ck = wl.workload_matrix(name, perm_index=k)
            pk = bm.Plan(n, Ak, ck, elem, **plan_kw)
            if not args.no_tune:
                pk.tune(pairs=bufs, stream=run.h)
            rk = run.time_plan(pk, bufs, nbytes, args.steps)
            okk, park = run.parity(pk, Ak, ck, x, bufs)
            okays += okk
            vals.append(rk["gbs"])
            log("perm %d: %.1f GB/s (%s) %s" % (k, vals[-1], plan_label(pk.describe()), park))
        sv = sorted(vals)
        pmed = 0.5 * (sv[(len(sv) - 1) // 2] + sv[len(sv) // 2])
        perm_stats = {"perms": len(vals), "min_gbs": round(sv[0], 2),
                      "median_gbs": round(pmed, 2), "max_gbs": round(sv[-1], 2),
                      "min_frac_of_copy": round(sv[0] / copy_gbs, 4),
                      "median_frac_of_copy": round(pmed / copy_gbs, 4),
                      "max_frac_of_copy": round(sv[-1] / copy_gbs, 4),
                      "parity": "bit-exact on %d of %d permutations" % (okays, len(vals))}
        if okays != len(vals):
            perm_stats["parity"] = "MISMATCH: " + perm_stats["parity"]

    ok, parity = run.parity(plan, A, c, x, bufs)
    if not ok:
        print("bench.py: output does not match the oracle: %s" % parity, file=sys.stderr)
    all_ok = ok and not (perm_stats and perm_stats["parity"].startswith("MISMATCH"))

    plan_options = plan.options()
    traffic = None if args.kind else read_traffic(name, plan_options, plan_tables_digest(plan))
    passes = plan.info.passes
    # average launch duration over every timed region (one launch per step
    # for a one-pass plan)
    achieved = algo_bytes / (r["ms_mean"] * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-normalised)",
        "algorithmic_bytes_per_launch": int(algo_bytes),
        "kernel": plan.describe()["kernels"][-1],
    }
    if passes > 1:
        roofline["kernel"] = "both passes of the two-pass plan (one step)"

    result = {
        "metric": "effective GB/s (bytes read+written / time) and fraction of copy ceiling",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {1: "u8", 2: "u16", 4: "u32", 8: "u64", 16: "u128"}[plan.info.unit_bytes],
        "data": "synthetic",
        "config": {
            "workload": workload_name,
            "n": n, "elem_bytes": elem, "bytes_per_step": int(algo_bytes),
            "residency": ("one buffer pair, repeated (cache-warm)" if args.warm else
                          "%d rotating buffer pairs, %.2f GiB working set (HBM)"
                          % (len(bufs), 2 * len(bufs) * nbytes / 2**30)),
            "plan": plan.describe(),
            "plan_options": plan_options,
            "timing": ("%d timed regions of %d eager calls from Python; median"
                       % (args.replays, args.steps) if args.no_graph else
                       "one HIP graph of the %d steps, replayed in %d timed regions; median"
                       % (args.steps, args.replays)),
        },
        "replays": {"count": r["replays"], "value_min": round(r["gbs_min"], 2),
                    "value_max": round(r["gbs_max"], 2),
                    "ms_per_step_min": round(r["ms_min"], 6),
                    "ms_per_step_max": round(r["ms_max"], 6)},
        "frac_of_copy": round(value / copy_gbs, 4),
        "copy_ceiling_gbs": round(copy_gbs, 2),
        "copy_ceiling_min_max_gbs": [round(cp["gbs_min"], 2), round(cp["gbs_max"], 2)],
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "launch_ms": {"median": round(med, 5), "min": round(mn, 5), "max": round(mx, 5)},
        "plan_create_us": round(plan_us, 1),
        "plan_tune_ms": round(tune_ms, 1) if tune_ms is not None else None,
        "parity": parity,
        "roofline": roofline,
    }
    if perm_stats:
        result["permutations"] = perm_stats
    if passes > 1:
        # bytes the passes move in total (each reads and writes the array)
        result["transfer_gbs"] = round(passes * value, 2)

    configs = None
    if with_configs:
        configs = {"c4_fused": {"workload": workload_name, "gbs": result["value"],
                                "frac_of_copy": result["frac_of_copy"],
                                "frac_of_hbm_peak": result["frac_of_hbm_peak"],
                                "parity": parity, "see": "headline"}}
        for key, cname, croute in CONFIG_CASES:
            if key == "c5":
                continue
            if cname != "c4":
                continue
            e, okc = measure_case(run, cname, croute, x=x, bufs=bufs, A=A, c=c)
            configs[key] = e
            all_ok &= okc
            log("%s: %.1f GB/s (%.3f of copy), %s" % (key, e["gbs"], e["frac_of_copy"],
                                                      e["parity"]))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, %d threads, about %.0f s)" % (oracle_threads(),
                                                                   1.2 * args.cpu_budget))
        result["cpu_baseline"] = cpu_baseline(A, c, x, args.cpu_budget)
    if with_configs:
        del bufs, step
        plan.close()
        x = None
        torch.cuda.empty_cache()
        for key, cname, croute in CONFIG_CASES:
            if cname == "c4":
                continue
            if key == "c5":
                e, okc = measure_c5(run)
            else:
                e, okc = measure_case(run, cname, croute)
            configs[key] = e
            all_ok &= okc
            log("%s: %s, %s" % (key, ("%.1f GB/s (%.3f of copy)" % (e["gbs"], e["frac_of_copy"])
                                      if "gbs" in e else
                                      "min/median/max %.3f/%.3f/%.3f of copy"
                                      % (e["min_frac_of_copy"], e["median_frac_of_copy"],
                                         e["max_frac_of_copy"])), e["parity"]))
            torch.cuda.empty_cache()
        result["configs"] = configs
    print(json.dumps(result))
    sys.stdout.flush()
    if not all_ok:
        sys.exit(3)


if __name__ == "__main__":
    main()
