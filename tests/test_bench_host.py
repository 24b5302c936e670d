"""CPU tests of bench.py's host-side parts: the oracle CPU baseline, the
ablation variants (planned on the host), the HBM-traffic reader and the
refusal of more than one GPU.  No GPU call is made."""
import json
import os
import subprocess
import sys

import pytest

import oracle
import bmmc_affine_index_amd as bm
from bmmc_affine_index_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_cpu_baseline_fields():
    oracle.build()
    A, c = wl.workload_matrix("c1b")
    x = wl.workload_data("c1b")
    r = bench.cpu_baseline(A, c, x, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["single_thread_value"] > 0 and r["cores"] >= 1
    assert isinstance(r["cpu_model"], str) and r["host_cpus"] >= 1
    json.dumps(r)


def test_ablation_variants_plan_on_host():
    for n in (20, 24):
        kinds = [wl.random_bpc(n, 7), (wl.bit_reverse_matrix(n), 0),
                 wl.random_bmmc(n, 7, bench.lib_accepts(n))]
        for A, c in kinds:
            for name, kw in bench.ABLATION_VARIANTS:
                kw = {k: v for k, v in kw.items() if k != "tune"}
                P = bm.Plan(n, A, c, 4, **kw)
                assert P.info.passes in (1, 2), name
                P = bm.Plan(n, A, c, 4, route=bm.ROUTE_TWO_PASS,
                            **{k: v for k, v in kw.items() if k != "route"})
                assert P.info.passes in (1, 2)


def test_traffic_reader_and_digest(tmp_path, monkeypatch):
    d = bench.kernel_source_digest()
    assert isinstance(d, str) and len(d) == 16
    A, c = wl.workload_matrix("c2")
    P = bm.Plan(24, A, c, 4)
    opts, tabs = P.options(), bench.plan_tables_digest(P)
    assert tabs == bench.plan_tables_digest(bm.Plan(24, A, c, 4, **opts))
    Q = bm.Plan(24, A, c, 4, tile_log2=opts["tile_log2"] + 1)
    assert bench.plan_tables_digest(Q) != tabs
    for w in ("c2", "c4"):
        t = bench.read_traffic(w, opts, tabs)
        assert t is None or t > 0
    # a summary counts only for the plan and tables it was taken with, at
    # this device code
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "hbm_traffic_%s.txt"))

    def entry(digest, options, tables, nbytes):
        return ("[entry]\n# comment = ignored\nkernel_source_digest=%s\nplan_options=%s\n"
                "plan_tables_digest=%s\nhbm_bytes_per_launch=%d\n"
                % (digest, json.dumps(options), tables, nbytes))

    def write(*entries):
        (tmp_path / "hbm_traffic_c2.txt").write_text("# header = ignored\n" + "".join(entries))
    write(entry(d, opts, tabs, 134618399))
    assert bench.read_traffic("c2", opts, tabs) == 134618399.0
    assert bench.read_traffic("c2", Q.options(), tabs) is None
    assert bench.read_traffic("c2", opts, bench.plan_tables_digest(Q)) is None
    # several plans counted: each finds its own entry
    qtabs = bench.plan_tables_digest(Q)
    write(entry(d, Q.options(), qtabs, 134300000), entry(d, opts, tabs, 134618399))
    assert bench.read_traffic("c2", opts, tabs) == 134618399.0
    assert bench.read_traffic("c2", Q.options(), qtabs) == 134300000.0
    write(entry("0" * 16, opts, tabs, 134618399))
    assert bench.read_traffic("c2", opts, tabs) is None
    assert bench.read_traffic("c3", opts, tabs) is None  # no summary at all


def test_plan_options_rebuild_the_plan():
    A, c = wl.workload_matrix("c3")
    P = bm.Plan(28, A, c, 4, launch=bm.LAUNCH_PERSISTENT, tile_log2=7, block_map=6)
    Q = bm.Plan(28, A, c, 4, **json.loads(json.dumps(P.options())))
    assert Q.describe() == P.describe()
    for a, b in zip(P.passes(), Q.passes()):
        assert bytes(a) == bytes(b)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_help_lists_protocol_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--no-graph", "--no-tune", "--ablation", "--perms",
                "--plan-options"):
        assert opt in r.stdout


def test_replay_stats_median_and_range():
    r = bench.replay_stats([2.0, 1.0, 4.0, 3.0, 5.0], 8e9)
    assert r["ms_per_step"] == 3.0 and r["ms_min"] == 1.0 and r["ms_max"] == 5.0
    assert r["replays"] == 5 and abs(r["ms_mean"] - 3.0) < 1e-12
    assert abs(r["gbs"] - 8e9 / 3e-3 / 1e9) < 1e-9
    assert r["gbs_min"] < r["gbs"] < r["gbs_max"]
    assert bench.replay_stats([2.0, 4.0], 1e9)["ms_per_step"] == 3.0


def test_oracle_threads_follows_the_host_share(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "5")
    assert bench.oracle_threads() == 5
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.oracle_threads() == len(os.sched_getaffinity(0))


def test_sampled_parity_on_host_tensors():
    """The device-gather parity check, run on CPU tensors: it passes the
    oracle's own output and catches a single planted misplacement."""
    import numpy as np
    import torch
    n = 16
    for elem in (4, 16):
        A, c = wl.random_bmmc(n, 3 + elem, lambda r: oracle.rank(r) == n)
        x = wl.fill_random_bytes(n, elem, 5)
        want = oracle.apply(A, c, x)
        out = torch.from_numpy(want.reshape(-1).copy())
        bad, checked = bench.sampled_parity(torch, A, c, x, out, samples=1 << 12)
        assert bad == 0 and checked == (1 << 12) + 2
        # swap two output elements the sample covers (the last index is always sampled)
        j = int(oracle.map_indices(A, c, np.array([(1 << n) - 1], dtype=np.uint64))[0])
        k = int(oracle.map_indices(A, c, np.array([0], dtype=np.uint64))[0])
        w2 = want.copy()
        w2[[j, k]] = w2[[k, j]]
        bad, _ = bench.sampled_parity(torch, A, c, x, torch.from_numpy(w2.reshape(-1).copy()),
                                      samples=1 << 12)
        assert bad >= 2


def test_plan_label_names_shape_threads_split_and_loads():
    import bmmc_affine_index_amd as bm
    from bmmc_affine_index_amd import workloads as wl
    P = bm.Plan(20, wl.bit_reverse_matrix(20), 0, 4, split_stage=1, tile_log2=7,
                tile_threads_log2=9, tile_skew=1)
    assert bench.plan_label(P.describe()) == "one_tile t=7 skew 1 threads 512 split order 5"
    Q = bm.Plan(20, wl.bit_reverse_matrix(20), 0, 4, launch=bm.LAUNCH_STREAMED, tile_log2=7)
    assert bench.plan_label(Q.describe()) == "streamed t=7 skew 0 order 5"
    R = bm.Plan(20, wl.identity_matrix(20), (1 << 20) - 1, 4)
    assert bench.plan_label(R.describe()) == "chunk_scatter"
    brief = bench.plan_brief(P)
    assert brief["tile_threads"] == 512 and brief["split_stage"] == 1 and brief["tile_skew"] == 1
    assert brief["buffer_loads"] == 0
    B = bm.Plan(20, wl.bit_reverse_matrix(20), 0, 4, buffer_loads=1, tile_log2=6, block_map=8)
    assert bench.plan_label(B.describe()) == "one_tile t=6 skew 0 buffer loads order 8"
    assert bench.plan_brief(B)["buffer_loads"] == 1


def test_frontend_cases_are_one_gib_and_plan_on_the_host():
    """The front-end benchmark's tensors hold 2^28 float32 elements, and the
    library plans each dimension permutation as one bit-permute-complement."""
    import bmmc_affine_index_amd as bm
    for name, shape, perm, flip in bench.FRONTEND_CASES:
        total = 1
        for s in shape:
            assert s & (s - 1) == 0
            total *= s
        assert total == 1 << 28, name
        assert sorted(perm) == list(range(len(shape)))
        A, c, n = bm.bmmc_tensor_permute_matrix([s.bit_length() - 1 for s in shape], list(perm),
                                                sum(1 << d for d in flip))
        P = bm.Plan(n, A, c, (4 << 28) >> n)
        assert P.info.kind in (bm.KIND_BPC, bm.KIND_IDENTITY)
        assert P.info.passes == 1


def _write_counter_csv(path, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for k, (name, counter, value) in enumerate(rows):
            r = dict.fromkeys(cols, "0")
            r.update(Dispatch_Id=str(k + 1), Process_Id="7", Kernel_Name=name,
                     Counter_Name=counter, Counter_Value=repr(value))
            w.writerow([r[c] for c in cols])


def test_traffic_summary_round_trip(tmp_path, monkeypatch):
    """bench_profiles.py turns two counter runs of --candidates into entries
    that read_traffic finds for exactly the plans counted: copies separate
    the candidates, torch's kernels are left out, each counter is scaled by
    the copy's reading, and the dispatches of a candidate are averaged over
    its timed runs and its parity run."""
    import bench_profiles
    nbytes = 1 << 26
    A, c = wl.workload_matrix("c2")
    P = bm.Plan(24, A, c, 4)
    cands = []
    for k, o in enumerate(bm.bmmc_plan_tune_candidates(P.handle)[:3]):
        Q = bm.Plan(24, A, c, 4, **o)
        cands.append({"index": k, "plan_options": Q.options(),
                      "plan_tables_digest": bench.plan_tables_digest(Q),
                      "kernels": Q.describe()["kernels"], "parity": "bit-exact"})
    line = {"workload": "transpose4096x4096_fp32_n24",
            "kernel_source_digest": bench.kernel_source_digest(), "bytes": nbytes,
            "runs_per_candidate": 3, "candidates": cands}
    copy_read_kib, copy_write_kib = nbytes / 2048.0, nbytes / 1024.0  # reads counted at half
    dirs = []
    for counter, copy_kib in (("FETCH_SIZE", copy_read_kib), ("WRITE_SIZE", copy_write_kib)):
        d = tmp_path / counter
        rows = [("at::native::fill", counter, 123.0)]
        for k in range(len(cands)):
            rows.append(("bmmc::bmmc_copy_kernel<0>", counter, copy_kib))
            for _ in range(4):  # 3 timed runs + the parity run
                rows.append(("bmmc::bmmc_tiled_kernel<2, 7, 0, true, 8>", counter,
                             copy_kib * (1.0 + 0.01 * k)))
                rows.append(("at::native::vectorized_gather_kernel", counter, 99.0))
        _write_counter_csv(str(d / "host" / "run_counter_collection.csv"), rows)
        (d / "candidates.json").write_text("log line\n" + json.dumps(line) + "\n")
        dirs.append(str(d))
    text = bench_profiles.traffic_summary("c2", [tuple(dirs)], ["cmd"])
    assert text.count("[entry]") == 3
    f = tmp_path / "hbm_traffic_c2.txt"
    f.write_text(text)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "hbm_traffic_%s.txt"))
    for k, cand in enumerate(cands):
        got = bench.read_traffic("c2", cand["plan_options"], cand["plan_tables_digest"])
        assert got == pytest.approx(2 * nbytes * (1.0 + 0.01 * k), rel=1e-6)
    # a plan that was not counted has no traffic
    assert bench.read_traffic("c2", cands[0]["plan_options"], "0" * 16) is None
    # the compact form: one table row per candidate with its ratio, no entries
    compact = bench_profiles.traffic_summary("c2", [tuple(dirs)], ["cmd"], compact=True)
    assert "[entry]" not in compact
    ratios = [float(line.rsplit("|", 2)[1]) for line in compact.splitlines()
              if line.startswith("| ") and line[2].isdigit()]
    assert ratios == pytest.approx([1.0 + 0.01 * k for k in range(len(cands))], rel=1e-5)
    # candidates that do not match the runs' copies are refused
    bad = dict(line, candidates=cands[:2])
    (tmp_path / "FETCH_SIZE" / "candidates.json").write_text(json.dumps(bad) + "\n")
    (tmp_path / "WRITE_SIZE" / "candidates.json").write_text(json.dumps(bad) + "\n")
    with pytest.raises(SystemExit):
        bench_profiles.traffic_summary("c2", [tuple(dirs)], ["cmd"])


def test_trace_summary_finds_the_timed_window(tmp_path):
    """The headline's timed dispatches are the steps x replays library
    dispatches right before the copy ceiling's first run of warm-up + upload
    + timed copies of one grid."""
    import csv
    import bench_profiles
    steps, warmup, replays = 4, 2, 3
    disp = [("bmmc::bmmc_copy_kernel<0>", 32, 100)] * 500  # a smaller array's copies
    disp += [("bmmc::bmmc_tiled_kernel<2, 6, 0, true, 9>", 64, 5000)] * 7  # tuning
    disp += [("bmmc::bmmc_tiled_kernel<2, 6, 0, true, 8>", 64, 1000)] * (warmup + steps)
    disp += [("at::native::fill", 8, 10)]
    disp += [("bmmc::bmmc_tiled_kernel<2, 6, 0, true, 8>", 64, 2000 + k)
             for k in range(replays * steps)]
    disp += [("bmmc::bmmc_copy_kernel<0>", 128, 1400)] * warmup
    disp += [("at::native::fill", 8, 10)]
    disp += [("bmmc::bmmc_copy_kernel<0>", 128, 1500)] * steps
    disp += [("bmmc::bmmc_copy_kernel<0>", 128, 1600 + k) for k in range(replays * steps)]
    disp += [("bmmc::bmmc_copy_kernel<0>", 32, 100)] * 50
    d = tmp_path / "trace"
    os.makedirs(d / "h")
    with open(d / "h" / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Grid_Size_Y",
                    "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for k, (name, grid, dur) in enumerate(disp):
            w.writerow(["KERNEL_DISPATCH", k + 1, name, grid, 1, 1, t, t + dur])
            t += dur + 10
    timed, copies = bench_profiles.headline_window(
        bench_profiles.trace_dispatches(str(d)), steps, warmup, replays, 128)
    assert [t for _, _, t in timed] == [2000 + k for k in range(replays * steps)]
    assert [t for _, _, t in copies] == [1600 + k for k in range(replays * steps)]
