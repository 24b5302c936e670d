"""Turn rocprofv3 output of bench.py runs into the text summaries kept under
profiles/ (no GPU needed; reads CSV files only).

HBM traffic of every tuning candidate, from two counter runs of
``bench.py --candidates`` (one with --pmc FETCH_SIZE, one with --pmc
WRITE_SIZE), each run's JSON line saved as candidates.json in its rocprofv3
output directory:

    python bench_profiles.py traffic --workload c4 FETCH_DIR WRITE_DIR [FETCH_DIR2 WRITE_DIR2 ...]

Kernel trace of a bench.py run (rocprofv3 --kernel-trace --stats), its JSON
line saved as bench.json in the output directory:

    python bench_profiles.py trace DIR

Both print the summary on stdout.  The commands that produced the input are
written into the summary by the caller's --command options.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DESCRIPTIONS = {
    "c1a": "random BMMC n = 20, int32 (4 MiB), fused single pass",
    "c1b": "bit reversal n = 20, int32 (4 MiB)",
    "c2": "4096 x 4096 fp32 transpose as a BMMC on n = 24 (64 MiB)",
    "c3": "bit reversal n = 28, int32 (1 GiB)",
    "c4": "random BMMC n = 30, int32 (4 GiB per array), fused single pass",
    "c5": "random 16-byte BPC n = 27 (2 GiB)",
}

COPY_KERNELS = ("bmmc_copy_kernel", "bmmc_copy_stride_kernel", "bmmc_copy_bytes_kernel")


def short_name(name: str) -> str:
    """A kernel's name without its return type and parameter list."""
    if name.startswith("void "):
        name = name[5:]
    if name.endswith(")"):
        depth = 0
        for k in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[k], 0)
            if depth == 0:
                return name[:k]
    return name


def is_copy(name: str) -> bool:
    return any(k in name for k in COPY_KERNELS)


def is_library(name: str) -> bool:
    return name.startswith("bmmc::") or " bmmc::" in name


def find_csvs(d: str, suffix: str):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit("bench_profiles.py: no *%s under %s" % (suffix, d))
    return hits


def pick(row: dict, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError("none of %s in %s" % (names, sorted(row)))


def last_json_line(path: str) -> dict:
    with open(path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.strip().startswith("{")]
    if not lines:
        raise SystemExit("bench_profiles.py: no JSON line in %s" % path)
    return json.loads(lines[-1])


# ---- counters ------------------------------------------------------------

def counter_dispatches(d: str, counter: str):
    """[(kernel name, value)] per dispatch in dispatch order; a counter that
    comes as several rows of one dispatch (one per hardware instance) is
    summed."""
    per = {}
    for path in find_csvs(d, "counter_collection.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if pick(r, "Counter_Name", "Counter") != counter:
                    continue
                key = (int(pick(r, "Process_Id", "Pid")) if "Process_Id" in r else 0,
                       int(pick(r, "Dispatch_Id", "Dispatch_ID")))
                name = pick(r, "Kernel_Name", "Kernel-Name")
                e = per.setdefault(key, [name, 0.0])
                e[1] += float(pick(r, "Counter_Value", "Value"))
    return [per[k] for k in sorted(per)]


def segments(dispatches):
    """Split the library's dispatches at the copies: (copy values, [candidate
    segments]), each segment the (name, value) dispatches after one copy."""
    copies, segs, cur = [], [], None
    for name, v in dispatches:
        if not is_library(name):
            continue  # torch's fills and gathers of the parity checks
        if is_copy(name):
            copies.append(v)
            cur = []
            segs.append(cur)
        elif cur is not None:
            cur.append((name, v))
    return copies, segs


def traffic_summary(workload: str, pairs, commands, compact: bool = False) -> str:
    """The summary text.  Entries (key=value blocks that bench.py reads back)
    per candidate, or with compact=True one table row per candidate."""
    out = []
    blocks = []
    for fetch_dir, write_dir in pairs:
        cf = last_json_line(os.path.join(fetch_dir, "candidates.json"))
        cw = last_json_line(os.path.join(write_dir, "candidates.json"))
        if cf != cw:
            raise SystemExit("bench_profiles.py: the two runs timed different candidates")
        nbytes = int(cf["bytes"])
        execs = int(cf["runs_per_candidate"]) + 1  # the timed runs and the parity run
        fc, fseg = segments(counter_dispatches(fetch_dir, "FETCH_SIZE"))
        wc, wseg = segments(counter_dispatches(write_dir, "WRITE_SIZE"))
        cands = cf["candidates"]
        if not (len(fseg) == len(wseg) == len(cands)):
            raise SystemExit("bench_profiles.py: %d / %d copy-separated segments for %d "
                             "candidates" % (len(fseg), len(wseg), len(cands)))
        fcopy, wcopy = statistics.median(fc), statistics.median(wc)
        rscale, wscale = nbytes / (fcopy * 1024.0), nbytes / (wcopy * 1024.0)
        entries, ratios = [], []
        for cand, fs, ws in zip(cands, fseg, wseg):
            if len(fs) != len(ws) or not fs or len(fs) % execs:
                raise SystemExit("bench_profiles.py: candidate %d has %d / %d dispatches"
                                 % (cand["index"], len(fs), len(ws)))
            names = sorted({short_name(n) for n, _ in fs})
            f_kib = sum(v for _, v in fs) / execs
            w_kib = sum(v for _, v in ws) / execs
            rd, wr = f_kib * 1024.0 * rscale, w_kib * 1024.0 * wscale
            ratio = (rd + wr) / (2.0 * nbytes)
            ratios.append(ratio)
            if compact:
                o = cand["plan_options"]
                entries.append("| %d | %s | %s | %s | %s | %s | %s | %.5f |" % (
                    cand["index"], ", ".join(n.replace("bmmc::bmmc_", "") for n in names),
                    o.get("tile_log2"), o.get("tile_skew"), o.get("block_map"),
                    "split" if o.get("split_stage") else "",
                    "buffer" if o.get("buffer_loads") else "", ratio))
                continue
            entries.append("\n".join([
                "[entry]",
                "# candidate %d: %s; %d dispatches each side; %s" % (
                    cand["index"], ", ".join(names), len(fs), cand["parity"]),
                "#   FETCH_SIZE %.1f KiB -> %d bytes read; WRITE_SIZE %.1f KiB -> %d bytes "
                "written; measured / algorithmic = %.5f" % (f_kib, rd, w_kib, wr, ratio),
                "kernel_source_digest=%s" % cf["kernel_source_digest"],
                "plan_tables_digest=%s" % cand["plan_tables_digest"],
                "plan_options=%s" % json.dumps(cand["plan_options"], sort_keys=True,
                                               separators=(",", ":")),
                "hbm_bytes_per_launch=%d" % round(rd + wr),
                "algorithmic_bytes_per_launch=%d" % (2 * nbytes),
            ]))
        blocks.append((cf, nbytes, fcopy, wcopy, rscale, wscale, ratios, entries))

    cf0, nbytes0 = blocks[0][0], blocks[0][1]
    what = DESCRIPTIONS.get(workload, cf0["workload"])
    perms = [b[0]["workload"] for b in blocks]
    out.append("# HBM traffic per launch of every plan the tuning times: %s%s" % (
        what, "" if len(blocks) == 1 else " (%s)" % ", ".join(perms)))
    out.append("#")
    out.append("# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 counter runs of")
    out.append("# bench.py --candidates per workload, which runs every candidate bmmc_plan_tune_pairs")
    out.append("# would time (bmmc_plan_tune_candidates), each after one bmmc_copy of the same")
    out.append("# %d bytes; the JSON line each run prints is saved as candidates.json in its" % nbytes0)
    out.append("# output directory, and this file is written by bench_profiles.py from the two:")
    for c in commands:
        out.append("#   " + c)
    out.append("# A candidate's dispatches are those between two copies (the timed runs and the")
    out.append("# run its parity check makes).  Each counter is scaled by what it reads for the")
    out.append("# copy, known to read and write exactly the array's bytes:")
    for cf, nbytes, fcopy, wcopy, rscale, wscale, ratios, entries in blocks:
        out.append("#   %s: copy FETCH_SIZE = %.1f KiB -> read scale %.5f; copy WRITE_SIZE = "
                   "%.1f KiB -> write scale %.5f; %d candidates, measured / algorithmic bytes "
                   "from %.4f to %.4f" % (cf["workload"], fcopy, rscale, wcopy, wscale,
                                          len(ratios), min(ratios), max(ratios)))
    if compact:
        out.append("# Algorithmic bytes per launch = 2 x %d = %d.  Device code: %s."
                   % (nbytes0, 2 * nbytes0, cf0["kernel_source_digest"]))
    else:
        out.append("# Algorithmic bytes per launch = 2 x %d = %d.  kernel_source_digest names the"
                   % (nbytes0, 2 * nbytes0))
        out.append("# device code the counters were taken with, plan_options the plan and")
        out.append("# plan_tables_digest its kernel tables; bench.py reports the traffic of the entry")
        out.append("# that matches its own plan and tables, while the device code matches, and none")
        out.append("# otherwise.")
    for b in blocks:
        if len(blocks) > 1:
            out.append("")
            out.append("# ---- %s ----" % b[0]["workload"])
        if compact:
            out.append("")
            out.append("| candidate | kernel | t | skew | order | staging | loads | "
                       "measured / algorithmic |")
            out.append("|---|---|---|---|---|---|---|---|")
            out.extend(b[7])
            continue
        for e in b[7]:
            out.append("")
            out.append(e)
    return "\n".join(out) + "\n"


# ---- kernel trace --------------------------------------------------------

def trace_dispatches(d: str):
    """[(kernel name, grid work-items, duration ns)] in the order the
    dispatches started (graph replays get their dispatch ids out of that
    order)."""
    rows = []
    for path in find_csvs(d, "kernel_trace.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                grid = 1
                for ax in ("X", "Y", "Z"):
                    k = "Grid_Size_" + ax
                    if k in r and r[k]:
                        grid *= int(r[k])
                if "Grid_Size" in r and r["Grid_Size"]:
                    grid = int(r["Grid_Size"])
                start = int(pick(r, "Start_Timestamp"))
                rows.append((start, int(pick(r, "Dispatch_Id")), pick(r, "Kernel_Name"), grid,
                             int(pick(r, "End_Timestamp")) - start))
    rows.sort()
    return [(n, g, t) for _, _, n, g, t in rows]


def kernel_stats(d: str):
    out = []
    for path in find_csvs(d, "kernel_stats.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                out.append((pick(r, "Name", "KERNEL_NAME"), int(pick(r, "Calls")),
                            float(pick(r, "TotalDurationNs")), float(pick(r, "AverageNs")),
                            float(pick(r, "MinNs")), float(pick(r, "MaxNs"))))
    out.sort(key=lambda e: -e[2])
    return out


def headline_window(disp, steps: int, warmup: int, replays: int, copy_grid: int):
    """The headline's timed dispatches and the copy ceiling's.  bench.py runs,
    after the tuning: the warm-up steps, the graph's upload replay and the
    timed replays of the headline (one dispatch per step of a one-pass plan),
    then the same for bmmc_copy of the same bytes (copy_grid work-items of 16
    bytes).  The first run of at least upload + timed consecutive copies of
    that grid marks the end of the headline's dispatches; its last
    replays x steps copies are the copy's timed ones."""
    need = steps + replays * steps
    i = 0
    while i < len(disp):
        if not (is_copy(disp[i][0]) and disp[i][1] == copy_grid):
            i += 1
            continue
        j = i
        while j < len(disp) and is_copy(disp[j][0]) and disp[j][1] == copy_grid:
            j += 1
        if j - i >= need:
            before = [e for e in disp[:i] if is_library(e[0]) and not is_copy(e[0])]
            return before[-replays * steps:], disp[j - replays * steps:j]
        i = j
    raise SystemExit("bench_profiles.py: no run of %d copies of %d work-items in the trace"
                     % (need, copy_grid))


def trace_summary(d: str, commands) -> str:
    b = last_json_line(os.path.join(d, "bench.json"))
    steps, warmup = int(b["steps"]), int(b["warmup"])
    replays = int(b["replays"]["count"])
    disp = trace_dispatches(d)
    copy_grid = int(b["config"]["bytes_per_step"]) // 2 // 16
    timed, copies = headline_window(disp, steps, warmup, replays, copy_grid)
    names = sorted({n for n, _, _ in timed})
    if len(names) != 1:
        raise SystemExit("bench_profiles.py: the timed window holds %s" % names)
    algo = float(b["roofline"]["algorithmic_bytes_per_launch"])
    durs = [t for _, _, t in timed]
    avg = sum(durs) / len(durs)
    cavg = sum(t for _, _, t in copies) / len(copies)
    cfg = b["config"]
    opts = cfg["plan"]
    out = ["# Kernel trace of the default benchmark command", "",
           "Command (`<repo>` is the repository root; the JSON line is saved as bench.json "
           "in `<dir>`, and this file is written by `python3 <repo>/bench_profiles.py trace "
           "<dir>`):", ""]
    out += ["    " + c for c in commands]
    out += ["", "The traced run printed the headline line below (the tuning's pick varies "
            "between near-tied candidates from run to run):", "",
            "| field | value |", "|---|---|",
            "| workload | %s |" % cfg["workload"],
            "| plan | %s t=%s skew %s, %s threads, order %s%s%s |" % (
                opts["kernels"][-1], opts.get("tile_log2"), opts.get("tile_skew"),
                opts.get("tile_threads"), opts.get("block_map"),
                ", split staging" if opts.get("split_stage") else "",
                ", buffer loads" if opts.get("buffer_loads") else ""),
            "| value (median of %d timed graph replays) | %.2f GB/s |" % (replays, b["value"]),
            "| ms per step, median / min / max | %.6f / %.6f / %.6f |" % (
                b["ms_per_step"], b["replays"]["ms_per_step_min"],
                b["replays"]["ms_per_step_max"]),
            "| roofline.achieved (mean step time over the timed replays) | %.2f GB/s |"
            % b["roofline"]["achieved"],
            "| frac of copy / of 8 TB/s | %.4f / %.4f |" % (b["frac_of_copy"],
                                                          b["frac_of_hbm_peak"]), "",
            "**Timed window in the trace.** The %d dispatches of `%s` right before the copy "
            "ceiling's first graph replays (after the %d warm-up steps and the graph's upload "
            "replay of %d) are the %d timed replays.  They average **%.2f us** (min %.2f, max %.2f): "
            "%.2f GB/s of algorithmic bytes (%d per launch), against %.2f GB/s in the bench "
            "line (%.2f%% apart; the trace times the kernel alone, the bench the graph replay "
            "between two events).  The copy ceiling `%s` averages %.2f us over its %d timed "
            "dispatches (%.2f GB/s)." % (
                len(timed), short_name(names[0]), warmup, steps, replays, avg / 1e3, min(durs) / 1e3,
                max(durs) / 1e3, algo / avg, int(algo), b["roofline"]["achieved"],
                100.0 * abs(algo / avg - b["roofline"]["achieved"]) / b["roofline"]["achieved"],
                short_name(copies[0][0]), cavg / 1e3, len(copies), algo / cavg), "",
            "**Every kernel of the run** (tuning candidates of every configuration included; "
            "rocprofv3 --stats):", "",
            "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, _tot, avg_ns, mn, mx in kernel_stats(d):
        out.append("| `%s` | %d | %.2f | %.2f | %.2f |" % (short_name(name), calls, avg_ns / 1e3,
                                                         mn / 1e3, mx / 1e3))
    if "configs" in b:
        out += ["", "**Configurations of the same run** (its `configs` object; under the tracer "
                "each dispatch carries the profiler's own cost, which the arrays of a few MiB "
                "(c1) feel most: their kernels and their copy alike run several times slower "
                "than untraced, so their fractions here are not the bench line's):", "",
                "| configuration | plan | GB/s (median of 5) | frac of copy | frac of 8 TB/s "
                "| parity |", "|---|---|---|---|---|---|"]
        for key, e in b["configs"].items():
            if e.get("see") == "headline":
                continue
            if "gbs" in e:
                p = e["plan"]
                label = "%s t=%s skew %s threads %s order %s%s%s" % (
                    "+".join(p["kernels"]), p["tile_log2"], p["tile_skew"], p["tile_threads"],
                    p["block_map"], " split" if p.get("split_stage") else "",
                    " buffer loads" if p.get("buffer_loads") else "")
                out.append("| %s | %s | %.1f | %.4f | %.4f | %s |" % (
                    key, label, e["gbs"], e["frac_of_copy"], e["frac_of_hbm_peak"], e["parity"]))
            else:
                out.append("| %s (%d permutations) | per permutation | min %.1f / median %.1f / "
                           "max %.1f | %.4f / %.4f / %.4f | median %.4f | %s |" % (
                               key, e["perms"], e["min_gbs"], e["median_gbs"], e["max_gbs"],
                               e["min_frac_of_copy"], e["median_frac_of_copy"],
                               e["max_frac_of_copy"], e["median_frac_of_hbm_peak"],
                               e["parity"]))
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--command", action="append", default=[],
                   help="a command that produced the input (repeatable)")
    t.add_argument("--compact", action="store_true",
                   help="one table row per candidate instead of entries bench.py reads")
    t.add_argument("dirs", nargs="+", help="FETCH_DIR WRITE_DIR [...]")
    k = sub.add_parser("trace")
    k.add_argument("--command", action="append", default=[])
    k.add_argument("dir")
    a = ap.parse_args()
    if a.what == "traffic":
        if len(a.dirs) % 2:
            raise SystemExit("bench_profiles.py: directories come in FETCH/WRITE pairs")
        pairs = list(zip(a.dirs[0::2], a.dirs[1::2]))
        sys.stdout.write(traffic_summary(a.workload, pairs, a.command, a.compact))
    else:
        sys.stdout.write(trace_summary(a.dir, a.command))


if __name__ == "__main__":
    main()
