"""rocprofv3 harness: parse kernel traces and counter passes into summaries.

The benchmark's roofline line needs three measurements of the same command:

  rocprofv3 --kernel-trace --stats -f csv -d <trace_dir> -o run -- python3 bench.py ...
  rocprofv3 --pmc FETCH_SIZE     -f csv -d <fetch_dir> -o run -- python3 bench.py ... --copy-calibration
  rocprofv3 --pmc WRITE_SIZE     -f csv -d <write_dir> -o run -- python3 bench.py ... --copy-calibration

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  The counter
passes also run one plain 1 GiB device-to-device copy; the ratio between its
known byte count and what each counter reads for it is the scale applied to
the GEMV's counts (on the MI355X measured here FETCH_SIZE reads half of the
copy's 1 GiB and WRITE_SIZE all of it).

    python -m compressed_gemv_amd.profiling --trace D1 --fetch D2 --write D3 \\
        --kernel gemv_b1_kernel=132120576+25:20 --sha <source sha> --out summary.md

The trace table splits every kernel by launch grid, so one kernel run at
several shapes (prefill at several token counts) gives one row per shape,
with mean, median, 10th and 90th percentile durations.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics

COPY_BYTES = 1 << 30


def _csv(path_glob):
    files = sorted(glob.glob(path_glob, recursive=True))
    if not files:
        raise FileNotFoundError(path_glob)
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    """Kernel name without its parameter list (template arguments kept)."""
    name = name.replace("(anonymous namespace)::", "")
    depth = 0
    for i, c in enumerate(name):
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == "(" and depth == 0:
            return name[:i]
    return name


def _grid(r):
    """Total work-items of the launch (traces give x, y, z; counter files the product)."""
    if "Grid_Size_X" in r:
        return str(int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
    return str(r.get("Grid_Size", "?"))


def _pct(sorted_vals, q):
    """Nearest-rank percentile of an ascending list."""
    k = max(0, min(len(sorted_vals) - 1, int(round(q * (len(sorted_vals) - 1)))))
    return sorted_vals[k]


def dist(vals):
    v = sorted(vals)
    return {"n": len(v), "mean": statistics.mean(v), "median": statistics.median(v),
            "p10": _pct(v, 0.10), "p90": _pct(v, 0.90), "min": v[0], "max": v[-1]}


def kernel_stats(trace_dir):
    """[(name, calls, avg_us, min_us, pct)] from *_kernel_stats.csv."""
    out = []
    for r in _csv(os.path.join(trace_dir, "**", "*kernel_stats.csv")):
        out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["Percentage"])))
    return out


def dispatch_groups(trace_dir):
    """{(short name, grid): [durations in us, in dispatch order]} from *_kernel_trace.csv,
    so one kernel launched at several shapes (prefill at several M) splits into rows."""
    rows = _csv(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = {}
    for r in rows:
        key = (_short(r["Kernel_Name"]), _grid(r))
        out.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def kernel_durations(trace_dir, match, grid=None):
    """Per-dispatch durations (us), in dispatch order, of kernels whose name
    contains `match` (and whose grid is `grid`, if given)."""
    rows = _csv(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
            if match in r["Kernel_Name"] and (grid is None or _grid(r) == grid)]


def counter_per_dispatch(counter_dir, match, grid=None):
    rows = _csv(os.path.join(counter_dir, "**", "*counter_collection.csv"))
    rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
    return [float(r["Counter_Value"]) for r in rows
            if match in r["Kernel_Name"] and (grid is None or _grid(r) == grid)]


def copy_scale(counter_dir):
    """Bytes per counter KiB, from the 1 GiB calibration copy (largest copy dispatch)."""
    vals = counter_per_dispatch(counter_dir, "copyBuffer")
    kib = max(vals)
    return COPY_BYTES / (kib * 1024.0), kib


def _window(vals, skip, take):
    vals = vals[skip:]
    return vals[:take] if take else vals


def summarize(trace_dir, fetch_dir, write_dir, kernel, alg_bytes, skip=0, take=0, grid=None):
    """Duration distribution of dispatches [skip, skip + take) of `kernel`
    (all after `skip` when take is 0), and its HBM traffic from the counter
    passes scaled by the calibration copy."""
    durs = _window(kernel_durations(trace_dir, kernel, grid), skip, take)
    d = dist(durs)
    out = {"duration_us": d, "alg_bytes": alg_bytes,
           "achieved_gbs": alg_bytes / (d["mean"] * 1e-6) / 1e9,
           "achieved_gbs_median": alg_bytes / (d["median"] * 1e-6) / 1e9}
    if fetch_dir and write_dir:
        fscale, fcopy = copy_scale(fetch_dir)
        wscale, wcopy = copy_scale(write_dir)
        fk = statistics.median(_window(counter_per_dispatch(fetch_dir, kernel, grid), skip, take))
        wk = statistics.median(_window(counter_per_dispatch(write_dir, kernel, grid), skip, take))
        out.update({"fetch_kib": fk, "write_kib": wk, "fetch_scale": fscale, "write_scale": wscale,
                    "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
                    "traffic_bytes": fk * 1024 * fscale + wk * 1024 * wscale})
    return out


def counter_table(counter_dirs, kernel, grid=None, skip=0, take=0):
    """{counter: median per dispatch} over dispatches [skip, skip + take) of
    `kernel` (all after `skip` when take is 0), from one or more counter runs."""
    out = {}
    for d in counter_dirs:
        rows = _csv(os.path.join(d, "**", "*counter_collection.csv"))
        rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        by = {}
        for r in rows:
            if kernel in r["Kernel_Name"] and (grid is None or _grid(r) == grid):
                by.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for name, vals in by.items():
            out[name] = statistics.median(_window(vals, skip, take))
    return out


def _kernel_spec(spec):
    """NAME=BYTES[@GRID][+SKIP][:TAKE] -> (name, bytes, grid, skip, take)."""
    name, rest = spec.rsplit("=", 1)
    take = 0
    if ":" in rest:
        rest, t = rest.split(":")
        take = int(t)
    skip = 0
    if "+" in rest:
        rest, sk = rest.split("+")
        skip = int(sk)
    grid = None
    if "@" in rest:
        rest, grid = rest.split("@")
    return name, float(rest), grid, skip, take


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--kernel", action="append", default=[],
                    help="NAME=BYTES[@GRID][+SKIP][:TAKE]: substring of the kernel name, algorithmic bytes per "
                         "dispatch, optional grid (total work-items, e.g. 262144), dispatches skipped and taken (the timed region)")
    ap.add_argument("--counters", action="append", default=[],
                    help="rocprofv3 --pmc output directory with other counters (median per dispatch is reported)")
    ap.add_argument("--sha", default="")
    ap.add_argument("--title", default="")
    ap.add_argument("--commands", default="", help="text block with the rocprofv3 commands")
    ap.add_argument("--note", action="append", default=[], help="extra bullet lines for the summary")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    lines = [f"# {a.title}", ""]
    if a.commands:
        lines += ["Commands (from the repository root, TMPDIR=/tmp):", "", "```", a.commands.strip(), "```", ""]
    lines += ["## Kernel stats (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | % time |", "|---|---|---|---|---|"]
    for name, calls, avg, mn, pct in kernel_stats(a.trace)[:40]:
        lines.append(f"| `{_short(name)[:120]}` | {calls} | {avg:.2f} | {mn:.2f} | {pct:.2f} |")
    lines += ["", "## Dispatches by kernel and grid (us)", "",
              "| kernel | grid | calls | mean | median | p10 | p90 | min |", "|---|---|---|---|---|---|---|---|"]
    for (name, grid), durs in dispatch_groups(a.trace).items():
        d = dist(durs)
        lines.append(f"| `{name[:110]}` | {grid} | {d['n']} | {d['mean']:.2f} | {d['median']:.2f} | "
                     f"{d['p10']:.2f} | {d['p90']:.2f} | {d['min']:.2f} |")
    for spec in a.kernel:
        name, nbytes, grid, skip, take = _kernel_spec(spec)
        s = summarize(a.trace, a.fetch, a.write, name, nbytes, skip, take, grid)
        d = s["duration_us"]
        sel = f"dispatches {skip}..{skip + d['n'] - 1} in order" + (f", grid {grid}" if grid else "")
        lines += ["", f"## {name}: duration and HBM traffic", "",
                  f"- {sel}: {d['n']} dispatches",
                  f"- duration us: mean {d['mean']:.3f}, median {d['median']:.3f}, p10 {d['p10']:.3f}, "
                  f"p90 {d['p90']:.3f}, min {d['min']:.3f}, max {d['max']:.3f}",
                  f"- algorithmic bytes per launch: {int(nbytes)}",
                  f"- achieved (algorithmic bytes / mean duration): {s['achieved_gbs']:.1f} GB/s "
                  f"(median: {s['achieved_gbs_median']:.1f} GB/s)"]
        if a.counters:
            ct = counter_table(a.counters, name, grid, skip, take)
            lines += [f"- {k} (median per dispatch): {v:.6g}" for k, v in sorted(ct.items())]
        if "traffic_bytes" in s:
            lines += [f"- FETCH_SIZE median per dispatch: {s['fetch_kib']:.1f} KiB; 1 GiB copy reads "
                      f"{s['copy_fetch_kib']:.1f} KiB -> scale {s['fetch_scale']:.5f} bytes/KiB-unit",
                      f"- WRITE_SIZE median per dispatch: {s['write_kib']:.1f} KiB; 1 GiB copy writes "
                      f"{s['copy_write_kib']:.1f} KiB -> scale {s['write_scale']:.5f}",
                      f"- traffic_bytes_per_launch: {s['traffic_bytes']:.0f}",
                      f"- traffic / algorithmic bytes: {s['traffic_bytes'] / nbytes:.4f}"]
    if a.sha:
        lines.append(f"- kernel_source_sha: {a.sha}")
    if a.note:
        lines += ["", "## Notes", ""] + [f"- {n}" for n in a.note]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
