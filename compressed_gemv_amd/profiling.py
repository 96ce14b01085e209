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
        --kernel gemv_b1_kernel --bytes 132120576 --sha <source sha> --out summary.md
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


def kernel_stats(trace_dir):
    """[(name, calls, avg_us, min_us, pct)] from *_kernel_stats.csv."""
    out = []
    for r in _csv(os.path.join(trace_dir, "**", "*kernel_stats.csv")):
        out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["Percentage"])))
    return out


def kernel_durations(trace_dir, match):
    """Per-dispatch durations (us) of kernels whose name contains `match`."""
    rows = _csv(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows if match in r["Kernel_Name"]]


def counter_per_dispatch(counter_dir, match):
    rows = _csv(os.path.join(counter_dir, "**", "*counter_collection.csv"))
    return [float(r["Counter_Value"]) for r in rows if match in r["Kernel_Name"]]


def copy_scale(counter_dir):
    """Bytes per counter KiB, from the 1 GiB calibration copy (largest copy dispatch)."""
    vals = counter_per_dispatch(counter_dir, "copyBuffer")
    kib = max(vals)
    return COPY_BYTES / (kib * 1024.0), kib


def summarize(trace_dir, fetch_dir, write_dir, kernel, alg_bytes, last=None):
    durs = kernel_durations(trace_dir, kernel)
    if last:
        durs = durs[-last:]
    avg_us = statistics.mean(durs)
    fscale, fcopy = copy_scale(fetch_dir)
    wscale, wcopy = copy_scale(write_dir)
    fk = statistics.median(counter_per_dispatch(fetch_dir, kernel))
    wk = statistics.median(counter_per_dispatch(write_dir, kernel))
    traffic = fk * 1024 * fscale + wk * 1024 * wscale
    return {
        "avg_us": avg_us, "n": len(durs), "min_us": min(durs), "max_us": max(durs),
        "fetch_kib": fk, "write_kib": wk, "fetch_scale": fscale, "write_scale": wscale,
        "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
        "traffic_bytes": traffic, "alg_bytes": alg_bytes,
        "achieved_gbs": alg_bytes / (avg_us * 1e-6) / 1e9,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--bytes", type=float, required=True)
    ap.add_argument("--last", type=int, default=0, help="average only the last N dispatches (timed region)")
    ap.add_argument("--sha", default="")
    ap.add_argument("--title", default="")
    ap.add_argument("--commands", default="", help="text block with the rocprofv3 commands")
    ap.add_argument("--note", action="append", default=[], help="extra bullet lines for the summary")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    lines = [f"# {a.title or a.kernel}", ""]
    if a.commands:
        lines += ["Commands (run from /tmp with TMPDIR=/tmp):", "", "```", a.commands.strip(), "```", ""]
    lines += ["## Kernel stats (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | % time |", "|---|---|---|---|---|"]
    for name, calls, avg, mn, pct in kernel_stats(a.trace)[:40]:
        lines.append(f"| `{name[:110]}` | {calls} | {avg:.2f} | {mn:.2f} | {pct:.2f} |")
    if a.fetch and a.write:
        s = summarize(a.trace, a.fetch, a.write, a.kernel, a.bytes, a.last or None)
        lines += ["", f"## {a.kernel}: duration and HBM traffic", "",
                  f"- dispatches averaged: {s['n']} (min {s['min_us']:.2f} us, max {s['max_us']:.2f} us)",
                  f"- average duration: {s['avg_us']:.3f} us",
                  f"- algorithmic bytes per launch: {int(s['alg_bytes'])}",
                  f"- achieved (algorithmic bytes / average duration): {s['achieved_gbs']:.1f} GB/s",
                  f"- FETCH_SIZE median per dispatch: {s['fetch_kib']:.1f} KiB; 1 GiB copy reads "
                  f"{s['copy_fetch_kib']:.1f} KiB -> scale {s['fetch_scale']:.5f} bytes/KiB-unit",
                  f"- WRITE_SIZE median per dispatch: {s['write_kib']:.1f} KiB; 1 GiB copy writes "
                  f"{s['copy_write_kib']:.1f} KiB -> scale {s['write_scale']:.5f}",
                  f"- traffic_bytes_per_launch: {s['traffic_bytes']:.0f}",
                  f"- traffic / algorithmic bytes: {s['traffic_bytes'] / s['alg_bytes']:.4f}"]
        if a.sha:
            lines.append(f"- kernel_source_sha: {a.sha}")
    if a.note:
        lines += ["", "## Notes", ""] + [f"- {n}" for n in a.note]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
