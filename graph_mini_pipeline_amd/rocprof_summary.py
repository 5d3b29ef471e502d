"""Short text summaries of rocprofv3 output for the profiles/ folder, and the reader that turns a
counter summary into per-launch memory traffic.

    python -m graph_mini_pipeline_amd.rocprof_summary trace OUT.txt KERNEL_TRACE.csv "COMMAND"
    python -m graph_mini_pipeline_amd.rocprof_summary counters OUT.txt WORKLOAD FETCH.csv WRITE.csv "COMMAND"
    python -m graph_mini_pipeline_amd.rocprof_summary metrics OUT.txt COUNTERS.csv "COMMAND"

A metrics summary averages every counter or derived metric of a --pmc run per kernel (for
instance VALUBusy and MfmaUtil, the percentages of the active cycles in which the vector ALUs or
the matrix cores issue).

Counter summaries hold one machine-readable line per kernel:
    counters <kernel> dispatches=<n> fetch_kib=<avg> write_kib=<avg> source=<file> sha256=<hash>
(mean-aggregation kernels as <kernel>@outer for the outermost block, which follows the gather,
and <kernel>@inner for the others; a gather that follows a mean, copying a super-batch's shared
outermost means to its sub-batches, as <kernel>@copy) and one for the calibration copy
(k_copy_probe, a plain copy of known size):
    calibration copy_bytes=<B> fetch_kib=<avg> write_kib=<avg>
FETCH_SIZE and WRITE_SIZE are scaled by (copy bytes) / (counter reading of the copy) each.
"""
from __future__ import annotations

import csv
import hashlib
import os
import sys
from collections import defaultdict
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))

# Kernel name prefix -> the source file that defines it (its hash dates the counters).
KERNEL_SOURCES = {
    "k_gather": "csrc/gather.hip",
    "k_mean_v5": "csrc/aggregate.hip",
    "k_mean_v1": "csrc/aggregate.hip",
    "k_sample": "csrc/sample.hip",
    "k_classify": "csrc/sample.hip",
    "k_mark": "csrc/relabel.hip",
    "k_emit": "csrc/relabel.hip",
    "k_rank": "csrc/relabel.hip",
    "k_popc": "csrc/relabel.hip",
    "k_dist": "csrc/superbatch.hip",
    "k_seed_concat": "csrc/superbatch.hip",
    "k_relabel_sort": "csrc/relabel.hip",
    "k_match": "csrc/match.hip",
    "k_overlap": "csrc/match.hip",
    "k_dyn": "csrc/dyncache.hip",
    "k_copy_probe": "csrc/probe.hip",
    "k_hash_probe": "csrc/probe.hip",
    "k_fill": "csrc/relabel.hip",
    "k_sage_update": "csrc/sage.hip",
}


def short_name(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "")
    n = n.split("(")[0].replace("void ", "").replace("gnnmb::", "").strip()
    return n


def source_of(kernel: str) -> Optional[str]:
    kernel = kernel.split("@")[0]
    for pre, src in KERNEL_SOURCES.items():
        if kernel.startswith(pre):
            return src
    return None


def source_hash(rel: str) -> str:
    with open(os.path.join(HERE, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _role(name: str, prev: str) -> str:
    """A dispatch's name with its role on the stream (prev: the previous dispatch's name with its
    role): a mean right after a gather is the outermost block (@outer), other means are inner
    blocks (@inner); a batched gather right after an outermost mean copies the shared outermost
    means of a super-batch out to its sub-batches (@copy; per-sub-batch gathers, k_gather_rows,
    alternate with outermost means and are never copies)."""
    if name.startswith("k_mean"):
        outer = prev.startswith("k_gather") and not prev.endswith("@copy")
        return name + ("@outer" if outer else "@inner")
    if name.startswith("k_gather_batch") and prev.startswith("k_mean") and prev.endswith("@outer"):
        return name + "@copy"
    return name


def trace_summary(trace_csv: str, command: str) -> str:
    """Per-kernel duration statistics of the library's dispatches on the stream of its first
    dispatch (the stream the benchmark's headline and per-kernel timings run on; dispatches on
    other streams, such as a pipelined region's, overlap one another and are left out)."""
    rows = [r for r in csv.DictReader(open(trace_csv)) if "gnnmb" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    stream = rows[0]["Stream_Id"] if rows else None
    per = defaultdict(list)
    others = 0
    prev = ""
    for r in rows:
        if r["Stream_Id"] != stream:
            others += 1
            continue
        key = _role(short_name(r["Kernel_Name"]), prev)
        per[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        prev = key
    out = [f"# rocprofv3 --kernel-trace summary (library kernels on stream {stream}, the stream of "
           f"the first library dispatch; {others} dispatches on other streams left out)",
           f"# command: {command}",
           f"# {'kernel':44s} {'calls':>7s} {'total_ms':>10s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{name:46s} {len(d):7d} {sum(d) / 1e6:10.3f} {sum(d) / len(d) / 1e3:9.2f} "
                   f"{min(d) / 1e3:9.2f} {max(d) / 1e3:9.2f}")
    return "\n".join(out) + "\n"


def _per_kernel(path: str, counter: str) -> Dict[str, list]:
    """Counter values per (kernel, grid size).  A mean-aggregation dispatch that directly follows a
    gather dispatch (the outermost block, reading the rows just gathered) is named <kernel>@outer,
    the other mean dispatches <kernel>@inner, so that the two block kinds are not averaged together."""
    rows = [r for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and "gnnmb" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    d = defaultdict(list)
    prev = ""
    for r in rows:
        key = _role(short_name(r["Kernel_Name"]), prev)
        d[(key, int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        prev = key
    return d


def counter_summary(workload: str, fetch_csv: str, write_csv: str, command: str) -> str:
    f = _per_kernel(fetch_csv, "FETCH_SIZE")
    w = _per_kernel(write_csv, "WRITE_SIZE")
    out = [f"# rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (two runs), workload: {workload}",
           f"# command: {command}",
           "# KiB per dispatch, averaged over dispatches of the same kernel and grid size;",
           "# scale each by the calibration copy (bytes / its reading) for bytes moved to/from memory."]
    by_kernel = defaultdict(lambda: [0, 0.0, 0.0])
    probe = None
    for key in sorted(f):
        name, grid = key
        fv, wv = f[key], w.get(key, [0.0])
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        out.append(f"#   {name:40s} grid {grid:9d} n {len(fv):5d} fetch_kib {fa:12.1f} write_kib {wa:12.1f}")
        if name == "k_copy_probe":
            probe = (fa, wa)
        agg = by_kernel[name]
        agg[0] += len(fv)
        agg[1] += sum(fv)
        agg[2] += sum(wv) * len(fv) / len(wv)
    for name, (n, fs, ws) in sorted(by_kernel.items()):
        src = source_of(name)
        h = source_hash(src) if src else "-"
        out.append(f"counters {name.replace(' ', '')} dispatches={n} fetch_kib={fs / n:.1f} "
                   f"write_kib={ws / n:.1f} source={src} sha256={h}")
    if probe:
        out.append(f"calibration copy_bytes={1 << 30} fetch_kib={probe[0]:.1f} write_kib={probe[1]:.1f}")
    return "\n".join(out) + "\n"


def metrics_summary(counters_csv: str, command: str) -> str:
    rows = [r for r in csv.DictReader(open(counters_csv)) if "gnnmb" in r["Kernel_Name"]]
    names = sorted({r["Counter_Name"] for r in rows})
    per = defaultdict(lambda: defaultdict(list))
    for r in rows:
        per[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = ["# rocprofv3 --pmc " + " ".join(names) + ": per-kernel averages over its dispatches",
           f"# command: {command}",
           "# kernel".ljust(40) + " dispatches " + " ".join(f"{n:>16s}" for n in names) + "  source"]
    for k in sorted(per):
        vals = per[k]
        n = max(len(v) for v in vals.values())
        src = source_of(k)
        tag = f"{src} sha256={source_hash(src)}" if src else "-"
        out.append(f"{k[:40]:40s} {n:10d} " +
                   " ".join(f"{sum(vals[c]) / len(vals[c]):16.3f}" if vals.get(c) else f"{'-':>16s}"
                            for c in names) + f"  {tag}")
    return "\n".join(out) + "\n"


def read_traffic(path: str, kernel: str, grid_free: bool = True) -> Optional[dict]:
    """Calibrated bytes per dispatch of `kernel` from a counter summary, or None when the file is
    missing, lacks the kernel or the calibration, or the kernel's source changed since."""
    if not os.path.exists(path):
        return None
    rec, cal = None, None
    for line in open(path):
        parts = line.split()
        if not parts:
            continue
        if parts[0] == "counters" and parts[1] == kernel.replace(" ", ""):
            rec = dict(p.split("=", 1) for p in parts[2:])
        elif parts[0] == "calibration":
            cal = dict(p.split("=", 1) for p in parts[1:])
    if rec is None or cal is None:
        return None
    src = rec.get("source")
    if not src or src == "None" or source_hash(src) != rec.get("sha256"):
        return None
    fscale = float(cal["copy_bytes"]) / (float(cal["fetch_kib"]) * 1024.0)
    wscale = float(cal["copy_bytes"]) / (float(cal["write_kib"]) * 1024.0)
    fetch = float(rec["fetch_kib"]) * 1024.0 * fscale
    write = float(rec["write_kib"]) * 1024.0 * wscale
    return {"bytes": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
            "fetch_scale": fscale, "write_scale": wscale}


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "trace":
        out, trace, cmd = sys.argv[2:5]
        text = trace_summary(trace, cmd)
    elif mode == "counters":
        out, workload, fcsv, wcsv, cmd = sys.argv[2:7]
        text = counter_summary(workload, fcsv, wcsv, cmd)
    elif mode == "metrics":
        out, ccsv, cmd = sys.argv[2:5]
        text = metrics_summary(ccsv, cmd)
    else:
        raise SystemExit(__doc__)
    with open(out, "w") as fh:
        fh.write(text)
    print(text)
