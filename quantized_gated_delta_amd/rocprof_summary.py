"""Summarize rocprofv3 CSV output for one kernel.

    python -m quantized_gated_delta_amd.rocprof_summary trace <dir> <kernel-substring>
    python -m quantized_gated_delta_amd.rocprof_summary pmc <dir> <kernel-substring> [<copy-dir>]
    python -m quantized_gated_delta_amd.rocprof_summary bygrid <dir> <kernel-substring>

trace: per-kernel dispatch count and average / median / min / max duration
       from ``*_kernel_trace.csv`` (rocprofv3 --kernel-trace --output-format csv).
bygrid: like trace, but one entry per (kernel, grid size), so one kernel
       launched on several workload shapes is summarised per shape.
pmc:   per-dispatch averages of every counter in ``*_counter_collection.csv``
       (rocprofv3 --pmc ... --output-format csv).  FETCH_SIZE and WRITE_SIZE
       are reported in KiB per dispatch; with a copy-run directory the same
       counters of the largest plain copy kernel there give the scale factor
       (counter KiB per byte actually moved) used to convert them to bytes.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys


def _rows(d: str, suffix: str):
    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, d))
    out = []
    for f in files:
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def trace(d: str, pattern: str) -> dict:
    rows = [r for r in _rows(d, "kernel_trace.csv") if pattern in r["Kernel_Name"]]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    if not durs:
        raise SystemExit("no dispatch of %r" % pattern)
    return {"kernel": rows[0]["Kernel_Name"], "dispatches": len(durs),
            "avg_us": statistics.mean(durs), "median_us": statistics.median(durs),
            "min_us": min(durs), "max_us": max(durs),
            "grid": rows[0].get("Grid_Size_X"), "workgroup": rows[0].get("Workgroup_Size_X"),
            "vgpr": rows[0].get("VGPR_Count"), "lds": rows[0].get("LDS_Block_Size")}


def bygrid(d: str, pattern: str) -> list:
    groups = {}
    for r in _rows(d, "kernel_trace.csv"):
        if pattern not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = []
    for (name, grid, wg), durs in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append({"kernel": name, "workgroups": grid // max(1, wg), "dispatches": len(durs),
                    "avg_us": statistics.mean(durs), "median_us": statistics.median(durs),
                    "min_us": min(durs), "max_us": max(durs)})
    return out


def pmc(d: str, pattern: str) -> dict:
    per = {}
    for r in _rows(d, "counter_collection.csv"):
        if pattern not in r["Kernel_Name"]:
            continue
        key = r["Counter_Name"]
        per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
        per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: statistics.mean(v.values()) for k, v in per.items()}


def copy_scale(d: str, counter: str, copy_bytes: int) -> float:
    """Counter value per byte moved for the plain copy kernel of a calibration
    run (average over its dispatches of kernels whose name contains 'copy')."""
    vals = [float(r["Counter_Value"]) for r in _rows(d, "counter_collection.csv")
            if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()]
    return statistics.mean(vals) / copy_bytes if vals else 0.0


def main(argv):
    mode, d, pattern = argv[1], argv[2], argv[3]
    if mode == "trace":
        print(json.dumps(trace(d, pattern), indent=1))
    elif mode == "bygrid":
        print(json.dumps(bygrid(d, pattern), indent=1))
    elif mode == "pmc":
        print(json.dumps(pmc(d, pattern), indent=1))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
