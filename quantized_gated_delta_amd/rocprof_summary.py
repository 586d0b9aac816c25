"""Summarize rocprofv3 CSV output for one kernel.

    python -m quantized_gated_delta_amd.rocprof_summary trace <dir> <kernel-substring>
    python -m quantized_gated_delta_amd.rocprof_summary pmc <dir> <kernel-substring> [<copy-dir>]
    python -m quantized_gated_delta_amd.rocprof_summary bygrid <dir> <kernel-substring>
    python -m quantized_gated_delta_amd.rocprof_summary decode <dir> <outdir> [variant ...]

trace: per-kernel dispatch count and average / median / min / max duration
       from ``*_kernel_trace.csv`` (rocprofv3 --kernel-trace --output-format csv).
bygrid: like trace, but one entry per (kernel, grid size), so one kernel
       launched on several workload shapes is summarised per shape.
pmc:   per-dispatch averages of every counter in ``*_counter_collection.csv``
       (rocprofv3 --pmc ... --output-format csv).  FETCH_SIZE and WRITE_SIZE
       are reported in KiB per dispatch; with a copy-run directory the same
       counters of the largest plain copy kernel there give the scale factor
       (counter KiB per byte actually moved) used to convert them to bytes.
decode: the counter profiles of the B = 512 x H = 48 decode variants
       (decode_commands lists the runs behind each), as markdown summaries and
       one JSON document under <outdir>.
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


# The B = 512 x H = 48 decode variants the counter profiles cover: bench.py
# arguments, the decode kernel's template prefix, and a description.
DECODE_VARIANTS = {
    "c3a": ("--workload c3a --no-variants --no-cpu", "decode_kernel<128, false, false, false, false",
            "GDN, 6-bit state on every head (the c3a workload)", "gdn6"),
    "c3b": ("--workload c3b --no-variants --no-cpu", "decode_kernel<128, false, false, false, false",
            "GDN, mixed 4/8-bit heads by gate half-life (the c3b workload)", "gdn48"),
    "kda_mixed": ("--only kda_mixed", "decode_kernel<128, true, false, false, false",
                  "KDA, 4/6/8-bit heads at 25/50/25 %", "kda468"),
    "kda_rows": ("--only kda_rows", "decode_kernel<128, true, false, false, true",
                 "KDA, 4/6/8-bit key rows at 25/50/25 % of every head", "kda468rows"),
    "kra": ("--only kra", "decode_kernel<128, false, false, true, false",
            "GDN 6-bit with the key-row-aware fit in the requantizer", "gdn6_kra"),
    "kda_rows_kra": ("--only kda_rows_kra", "decode_kernel<128, true, false, true, true",
                     "KDA, 4/6/8-bit key rows with the key-row-aware fit", "kda468rows_kra"),
    # the unquantized comparator (the same step on an fp32 state pool); its
    # launches include the warm-up's, which have the same shape
    "fp32_state": ("--only fp32_state", "f32_decode_kernel<128, false, unsigned short",
                   "fp32 state pool, the unquantized comparator (GDN)", "f32state"),
}
PMC_SETS = [
    "SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VALU2 SQ_BUSY_CYCLES SQ_WAVE_CYCLES "
    "SQ_INSTS_LDS SQ_INSTS_SALU",
    "GRBM_GUI_ACTIVE SQ_ACTIVE_INST_ANY SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_LDS_BANK_CONFLICT "
    "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_INSTS_MFMA",
    "FETCH_SIZE",
    "WRITE_SIZE",
]


def decode_commands(v: str) -> list:
    """The rocprofv3 runs behind one variant's profile ($O: output folder)."""
    args, pat, _, _ = DECODE_VARIANTS[v]
    pat = "namespace)::" + pat
    # the trace: the benchmark's own timing (0.3 s of untimed launches, then
    # the warm-up and timed steps), so that its average is the launch time
    # the benchmark reports
    out = ["rocprofv3 --kernel-trace --stats --output-format csv -d $O/%s_trace -o run -- \\\n"
           "    python3 bench.py %s" % (v, args)]
    for i, ctr in enumerate(PMC_SETS):
        out.append("rocprofv3 --pmc %s --output-format csv -d $O/%s_p%d -o run -- \\\n"
                   "    python3 bench.py %s --steps 10 --warmup 2 --prewarm 0" % (ctr, v, i + 1, args))
    return out


def _fmt(x) -> str:
    return "{:,}".format(int(round(x))).replace(",", " ")


def decode_profiles(o: str, outdir: str, variants: list, algo_bytes: dict, B: int, H: int,
                    d: int, src: str, src_hash: str) -> dict:
    """Assemble the counter profiles of decode variants from the rocprofv3 runs
    of decode_commands (folders <v>_trace, <v>_p1.._p4 under o) and the copy
    calibration (copy_FETCH_SIZE, copy_WRITE_SIZE: a 1 GiB copy, bench.py
    --copy-calib): writes decode_<tag>_B<B>_H<H>_counters.md per variant and
    returns the JSON document (every figure, with the kernel source hash)."""
    gib = float(1 << 30)
    cf = copy_scale(os.path.join(o, "copy_FETCH_SIZE"), "FETCH_SIZE", 1 << 30) * gib
    cw = copy_scale(os.path.join(o, "copy_WRITE_SIZE"), "WRITE_SIZE", 1 << 30) * gib
    doc = {"kernel_src": src, "kernel_src_sha256_16": src_hash, "shape": {"B": B, "H": H, "d": d},
           "copy_fetch_size_kib_per_GiB": cf, "copy_write_size_kib_per_GiB": cw, "variants": {}}
    elems = B * H * d * d
    for v in variants:
        args, pat, desc, tag = DECODE_VARIANTS[v]
        pat = "namespace)::" + pat
        tr = trace(os.path.join(o, v + "_trace"), pat)
        c = {}
        for i in range(len(PMC_SETS)):
            c.update(pmc(os.path.join(o, "%s_p%d" % (v, i + 1)), pat))
        waves = c["SQ_WAVES"]
        grbm = c["GRBM_GUI_ACTIVE"] / 8.0                # per XCD
        fetch = c["FETCH_SIZE"] / cf * gib
        write = c["WRITE_SIZE"] / cw * gib
        valu2 = c["SQ_ACTIVE_INST_VALU2"]
        r = {"workload": v, "description": desc, "kernel": tr["kernel"],
             "trace": {k: tr[k] for k in ("dispatches", "avg_us", "median_us", "min_us", "max_us",
                                          "vgpr", "lds")},
             "counters_per_dispatch": c,
             "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
             "bytes_per_launch": fetch + write, "algorithmic_bytes_per_launch": algo_bytes[v],
             "valu_insts_per_wave": c["SQ_INSTS_VALU"] / waves,
             "valu_insts_per_element": c["SQ_INSTS_VALU"] * 64 / elems,
             "valu_issue_frac": (c["SQ_ACTIVE_INST_VALU"] - valu2) * 4 / 1024 / grbm,
             "valu_issue_frac_at_4_cycles": c["SQ_ACTIVE_INST_VALU"] * 4 / 1024 / grbm,
             "valu_dual_issue_share": valu2 / c["SQ_ACTIVE_INST_VALU"],
             "mfma_insts_per_wave": c["SQ_INSTS_MFMA"] / waves,
             "lds_insts_per_wave": c["SQ_INSTS_LDS"] / waves,
             "salu_insts_per_wave": c["SQ_INSTS_SALU"] / waves,
             "wave_cycles": 4 * c["SQ_WAVE_CYCLES"] / waves}
        doc["variants"][v] = r
        cmds = "\n".join("    " + x.replace("\n", "\n    ") for x in decode_commands(v))
        rows = [
            ("dispatches traced", "%d" % tr["dispatches"]),
            ("duration avg / median / min / max (us)", "%.1f / %.1f / %.1f / %.1f" % (
                tr["avg_us"], tr["median_us"], tr["min_us"], tr["max_us"])),
            ("VGPRs / LDS bytes per workgroup", "%s / %s" % (tr["vgpr"], tr["lds"])),
            ("SQ_WAVES", _fmt(waves)),
            ("SQ_INSTS_VALU", "%s (%.0f per wave, %.2f per state element)" % (
                _fmt(c["SQ_INSTS_VALU"]), r["valu_insts_per_wave"], r["valu_insts_per_element"])),
            ("SQ_ACTIVE_INST_VALU / SQ_ACTIVE_INST_VALU2 (four-cycle slots per VALU instruction; "
             "VALU2: slots carrying a second VALU instruction)",
             "%s / %s (%.0f %% of VALU instructions issue paired)" % (
                 _fmt(c["SQ_ACTIVE_INST_VALU"]), _fmt(valu2),
                 100 * 2 * valu2 / c["SQ_INSTS_VALU"])),
            ("SQ_INSTS_MFMA / LDS / SALU per wave", "%.1f / %.1f / %.1f" % (
                r["mfma_insts_per_wave"], r["lds_insts_per_wave"], r["salu_insts_per_wave"])),
            ("SQ_INSTS_VMEM_RD / _WR", "%s / %s" % (_fmt(c["SQ_INSTS_VMEM_RD"]),
                                                  _fmt(c["SQ_INSTS_VMEM_WR"]))),
            ("SQ_LDS_BANK_CONFLICT", _fmt(c["SQ_LDS_BANK_CONFLICT"])),
            ("SQ_WAVE_CYCLES per wave (cycles)", _fmt(r["wave_cycles"])),
            ("SQ_ACTIVE_INST_ANY / SQ_WAIT_INST_ANY / SQ_WAIT_ANY", "%s / %s / %s" % (
                _fmt(c["SQ_ACTIVE_INST_ANY"]), _fmt(c["SQ_WAIT_INST_ANY"]),
                _fmt(c["SQ_WAIT_ANY"]))),
            ("GRBM_GUI_ACTIVE (sum over 8 XCDs)", _fmt(c["GRBM_GUI_ACTIVE"])),
            ("SIMD cycles issuing VALU ((SQ_ACTIVE_INST_VALU - SQ_ACTIVE_INST_VALU2) x 4 / 1024 "
             "SIMDs / (GRBM_GUI_ACTIVE / 8))", "%.3f (%.3f counting every instruction as a "
             "quad-cycle of its own)" % (r["valu_issue_frac"], r["valu_issue_frac_at_4_cycles"])),
            ("FETCH_SIZE / WRITE_SIZE (KiB per dispatch)", "%s / %s" % (
                _fmt(c["FETCH_SIZE"]), _fmt(c["WRITE_SIZE"]))),
            ("copy calibration, KiB counted per GiB copied (fetch / write)", "%s / %s" % (
                _fmt(cf), _fmt(cw))),
            ("HBM bytes per launch, scaled (fetch + write)", "%.1f + %.1f = %.1f MB" % (
                fetch / 1e6, write / 1e6, (fetch + write) / 1e6)),
            ("algorithmic bytes per launch", "%.1f MB (ratio %.4f)" % (
                algo_bytes[v] / 1e6, (fetch + write) / algo_bytes[v])),
        ]
        md = ["# Decode kernel counters: %s, B = %d x H = %d, d = %d (MI355X)" % (desc, B, H, d), "",
              "Kernel: `%s` (source `%s`, sha256 prefix %s)." % (tr["kernel"][:100], src, src_hash),
              "",
              "Commands (repository root on the GPU box, `cd /tmp && export TMPDIR=/tmp` first; "
              "one counter set per run; `$O` is an output folder):", "", cmds,
              "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d $O/copy_FETCH_SIZE -o run -- "
              "python3 bench.py --copy-calib",
              "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d $O/copy_WRITE_SIZE -o run -- "
              "python3 bench.py --copy-calib",
              "    python3 -m quantized_gated_delta_amd.rocprof_summary decode $O profiles %s" % v,
              "", "| figure | value |", "|---|---|"]
        md += ["| %s | %s |" % kv for kv in rows]
        md += ["", "`decode_B%d_H%d_counters.json` holds every figure above with the kernel source "
               "hash; `bench.py` takes the traffic and the VALU issue fraction from it only while "
               "that hash matches the source it runs." % (B, H), ""]
        with open(os.path.join(outdir, "decode_%s_B%d_H%d_counters.md" % (tag, B, H)), "w") as f:
            f.write("\n".join(md))
    return doc


def decode_main(o: str, outdir: str, variants: list) -> None:
    """decode mode: profiles of the given variants (all when none), merged into
    <outdir>/decode_B512_H48_counters.json."""
    import hashlib
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    import workload as W
    src = "quantized_gated_delta_amd/csrc/sq_kernels.hip"
    with open(os.path.join(root, src), "rb") as f:
        h = hashlib.sha256(f.read()).hexdigest()[:16]
    B, H, d = 512, 48, 128
    c3a = W.make("c3a").layers[0]
    c3b = W.make("c3b").layers[0]
    kda = W.mixed_bits(0, 0, H)
    algo = {"c3a": bench.algo_bytes_per_step(B, H, d, c3a.head_bits, "gdn"),
            "c3b": bench.algo_bytes_per_step(B, H, d, c3b.head_bits, "gdn"),
            "kda_mixed": bench.algo_bytes_per_step(B, H, d, kda, "kda"),
            "kda_rows": bench.algo_bytes_per_step(B, H, d, [6] * H, "kda")}
    algo["fp32_state"] = bench.f32_bytes_per_step(B, H, d, "gdn")
    algo["kra"] = algo["c3a"]
    algo["kda_rows_kra"] = algo["kda_rows"]
    variants = variants or list(DECODE_VARIANTS)
    doc = decode_profiles(o, outdir, variants, algo, B, H, d, src, h)
    path = os.path.join(outdir, "decode_B%d_H%d_counters.json" % (B, H))
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f)
        if old.get("kernel_src_sha256_16") == h:     # same kernel: keep the other variants
            old["variants"].update(doc["variants"])
            doc["variants"] = old["variants"]
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


def main(argv):
    if argv[1] == "decode":
        decode_main(argv[2], argv[3], argv[4:])
        return
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
