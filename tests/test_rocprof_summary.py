"""The profile assembly (rocprof_summary decode mode) on synthetic rocprofv3
CSV files with round numbers: durations, per-wave and per-element counts,
the copy-calibrated HBM bytes and the VALU issue fractions."""
import csv
import json
import os

from quantized_gated_delta_amd import rocprof_summary as R

KERNEL = ("void sqk::(anonymous namespace)::decode_kernel<128, false, false, false, false, "
          "unsigned short, unsigned short>(sqk::PoolView, sqk::HeadTable, sqk::StepIO)")


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counters(path, kernel, values, dispatches=(1, 2)):
    rows = [[d, kernel, name, v] for d in dispatches for name, v in values.items()]
    _write(path, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def test_decode_profile_figures(tmp_path):
    o = str(tmp_path / "prof")
    # three dispatches of 100, 200 and 300 us, and one launch of another kernel
    trace = [[KERNEL, 0, 100_000, 24576 * 256, 256, 48, 23552],
             [KERNEL, 0, 200_000, 24576 * 256, 256, 48, 23552],
             [KERNEL, 0, 300_000, 24576 * 256, 256, 48, 23552],
             ["other_kernel", 0, 5_000, 256, 256, 8, 0]]
    _write(os.path.join(o, "c3a_trace", "run_kernel_trace.csv"),
           ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X",
            "VGPR_Count", "LDS_Block_Size"], trace)
    waves = 98304
    _counters(os.path.join(o, "c3a_p1", "run_counter_collection.csv"), KERNEL, {
        "SQ_WAVES": waves, "SQ_INSTS_VALU": waves * 1000, "SQ_ACTIVE_INST_VALU": 1024 * 200,
        "SQ_ACTIVE_INST_VALU2": 1024 * 50, "SQ_BUSY_CYCLES": 1, "SQ_WAVE_CYCLES": waves * 3000,
        "SQ_INSTS_LDS": waves * 60, "SQ_INSTS_SALU": waves * 100})
    _counters(os.path.join(o, "c3a_p2", "run_counter_collection.csv"), KERNEL, {
        "GRBM_GUI_ACTIVE": 8 * 1000, "SQ_ACTIVE_INST_ANY": 1, "SQ_INSTS_VMEM_RD": 1,
        "SQ_INSTS_VMEM_WR": 1, "SQ_LDS_BANK_CONFLICT": 16, "SQ_WAIT_ANY": 1,
        "SQ_WAIT_INST_ANY": 1, "SQ_INSTS_MFMA": waves * 4})
    # counters of a dispatch are summed over rows (one row per XCD / SE)
    _write(os.path.join(o, "c3a_p3", "run_counter_collection.csv"),
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
           [[1, KERNEL, "FETCH_SIZE", 131072], [1, KERNEL, "FETCH_SIZE", 131072]])
    _counters(os.path.join(o, "c3a_p4", "run_counter_collection.csv"), KERNEL,
              {"WRITE_SIZE": 524288})
    # the copy calibration: a 1 GiB copy counts 524288 KiB fetched, 1048576 written
    _counters(os.path.join(o, "copy_FETCH_SIZE", "run_counter_collection.csv"),
              "elementwise_copy_kernel", {"FETCH_SIZE": 524288})
    _counters(os.path.join(o, "copy_WRITE_SIZE", "run_counter_collection.csv"),
              "elementwise_copy_kernel", {"WRITE_SIZE": 1048576})
    out = str(tmp_path / "out")
    os.makedirs(out)
    doc = R.decode_profiles(o, out, ["c3a"], {"c3a": 1 << 30}, 512, 48, 128, "src.hip",
                            "0123456789abcdef")
    json.dumps(doc)                                   # serialisable
    v = doc["variants"]["c3a"]
    assert v["trace"]["dispatches"] == 3
    assert v["trace"]["avg_us"] == 200.0 and v["trace"]["median_us"] == 200.0
    assert v["valu_insts_per_wave"] == 1000
    assert v["valu_insts_per_element"] == waves * 1000 * 64 / (512 * 48 * 128 * 128)
    assert abs(v["valu_issue_frac"] - 0.6) < 1e-12           # (200 - 50) x 4 / 1000
    assert abs(v["valu_issue_frac_at_4_cycles"] - 0.8) < 1e-12
    assert v["valu_dual_issue_share"] == 0.25
    assert v["mfma_insts_per_wave"] == 4 and v["lds_insts_per_wave"] == 60
    assert v["wave_cycles"] == 4 * 3000                      # SQ_WAVE_CYCLES counts quad-cycles
    assert v["fetch_bytes_per_launch"] == 1 << 29            # 262144 of 524288 KiB per GiB
    assert v["write_bytes_per_launch"] == 1 << 29
    assert v["bytes_per_launch"] == v["algorithmic_bytes_per_launch"] == 1 << 30
    md = open(os.path.join(out, "decode_gdn6_B512_H48_counters.md")).read()
    assert "| duration avg / median / min / max (us) | 200.0 / 200.0 / 100.0 / 300.0 |" in md
    assert "ratio 1.0000" in md and "0123456789abcdef" in md
    assert "rocprofv3 --kernel-trace" in md and "python3 bench.py --workload c3a" in md
