"""Benchmark of the fused quantized gated Delta-rule decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3a]

A step is one sq_decode_step over the whole batch (dequantize, gate, look-up,
delta write, read-out, requantize in place) for B = 512 requests x 48 heads,
d = 128, 6-bit codes with fp32 row / column scales, bf16 inputs, requests
reached through a seeded permutation of 640 pool slots.  Inputs and the pool
are resident in HBM before timing starts.

Prints ONE JSON line: state-updates/s (request x head x step), the roofline
of the decode kernel (algorithmic bytes / average launch time against the
8 TB/s HBM3E peak), the same step on an fp32 state pool, the mixed 4/8-bit
variant, and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Per state element, the vector operations the fused step cannot avoid once
# the look-up and read-out sums run on the matrix cores, by opcode class:
# extract the code (bit-field extract; at 6 bits 1/16 more for fields that
# straddle words, at 8 bits a shift for half of the bytes), widen it (byte to
# fp32), three products ((a r_i) c_j, k_i u_j and s = S' / c'), two FMAs (the
# update and the rounding), one max3 (half for the column and half for the
# row maxima, two new values each) and the pack (funnel shift; 1/16 more at
# 6 bits).
def essential_mix(bits):
    ext = {4: 1.0, 6: 1.0625, 8: 0.5}.get(bits, 1.0)
    pack = {6: 1.0625}.get(bits, 1.0)
    return {"bfe": ext, "cvt": 1.0, "mul": 3.0, "fma": 2.0, "max3": 1.0, "alignbit": pack}


# Vector-ALU peak from the chip's unit counts: 256 CUs x 4 SIMDs x 64 lanes at
# 2.4 GHz, each SIMD issuing two wave64 instructions (from two waves) per four
# cycles, at most one of them from the single-issue classes (conversions,
# shifts, bit-field extract, funnel shift, max / max3, FP64): 78.6 T lane-ops/s
# for pairable instructions (the published 157.3 TFLOP/s fp32 at 2 flops per
# FMA), 39.3 T for single-issue ones.  A mix with n_single single-issue
# operations of n per element runs at most at
# n / max(n_single / 39.3 T, n / 78.6 T).
VALU_PAIR_PEAK = 256 * 4 * 64 * 2.4e9 / 2 / 1e12
VALU_SINGLE_PEAK = VALU_PAIR_PEAK / 2
SINGLE_ISSUE = ("bfe", "cvt", "max3", "alignbit")


def valu_peak(mix):
    n = sum(mix.values())
    n_single = sum(v for k, v in mix.items() if k in SINGLE_ISSUE)
    return n / max(n_single / VALU_SINGLE_PEAK, n / VALU_PAIR_PEAK)


COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_B512_H48_counters.json")
KERNEL_SRC = os.path.join(ROOT, "quantized_gated_delta_amd", "csrc", "sq_kernels.hip")


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def algo_bytes_per_step(B, H, d, head_bits, gate, io_bytes=2):
    """Algorithmic bytes one step must move: packed codes and fp32 scales read
    and written, q, k, v, beta, g read, y written, one slot index per request."""
    total = 0
    for b in head_bits:
        codes = d * d * int(b) // 8
        scales = 8 * d
        io = (3 * d + 1 + (d if gate == "kda" else 1) + d) * io_bytes
        total += 2 * codes + 2 * scales + io
    return B * total + 4 * B


def f32_bytes_per_step(B, H, d, gate, io_bytes=2):
    io = (3 * d + 1 + (d if gate == "kda" else 1) + d) * io_bytes
    return B * H * (2 * 4 * d * d + io) + 4 * B


def impact_from_workload(wl, layer, steps):
    """Row-impact scores [H, d] from the last `steps` warm-up steps' inputs
    (the offline calibration; tokens = steps x requests)."""
    import workload as W
    from quantized_gated_delta_amd import allocate as A
    acc = A.RowImpact()
    B, H, d = wl.B, wl.H, wl.d
    for t in range(-steps, 0):
        x = {k: W.to_f32(v) for k, v in wl.step_inputs(layer, t).items()}
        acc.add(x["q"].reshape(B, H, d), x["k"].reshape(B, H, d), x["beta"].reshape(B, H),
                x["g"].reshape((B, H, d) if layer.gate == "kda" else (B, H)))
    return acc.scores()


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3a")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-variants", action="store_true", help="only the headline kernel")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prewarm", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up steps")
    ap.add_argument("--timeline", action="store_true",
                    help="only the per-phase wave timeline of the workload's step, from the "
                         "instrumented build (python -m quantized_gated_delta_amd.build "
                         "--timeline); prints one JSON line")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for profiles)")
    ap.add_argument("--trajectory", action="store_true",
                    help="only the c4 trajectory: GDN + KDA layers, per-step y error of the "
                         "quantized step against the fp32-state step")
    ap.add_argument("--traj-steps", type=int, default=1024)
    ap.add_argument("--allocate", action="store_true",
                    help="with --trajectory: also run uniform-6 and lifetime-aware pools")
    ap.add_argument("--pivots", type=int, default=2,
                    help="FP16 pivot heads per layer for the --allocate comparison")
    ap.add_argument("--calib", type=int, default=256,
                    help="requests whose warm-up states calibrate the allocation")
    ap.add_argument("--only", choices=("kda_mixed", "kda_rows", "kra", "kda_rows_kra",
                                       "fp32_state"),
                    help="time only this variant of the B=512 H=48 step (for profiling runs): "
                         "KDA 4/6/8 per head, KDA with per-key-row widths, the key-row-aware "
                         "fit on the 6-bit GDN pool, that fit on the per-key-row widths, or "
                         "the fp32-state comparator; prints one short JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: every (request, head) update is independent "
              "and the path has no collective; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.timeline:
        tl_lib = os.path.join(ROOT, "quantized_gated_delta_amd", "libsq_timeline.so")
        if not os.path.exists(tl_lib):
            print("--timeline needs the instrumented build: python -m "
                  "quantized_gated_delta_amd.build --timeline", file=sys.stderr)
            sys.exit(2)
        os.environ["SQ_LIBRARY"] = tl_lib

    import numpy as np
    import torch

    import quantized_gated_delta_amd as Q
    import workload as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calib:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        eprint("copied 3 x 1 GiB")
        return

    if args.trajectory:
        trajectory(args, dev)
        return

    wl = W.make(args.workload)
    layer = wl.layers[0]
    B, H, d = wl.B, wl.H, wl.d
    kda = layer.gate == "kda"
    io_dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def make_pool(lay):
        pool = Q.StatePool(wl.n_slots, H, d, lay.head_bits.tolist(), lay.gate, device=dev)
        slot = to_dev(lay.slot_of.astype(np.int32))
        return pool, slot

    # ---- initial state: 128 unquantized fp32 warm-up steps on the GPU, then quantize
    eprint("warm-up: %d fp32 steps for %d x %d heads" % (W.WARMUP_STEPS, B, H))
    t0 = time.time()
    state = torch.zeros((wl.n_slots, H, d, d), dtype=torch.float32, device=dev)
    slot_l = to_dev(layer.slot_of.astype(np.int32))
    y = torch.empty((B, H, d), dtype=io_dt, device=dev)
    for t in range(-W.WARMUP_STEPS, 0):
        x = {k: to_dev(v) for k, v in wl.step_inputs(layer, t).items()}
        Q.sq_f32_decode_step(state, wl.n_slots, H, d, d, int(kda), slot_l, B, x["q"], x["k"],
                             x["v"], x["beta"], x["g"], y)
    torch.cuda.synchronize()
    eprint("warm-up done in %.1f s" % (time.time() - t0))
    pool, slot = make_pool(layer)
    pool.quant_state(slot, state[slot.long()])

    # ---- resident inputs for the timed steps (4 distinct steps, cycled)
    steps_in = [{k: to_dev(v) for k, v in wl.step_inputs(layer, t).items()} for t in range(4)]
    y = torch.empty((B * H, d), dtype=io_dt, device=dev)
    stream = torch.cuda.current_stream()

    if args.timeline:
        print(json.dumps(timeline(pool, slot, steps_in, y, args, B, H)), flush=True)
        return

    def run(pl, sl, n, per_launch=None):
        for i in range(n):
            x = steps_in[i % 4]
            if per_launch is not None:
                per_launch[i][0].record(stream)
            pl.decode_step(sl, x["q"], x["k"], x["v"], x["beta"], x["g"], y)
            if per_launch is not None:
                per_launch[i][1].record(stream)

    def timed(pl, sl, fn=None):
        fn = fn or (lambda n, ev=None: run(pl, sl, n, ev))
        # bring the clocks to their loaded steady state first (untimed), then
        # the W warm-up steps, then exactly K timed steps
        t_end = time.perf_counter() + args.prewarm
        while time.perf_counter() < t_end:
            fn(10)
            torch.cuda.synchronize()
        fn(args.warmup)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        fn(args.steps)
        t_host = time.perf_counter() - t_start
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        eprint("  host enqueue %.1f us/step, wall %.1f us/step" % (t_host / args.steps * 1e6,
                                                                  wall / args.steps * 1e6))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        fn(args.steps, ev)
        torch.cuda.synchronize()
        launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        return wall / args.steps * 1e3, launch_ms

    def kda_setup(per_row):
        """KDA at the c3 shape: bits 4/6/8 at 25/50/25 % per head, or 4/6/8 on
        25/50/25 % of every head's key rows; pool quantized from the warm-up
        state.  Returns (pool, run function, algorithmic bytes per step,
        workload, layer)."""
        wk = W.custom("kda", B, H, d, W.mixed_bits(0, 0, H), dtype="bf16",
                      n_slots=wl.n_slots, permute=True, seed=0, name="kda_mixed")
        lk = wk.layers[0]
        if per_row:
            rb, _ = W.row_widths_by_lifetime(lk.gate_rates)
            pk = Q.StatePool(wl.n_slots, H, d, [0] * H, "kda", device=dev, row_bits=rb)
            kb = algo_bytes_per_step(B, H, d, [6] * H, "kda")   # 6 bits on average per head
        else:
            pk = Q.StatePool(wl.n_slots, H, d, lk.head_bits.tolist(), "kda", device=dev)
            kb = algo_bytes_per_step(B, H, d, lk.head_bits, "kda")
        sk = to_dev(lk.slot_of.astype(np.int32))
        st = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
        st.copy_(state[slot_l.long()])
        pk.quant_state(sk, st)
        del st
        kin = [{k: to_dev(v) for k, v in wk.step_inputs(lk, t).items()} for t in range(4)]

        def run_k(n, ev=None):
            for i in range(n):
                x = kin[i % 4]
                if ev is not None:
                    ev[i][0].record(stream)
                pk.decode_step(sk, x["q"], x["k"], x["v"], x["beta"], x["g"], y)
                if ev is not None:
                    ev[i][1].record(stream)
        return pk, run_k, kb, wk, lk

    if args.only:
        if args.only == "fp32_state":
            def run_f(n, ev=None):
                for i in range(n):
                    x = steps_in[i % 4]
                    if ev is not None:
                        ev[i][0].record(stream)
                    Q.sq_f32_decode_step(state, wl.n_slots, H, d, d, int(kda), slot_l, B, x["q"],
                                         x["k"], x["v"], x["beta"], x["g"], y)
                    if ev is not None:
                        ev[i][1].record(stream)
            o_ms, o_launch = timed(None, None, run_f)
            ob = f32_bytes_per_step(B, H, d, layer.gate, 2 if wl.dtype == "bf16" else 4)
        elif args.only == "kra":
            pool.set_row_impact(torch.from_numpy(impact_from_workload(wl, layer, 4)).to(dev))
            o_ms, o_launch = timed(pool, slot)
            ob = algo_bytes_per_step(B, H, d, layer.head_bits, layer.gate)
        else:
            pk, run_k, ob, wk, lk = kda_setup(args.only != "kda_mixed")
            if args.only == "kda_rows_kra":
                pk.set_row_impact(torch.from_numpy(impact_from_workload(wk, lk, 4)).to(dev))
            o_ms, o_launch = timed(None, None, run_k)
        print(json.dumps({"variant": args.only, "us_per_step": o_ms * 1e3,
                          "us_per_launch": o_launch * 1e3, "algo_bytes_per_step": ob,
                          "achieved_GBps": ob / (o_launch * 1e-3) / 1e9}), flush=True)
        return

    eprint("timing the quantized decode step (%s)" % args.workload)
    ms_step, ms_launch = timed(pool, slot)
    updates = B * H
    bytes_step = algo_bytes_per_step(B, H, d, layer.head_bits, layer.gate,
                                     2 if wl.dtype == "bf16" else 4)
    achieved = bytes_step / (ms_launch * 1e-3) / 1e9
    eprint("quantized: %.2f us/step wall, %.2f us/launch, %.1f GB/s (%.1f%% of 8 TB/s)"
           % (ms_step * 1e3, ms_launch * 1e3, achieved, 100 * achieved / HBM_PEAK_GBS))

    variants = {}
    if not args.no_variants:
        # fp32-state comparator on the same inputs
        def run_f32(n, ev=None):
            for i in range(n):
                x = steps_in[i % 4]
                if ev is not None:
                    ev[i][0].record(stream)
                Q.sq_f32_decode_step(state, wl.n_slots, H, d, d, int(kda), slot_l, B, x["q"],
                                     x["k"], x["v"], x["beta"], x["g"], y)
                if ev is not None:
                    ev[i][1].record(stream)
        f_ms, f_launch = timed(None, None, run_f32)
        fb = f32_bytes_per_step(B, H, d, layer.gate, 2 if wl.dtype == "bf16" else 4)
        variants["fp32_state"] = {
            "updates_per_s": updates / (f_ms * 1e-3), "us_per_step": f_ms * 1e3,
            "us_per_launch": f_launch * 1e3, "algo_bytes_per_step": fb,
            "achieved_GBps": fb / (f_launch * 1e-3) / 1e9,
            "speedup_quantized_vs_fp32": f_ms / ms_step}
        eprint("fp32 state: %.2f us/step, %.1f GB/s" % (f_ms * 1e3, variants["fp32_state"]["achieved_GBps"]))
        variants["split_epilogue"] = split_epilogue(pool, slot, steps_in, y, timed, ms_step,
                                                    stream, dev, B, H, d, io_dt)
        # the key-row-aware fit in the fused epilogue (scores from warm-up inputs)
        imp = torch.from_numpy(impact_from_workload(wl, layer, 4)).to(dev)
        pool.set_row_impact(imp)
        r_ms, r_launch = timed(pool, slot)
        pool.set_row_impact(None)
        variants["key_row_aware_fit_6bit"] = {
            "updates_per_s": updates / (r_ms * 1e-3), "us_per_step": r_ms * 1e3,
            "us_per_launch": r_launch * 1e3, "algo_bytes_per_step": bytes_step,
            "achieved_GBps": bytes_step / (r_launch * 1e-3) / 1e9,
            "hbm_frac": bytes_step / (r_launch * 1e-3) / 1e9 / HBM_PEAK_GBS}
        eprint("key-row-aware fit: %.2f us/step, %.1f GB/s"
               % (r_ms * 1e3, variants["key_row_aware_fit_6bit"]["achieved_GBps"]))
        # the mixed 4/8-bit variant (8-bit for heads whose half-life exceeds 64 steps)
        if args.workload == "c3a":
            wb = W.make("c3b")
            lb = wb.layers[0]
            pool_b, slot_b = make_pool(lb)
            stb = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
            stb.copy_(state[slot_l.long()])
            pool_b.quant_state(slot_b, stb)
            del stb
            b_ms, b_launch = timed(pool_b, slot_b)
            bb = algo_bytes_per_step(B, H, d, lb.head_bits, lb.gate)
            variants["mixed_4_8_halflife"] = {
                "n_8bit_heads": int((lb.head_bits == 8).sum()), "seed": wb.seed,
                "updates_per_s": updates / (b_ms * 1e-3), "us_per_step": b_ms * 1e3,
                "us_per_launch": b_launch * 1e3, "algo_bytes_per_step": bb,
                "achieved_GBps": bb / (b_launch * 1e-3) / 1e9,
                "hbm_frac": bb / (b_launch * 1e-3) / 1e9 / HBM_PEAK_GBS}
            eprint("mixed 4/8: %.2f us/step, %.1f GB/s" % (b_ms * 1e3, variants["mixed_4_8_halflife"]["achieved_GBps"]))
            pool_b.close()
            # KDA (per-key-channel gate) at the same shape, bits 4/6/8 at 25/50/25 %
            pool_k, run_k, kb, _, _ = kda_setup(False)
            k_ms, k_launch = timed(None, None, run_k)
            variants["kda_mixed_4_6_8"] = {
                "updates_per_s": updates / (k_ms * 1e-3), "us_per_step": k_ms * 1e3,
                "us_per_launch": k_launch * 1e3, "algo_bytes_per_step": kb,
                "achieved_GBps": kb / (k_launch * 1e-3) / 1e9,
                "hbm_frac": kb / (k_launch * 1e-3) / 1e9 / HBM_PEAK_GBS}
            eprint("kda mixed: %.2f us/step, %.1f GB/s" % (k_ms * 1e3, variants["kda_mixed_4_6_8"]["achieved_GBps"]))
            pool_k.close()
            # the same KDA step with per-key-row widths: 4/6/8 bits on 25/50/25 %
            # of every head's key rows (the KDA unit of the allocation)
            pool_r, run_r, pb, wk, lk = kda_setup(True)
            p_ms, p_launch = timed(None, None, run_r)
            variants["kda_per_row_4_6_8"] = {
                "updates_per_s": updates / (p_ms * 1e-3), "us_per_step": p_ms * 1e3,
                "us_per_launch": p_launch * 1e3, "algo_bytes_per_step": pb,
                "achieved_GBps": pb / (p_launch * 1e-3) / 1e9,
                "hbm_frac": pb / (p_launch * 1e-3) / 1e9 / HBM_PEAK_GBS}
            eprint("kda per-row widths: %.2f us/step, %.1f GB/s"
                   % (p_ms * 1e3, variants["kda_per_row_4_6_8"]["achieved_GBps"]))
            # the same pool with the key-row-aware fit (scores from warm-up inputs)
            pool_r.set_row_impact(torch.from_numpy(impact_from_workload(wk, lk, 4)).to(dev))
            pk_ms, pk_launch = timed(None, None, run_r)
            variants["kda_per_row_4_6_8_key_row_aware"] = {
                "updates_per_s": updates / (pk_ms * 1e-3), "us_per_step": pk_ms * 1e3,
                "us_per_launch": pk_launch * 1e3, "algo_bytes_per_step": pb,
                "achieved_GBps": pb / (pk_launch * 1e-3) / 1e9,
                "hbm_frac": pb / (pk_launch * 1e-3) / 1e9 / HBM_PEAK_GBS}
            eprint("kda per-row widths, key-row-aware fit: %.2f us/step, %.1f GB/s"
                   % (pk_ms * 1e3, pb / (pk_launch * 1e-3) / 1e9))
            pool_r.close()
    del state
    copy_GBps, torch_copy_GBps = device_copy_GBps(dev)
    eprint("device copy: %.0f GB/s (streaming kernel), %.0f GB/s (torch copy)"
           % (copy_GBps, torch_copy_GBps))
    rates = issue_rates(dev)
    eprint("issue rates (T lane-ops/s): " + ", ".join("%s %.1f" % kv for kv in rates.items()))
    if not args.no_variants:
        variants["smaller_configs"] = config_timings(dev)

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, layer, args.cpu_seconds)
        eprint("cpu oracle: %.3g updates/s on %d threads" % (cpu["value"], cpu["cores"]))

    # HBM traffic and VALU issue from the committed counter profile, while the
    # kernel source it was taken on is the one built here
    prof = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            cp = json.load(f)
        if cp.get("kernel_src_sha256_16") == kernel_hash():
            prof = cp["variants"].get(args.workload)
    elems = B * H * d * d
    hb = [int(b) for b in layer.head_bits]
    mix = {}
    for b in hb:
        for k, v in essential_mix(b).items():
            mix[k] = mix.get(k, 0.0) + v / len(hb)
    ess = sum(mix.values())
    # lane-operations per second: achieved (essential work over the launch
    # time) and the unit-count issue limit of the same operation mix
    alu_achieved = ess * elems / (ms_launch * 1e-3) / 1e12
    alu_peak = valu_peak(mix)

    out = {
        "metric": "state-updates/s (req x head x step) and achieved HBM GB/s vs peak at B=512",
        "value": updates / (ms_step * 1e-3),
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generator; state from 128 fp32 warm-up steps)",
        "config": {"workload": "gdn_decode_%s" % args.workload, "B": B, "H": H, "d_k": d,
                   "d_v": d, "bits": sorted(set(int(b) for b in layer.head_bits)),
                   "pool_slots": wl.n_slots, "io_dtype": wl.dtype, "scales": "fp32",
                   "arithmetic": "look-up and read-out sums exact on int8 matrix cores, "
                                 "combined in f64, u rounded once to f32; update and "
                                 "requantizer in f32",
                   "gate": layer.gate},
        "roofline": {"bound": "alu", "achieved": alu_achieved, "peak": alu_peak,
                     "unit": "T lane-ops/s", "frac": alu_achieved / alu_peak,
                     "traffic": None if prof is None else prof["bytes_per_launch"],
                     "essential_valu_per_element": ess,
                     "essential_mix_per_element": mix,
                     "single_issue_classes": list(SINGLE_ISSUE),
                     "peak_pairable_T": VALU_PAIR_PEAK, "peak_single_issue_T": VALU_SINGLE_PEAK,
                     "issue_rates_T_lane_ops_per_s": rates,
                     "state_elements_per_launch": elems,
                     "valu_insts_per_element": None if prof is None else prof["valu_insts_per_element"],
                     "valu_issue_frac": None if prof is None else prof["valu_issue_frac"],
                     "valu_issue_frac_at_4_cycles":
                         None if prof is None else prof["valu_issue_frac_at_4_cycles"],
                     "kernel_src_sha256_16": kernel_hash(),
                     "us_per_launch": ms_launch * 1e3,
                     "kernel": "decode_kernel<128, %s, bf16, bf16>" % layer.gate.upper(),
                     "hbm": {"achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": achieved / HBM_PEAK_GBS,
                             "algo_bytes_per_launch": bytes_step,
                             "device_copy_GBps": copy_GBps, "torch_copy_GBps": torch_copy_GBps,
                             "frac_of_device_copy": achieved / copy_GBps}},
        "cpu_baseline": cpu,
        "variants": variants,
    }
    print(json.dumps(out), flush=True)


# Phases of the timeline build's stamps (slot pairs; see sq_kernels.hip)
TL_SLOTS = 16
TL_PHASES = [("slot resolve", 0, 1), ("tile loads in flight", 1, 2), ("codes to LDS", 2, 3),
             ("exponent bounds, k.q", 3, 4), ("digit rows", 4, 5), ("barrier 1", 5, 6),
             ("matrix cores, u, y", 6, 7), ("barrier 2", 7, 8), ("S', column partials", 8, 9),
             ("barrier 3", 9, 10), ("column fold (waves 0-1)", 10, 11), ("barrier 4", 11, 12),
             ("requantize, pack, store", 12, 13)]


def timeline(pool, slot, steps_in, y, args, B, H):
    """Per-wave phase durations of one decode launch from the timeline build:
    untimed steps for --prewarm seconds, then three launches with the stamps
    cleared before each; the last one is summarised.  Shader-clock cycles
    (s_memtime), mean and median over the launch's tiles, per wave of the
    workgroup.  The stamps add a few per cent to the launch time."""
    import ctypes

    import numpy as np
    import torch

    from quantized_gated_delta_amd import sq as S
    L = S.lib()
    L.sq_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.sq_timeline_read.restype = ctypes.c_int
    L.sq_timeline_clear.restype = ctypes.c_int
    n_tiles = B * H
    if n_tiles > 24576:
        raise SystemExit("the timeline build records the first 24576 tiles; this workload has %d"
                         % n_tiles)
    t0, i = time.time(), 0
    while time.time() - t0 < max(args.prewarm, 0.3):
        x = steps_in[i % 4]
        i += 1
        pool.decode_step(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y)
    torch.cuda.synchronize()
    buf = np.zeros(24576 * 4 * TL_SLOTS, np.uint64)
    us = []
    for rep in range(3):
        if L.sq_timeline_clear() != 0:
            raise SystemExit("sq_timeline_clear failed")
        torch.cuda.synchronize()
        x = steps_in[rep % 4]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pool.decode_step(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y)
        e1.record()
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3)
    if L.sq_timeline_read(buf.ctypes.data, buf.nbytes) != 0:
        raise SystemExit("sq_timeline_read failed")
    tl = buf.reshape(24576, 4, TL_SLOTS)[:n_tiles].astype(np.int64)
    if (tl[:, :, :14] == 0).any():
        raise SystemExit("missing stamps: the workload's heads do not all take the uniform "
                         "fused path this build instruments")
    waves = {}
    for w in range(4):
        ph = {}
        for name, a, b in TL_PHASES:
            dt = tl[:, w, b] - tl[:, w, a]
            ph[name] = {"mean": float(dt.mean()), "median": float(np.median(dt))}
        life = tl[:, w, 13] - tl[:, w, 0]
        ph["wave life"] = {"mean": float(life.mean()), "median": float(np.median(life))}
        waves["wave %d" % w] = ph
        eprint("wave %d: " % w + ", ".join("%s %.0f" % (k, v["mean"]) for k, v in ph.items()))
    return {"timeline": "decode step, per-wave phase cycles (s_memtime)",
            "workload": args.workload, "tiles": n_tiles, "launch_us_instrumented": us,
            "waves": waves}


def device_copy_GBps(dev, nbytes=2 << 30, reps=10):
    """Device copies of nbytes (read + write) timed with HIP events on the
    launch stream: the library's hand-written streaming copy (16-byte
    non-temporal loads and stores), the practically reachable HBM rate next
    to the 8 TB/s peak, and torch's copy for comparison.  Returns
    (streaming copy GB/s, torch copy GB/s)."""
    import torch

    import quantized_gated_delta_amd as Q
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    stream = torch.cuda.current_stream()

    def rate(fn):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return 2 * nbytes / (ev[0].elapsed_time(ev[1]) * 1e-3 / reps) / 1e9

    own = rate(lambda: Q.sq_device_copy(a, b, nbytes, stream))
    tc = rate(lambda: b.copy_(a))
    del a, b
    return own, tc


def issue_rates(dev, reps=4):
    """Measured issue rate of each opcode class of the decode step's
    per-element work (the library's sq_issue_probe: independent chains of one
    opcode over the whole chip; "fma+cvt" interleaves the two, which pair),
    timed with HIP events on the launch stream, reported next to the
    unit-count peak.  Returns {class: T lane-operations per second}."""
    import torch

    import quantized_gated_delta_amd as Q
    classes = {"fma": Q.SQ_PROBE_FMA_F32, "mul": Q.SQ_PROBE_MUL_F32,
               "max3": Q.SQ_PROBE_MAX3_F32, "cvt": Q.SQ_PROBE_CVT_BYTE,
               "bfe": Q.SQ_PROBE_BFE, "alignbit": Q.SQ_PROBE_ALIGNBIT,
               "fma_f64": Q.SQ_PROBE_FMA_F64, "fma+cvt": Q.SQ_PROBE_FMA_CVT_PAIR}
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    out = {}
    for name, op in classes.items():
        Q.sq_issue_probe(op, sink, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            Q.sq_issue_probe(op, sink, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        out[name] = Q.SQ_PROBE_OPS_PER_LAUNCH * reps / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12
    return out


def config_timings(dev, K=20, G=20, R=5):
    """The smaller workloads: c0 latency; c1 and c2 hot (K back-to-back steps)
    and flushed (a 1 GiB buffer written before each step, so the pool comes
    from HBM rather than the 256 MB Infinity Cache).  Per-step HIP events.
    "graph": G steps captured in one HIP graph (the step allocates nothing and
    enqueues no memset), replayed R times between two events, so the host's
    launch path is out of the per-step time as in a serving loop."""
    import numpy as np
    import torch

    import quantized_gated_delta_amd as Q
    import workload as W

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    out = {}
    for name in ("c0", "c1", "c2"):
        wl = W.make(name)
        lay = wl.layers[0]
        B, H, d = wl.B, wl.H, wl.d
        kda = lay.gate == "kda"
        pool = Q.StatePool(wl.n_slots, H, d, lay.head_bits.tolist(), lay.gate, device=dev)
        slot = to_dev(lay.slot_of.astype(np.int32))
        state = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
        ident = torch.arange(B, dtype=torch.int32, device=dev)
        ins = [{k: to_dev(v) for k, v in wl.step_inputs(lay, t).items()} for t in range(4)]
        y = torch.empty((B * H, d), dtype=ins[0]["q"].dtype, device=dev)
        for i in range(8):
            x = ins[i % 4]
            Q.sq_f32_decode_step(state, B, H, d, d, int(kda), ident, B, x["q"], x["k"], x["v"],
                                 x["beta"], x["g"], y)
        pool.quant_state(slot, state)
        res = {}
        for mode in ("hot", "flushed"):
            if mode == "flushed" and name == "c0":
                continue
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(K)]
            for i in range(K + 3):
                x = ins[i % 4]
                if mode == "flushed":
                    flush.fill_(i & 0xFF)
                if i >= 3:
                    ev[i - 3][0].record()
                pool.decode_step(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y)
                if i >= 3:
                    ev[i - 3][1].record()
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
            nb = algo_bytes_per_step(B, H, d, lay.head_bits, lay.gate,
                                     2 if wl.dtype == "bf16" else 4)
            res[mode] = {"us_per_step": us, "updates_per_s": B * H / (us * 1e-6),
                         "achieved_GBps": nb / (us * 1e-6) / 1e9}
        # graph replay: capture on a side stream after an eager warm-up there
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            pool.decode_step(slot, ins[0]["q"], ins[0]["k"], ins[0]["v"], ins[0]["beta"],
                             ins[0]["g"], y)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                x = ins[i % 4]
                pool.decode_step(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(R):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (R * G)
        nb = algo_bytes_per_step(B, H, d, lay.head_bits, lay.gate, 2 if wl.dtype == "bf16" else 4)
        res["graph"] = {"us_per_step": us, "updates_per_s": B * H / (us * 1e-6),
                        "achieved_GBps": nb / (us * 1e-6) / 1e9}
        del g
        out[name] = res
        pool.close()
        eprint("%s: %s" % (name, {m: round(v["us_per_step"], 1) for m, v in res.items()}))
    del flush
    return out


def split_epilogue(pool, slot, steps_in, y, timed, fused_ms, stream, dev, B, H, d, io_dt):
    """The pages' split design: the update kernel writes S' (fp32) and y, and
    the requantization (sq_quant_state of S') runs on a second stream.
    One layer: the next step's update of the same slots waits for the
    epilogue.  Two layers (two pools of this shape): the epilogue of one
    layer overlaps the update of the other.  Compared with the fused step."""
    import torch

    import quantized_gated_delta_amd as Q
    epi = torch.cuda.Stream()
    S_a = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    upd_done = [torch.cuda.Event(), torch.cuda.Event()]
    epi_done = [torch.cuda.Event(), torch.cuda.Event()]

    def split_one(pl, x, yy, S, i):
        stream.wait_event(epi_done[i])
        pl.decode_update(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], yy, S)
        upd_done[i].record(stream)
        epi.wait_event(upd_done[i])
        pl.quant_state(slot, S, stream=epi)
        epi_done[i].record(epi)

    def run_split(n, ev=None):
        for i in range(n):
            if ev is not None:
                ev[i][0].record(stream)
            split_one(pool, steps_in[i % 4], y, S_a, 0)
            stream.wait_event(epi_done[0])
            if ev is not None:
                ev[i][1].record(stream)

    def run_update_only(n, ev=None):
        for i in range(n):
            x = steps_in[i % 4]
            if ev is not None:
                ev[i][0].record(stream)
            pool.decode_update(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y, S_a)
            if ev is not None:
                ev[i][1].record(stream)

    def run_quant_only(n, ev=None):
        for i in range(n):
            if ev is not None:
                ev[i][0].record(stream)
            pool.quant_state(slot, S_a)
            if ev is not None:
                ev[i][1].record(stream)

    s1_ms, _ = timed(None, None, run_split)
    _, upd_launch = timed(None, None, run_update_only)
    _, q_launch = timed(None, None, run_quant_only)
    eprint("split, one layer: %.2f us/step (update %.1f + requantize %.1f us per launch); "
           "fused %.2f" % (s1_ms * 1e3, upd_launch * 1e3, q_launch * 1e3, fused_ms * 1e3))

    pool2 = Q.StatePool(pool.n_slots, H, d, pool.head_bits,
                        "kda" if pool.gate == Q.SQ_GATE_KDA else "gdn", device=dev)
    pool2.buf.copy_(pool.buf)
    S_b = torch.empty_like(S_a)
    y2 = torch.empty_like(y)

    # (wall time per step is the figure here; the per-step events only mark
    # the main stream)
    def run_fused2(n, ev=None):
        for i in range(n):
            x = steps_in[i % 4]
            if ev is not None:
                ev[i][0].record(stream)
            pool.decode_step(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y)
            pool2.decode_step(slot, x["q"], x["k"], x["v"], x["beta"], x["g"], y2)
            if ev is not None:
                ev[i][1].record(stream)

    def run_split2(n, ev=None):
        for i in range(n):
            x = steps_in[i % 4]
            if ev is not None:
                ev[i][0].record(stream)
            split_one(pool, x, y, S_a, 0)
            split_one(pool2, x, y2, S_b, 1)
            if ev is not None:
                ev[i][1].record(stream)
        stream.wait_event(epi_done[0])
        stream.wait_event(epi_done[1])

    f2_ms, _ = timed(None, None, run_fused2)
    s2_ms, _ = timed(None, None, run_split2)
    eprint("two layers: fused %.2f us/step, split with overlapped epilogues %.2f us/step"
           % (f2_ms * 1e3, s2_ms * 1e3))
    pool2.close()
    return {"one_layer_us_per_step": s1_ms * 1e3, "fused_one_layer_us_per_step": fused_ms * 1e3,
            "update_kernel_us_per_launch": upd_launch * 1e3,
            "requantize_kernel_us_per_launch": q_launch * 1e3,
            "two_layers_fused_us_per_step": f2_ms * 1e3,
            "two_layers_split_overlapped_us_per_step": s2_ms * 1e3,
            "workspace_bytes_per_layer": B * H * d * d * 4}


def trajectory(args, dev):
    """c4: two layers (GDN, KDA), B = 1024, H = 32, bits 4/6/8 at 25/50/25 %.
    Both the packed pool and an fp32 state pool start from the same fp32
    warm-up state and see identical bf16 inputs; y of the quantized step is
    compared with y of the fp32-state step at every step (relative L2 over
    the whole [B, H, d] output).

    With --allocate the same trajectory also runs, side by side, pools whose
    per-head widths come from other rules at the same 6-bit average: uniform
    6 bits, the lifetime-aware allocation (calibrated on the warm-up states
    of the first --calib requests and the warm-up log-gates), and that
    allocation plus --pivots FP16 pivot heads outside the budget, and the
    same with the pivots' 16 bits counted inside the 6-bit average."""
    import numpy as np
    import torch

    import quantized_gated_delta_amd as Q
    import workload as W
    from quantized_gated_delta_amd import allocate as A

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    wl = W.make("c4", steps=args.traj_steps)
    B, H, d, T = wl.B, wl.H, wl.d, args.traj_steps
    ident = torch.arange(B, dtype=torch.int32, device=dev)
    layers = []
    for layer in wl.layers:
        kda = layer.gate == "kda"
        state = torch.zeros((B, H, d, d), dtype=torch.float32, device=dev)
        yw = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
        gsum = []
        for t in range(-W.WARMUP_STEPS, 0):
            xh = wl.step_inputs(layer, t)
            gsum.append(W.to_f32(xh["g"]).reshape((B, H, d) if kda else (B, H)).mean(axis=0))
            x = {k: to_dev(v) for k, v in xh.items()}
            Q.sq_f32_decode_step(state, B, H, d, d, int(kda), ident, B, x["q"], x["k"], x["v"],
                                 x["beta"], x["g"], yw)
        schemes = {"fixed_c4_mix": layer.head_bits.astype(np.uint8)}
        cal = None
        kra = set()
        if args.allocate:
            cal = A.calibrate(state[:args.calib], np.stack(gsum), avg_bits=6.0, n_pivots=0)
            schemes["uniform_6"] = np.full(H, 6, np.uint8)
            schemes["lifetime_6"] = cal["bits"]
            piv = A.allocate_bits(cal["distortion"], cal["weights"], 6.0, n_pivots=args.pivots)
            schemes["lifetime_6+%d_fp16_pivots" % args.pivots] = piv
            schemes["lifetime_6_incl_%d_fp16_pivots" % args.pivots] = A.allocate_bits(
                cal["distortion"], cal["weights"], 6.0, n_pivots=args.pivots,
                pivots_in_budget=True)
            # the same widths with the key-row-aware fit (scores from the warm-up inputs)
            schemes["uniform_6_key_row_aware"] = np.full(H, 6, np.uint8)
            schemes["lifetime_6+%d_fp16_pivots_key_row_aware" % args.pivots] = piv
            kra = {"uniform_6_key_row_aware",
                   "lifetime_6+%d_fp16_pivots_key_row_aware" % args.pivots}
            imp = torch.from_numpy(impact_from_workload(wl, layer, 16)).to(dev)
        perms, row_bits, imp_of = {}, {}, {}
        if args.allocate and kda:
            # per-key-row widths (the KDA unit): key channels permuted offline
            # so each head's rows run from the fastest- to the slowest-decaying
            # channel; 4/6/8 bits at 25/50/25 % of the rows in that order
            rb, perm = W.row_widths_by_lifetime(layer.gate_rates)
            name = "per_row_lifetime_4_6_8"
            schemes[name] = np.zeros(H, np.uint8)
            row_bits[name] = rb
            perms[name] = torch.from_numpy(perm).to(dev)
            # the same rows with the key-row-aware fit (scores permuted with
            # the key channels)
            name_k = "per_row_lifetime_4_6_8_key_row_aware"
            schemes[name_k] = np.zeros(H, np.uint8)
            row_bits[name_k] = rb
            perms[name_k] = perms[name]
            kra.add(name_k)
            imp_of[name_k] = torch.gather(imp, 1, perms[name].long())
            # per-row widths chosen by the lifetime objective (R22-R23 at the
            # key-row unit): per-row distortion of the calibration states,
            # per-row lifetime weights from the warm-up log-gates
            E = A.measure_row_distortion(state[:args.calib])
            rb2, perm2 = A.allocate_row_bits(E, A.row_lifetime_weights(np.stack(gsum)), 6.0)
            name = "per_row_lifetime_optimized_6"
            schemes[name] = np.zeros(H, np.uint8)
            row_bits[name] = rb2
            perms[name] = torch.from_numpy(perm2).to(dev)
        pools = {}
        for name, hb in schemes.items():
            pool = Q.StatePool(B, H, d, [int(b) for b in hb], layer.gate, device=dev,
                               row_bits=row_bits.get(name))
            if name in kra:
                pool.set_row_impact(imp_of.get(name, imp).contiguous())
            if name in perms:
                idx = perms[name][None, :, :, None].expand(B, H, d, d)
                pool.quant_state(ident, torch.gather(state, 2, idx).contiguous())
            else:
                pool.quant_state(ident, state)
            pools[name] = pool
        layers.append((layer, kda, state, pools, schemes, cal, perms, row_bits))
    torch.cuda.synchronize()
    errs = {(l.index, n): [] for l, _, _, pools, _, _, _, _ in layers for n in pools}
    yq = torch.empty((B * H, d), dtype=torch.bfloat16, device=dev)
    yf = torch.empty((B * H, d), dtype=torch.bfloat16, device=dev)
    t0 = time.time()
    for t in range(T):
        for layer, kda, state, pools, _, _, perms, _ in layers:
            x = {k: to_dev(v) for k, v in wl.step_inputs(layer, t).items()}
            Q.sq_f32_decode_step(state, B, H, d, d, int(kda), ident, B, x["q"], x["k"], x["v"],
                                 x["beta"], x["g"], yf)
            b = yf.float()
            nb = torch.linalg.vector_norm(b)
            for name, pool in pools.items():
                xi = x
                if name in perms:  # the same inputs with the key channels permuted
                    idx = perms[name][None].expand(B, H, d)
                    xi = dict(x)
                    for key in ("q", "k", "g"):
                        xi[key] = torch.gather(x[key].view(B, H, d), 2, idx).reshape(B * H, d)
                pool.decode_step(ident, xi["q"], xi["k"], xi["v"], xi["beta"], xi["g"], yq)
                errs[(layer.index, name)].append(
                    float(torch.linalg.vector_norm(yq.float() - b) / nb))
        if t in (0, 15, 63, 255, T - 1) or (t + 1) % 64 == 0:
            eprint("step %d: %s (%.0f s)" % (t + 1, {"%d/%s" % k: round(v[-1], 4)
                                                     for k, v in errs.items()},
                                            time.time() - t0))
    out = {"workload": "c4: GDN + KDA layers, B=1024, H=32, d=128, bf16, %d steps" % T,
           "y_rel_l2_vs_fp32_state": {}}
    for layer, _, _, pools, schemes, cal, _, row_bits in layers:
        per = {}
        for name, pool in pools.items():
            hb = schemes[name]
            e = np.array(errs[(layer.index, name)])
            marks = {str(s): float(e[s - 1]) for s in (1, 16, 64, 256, T) if s <= T}
            rbn = row_bits.get(name)
            per[name] = {"bits": {str(b): int((hb == b).sum()) for b in (0, 4, 6, 8, 16)
                                  if (hb == b).any()},
                         "row_bits": None if rbn is None else
                         {str(b): int((rbn == b).sum()) for b in (4, 6, 8)},
                         "slot_bytes": int(pool.slot_stride),
                         "at_step": marks, "mean": float(e.mean()), "max": float(e.max())}
        entry = per if args.allocate else per["fixed_c4_mix"]
        if cal is not None:
            entry = {"schemes": per,
                     "calibration": {"requests": int(args.calib),
                                     "half_life_steps": [round(float(x), 2)
                                                         for x in cal["half_life_steps"]],
                                     "nmse_4_6_8": [[float("%.3g" % v) for v in row]
                                                    for row in cal["distortion"]]}}
        out["y_rel_l2_vs_fp32_state"][layer.gate] = entry
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, layer, seconds, single_seconds=3.0):
    """The oracle, as it stands, on sampled (b, h) rows of the same workload,
    all host threads; repeated until `seconds` of wall time have passed.
    Then the same on one thread for `single_seconds`."""
    import numpy as np

    import oracle as O
    import workload as W
    d, H = wl.d, wl.H
    nthr = O.n_threads()
    rng = np.random.default_rng(0)
    n_rows = 64 * nthr
    flat = rng.choice(wl.B * H, size=n_rows, replace=False)
    rows = np.stack([flat // H, flat % H], 1)
    # initial records: a short FP64 warm-up of the sampled rows, then the pinned quantizer
    S = np.zeros((n_rows, d, d))
    for t in range(-8, 0):
        x = {k: W.to_f32(v) for k, v in wl.step_inputs(layer, t, rows).items()}
        O.f64_step(layer.gate == "kda", S, x["q"], x["k"], x["v"], x["beta"], x["g"])
    bits = layer.head_bits[rows[:, 1]]
    sizes = np.array([d * d * int(b) // 8 + 8 * d for b in bits], np.int64)
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    base = np.zeros(int(sizes.sum()), np.uint8)
    O.records_quantize(base, offs, bits, S.astype(np.float32), d, d)
    x = {k: W.to_f32(v) for k, v in wl.step_inputs(layer, 0, rows).items()}

    def run(secs, rows_per_pass):
        sub = slice(0, rows_per_pass)
        xs = {k: v[sub] for k, v in x.items()}
        done = 0
        t0 = time.perf_counter()
        while True:
            O.records_step(layer.gate == "kda", base, offs[sub], bits[sub], d, d, xs["q"],
                           xs["k"], xs["v"], xs["beta"], xs["g"])
            done += rows_per_pass
            el = time.perf_counter() - t0
            if el >= secs:
                return done, el

    done, el = run(seconds, n_rows)
    prev = os.environ.get("SQO_THREADS")
    os.environ["SQO_THREADS"] = "1"
    try:
        done1, el1 = run(single_seconds, 16)
    finally:
        if prev is None:
            del os.environ["SQO_THREADS"]
        else:
            os.environ["SQO_THREADS"] = prev
    return {"value": done / el, "unit": "state-updates/s", "cores": nthr, "kind": "oracle",
            "sample": "%d rows x %d passes of the B=%d H=%d d=%d step (%.1f s wall)"
                      % (n_rows, done // n_rows, wl.B, H, d, el),
            "single_thread_value": done1 / el1,
            # the same per-update byte model as the GPU line (codes + scales
            # read and written, q/k/v/beta/g/y), per sampled update
            "equivalent_GBps": done / el * algo_bytes_per_step(
                1, n_rows, d, bits, layer.gate, 2 if wl.dtype == "bf16" else 4) / n_rows / 1e9}


if __name__ == "__main__":
    main()
