#!/usr/bin/env python3
"""Throughput of the software-pipelined f16 NT GEMM on one MI355X.

Workload: out f16[8192, 8192] = lhs f16[8192, 8192] . rhs f16[8192, 8192]^T
with fp32 accumulation, operands uniform in [-1, 1) from the seeded SplitMix64
generator.  A step is one GEMM call of the producer/consumer kernel
(pgemm_f16_nt_ws) at the stage count that the untimed sweep over {1, 2, 3, 4}
finds fastest; the single-schedule kernel is swept too and reported beside it.

Prints one JSON line (rank 0) with TFLOP/s, the roofline position of the
kernel (average launch time from HIP events on the launch stream), the
vendor library's rate on the same operands (torch.matmul or torch.mm), and
the CPU oracle timed on a bounded sample of the same product (whose rows
are then compared with the library's, the only use of the oracle here).
Other
workloads (--workload): 4096^3, the ragged bf16 4095 x 1000 x 1000 and the
skinny 128 x 8192 x 16384 product (reported against the HBM roofline), and
the int32 NN 128 x 256 x 256 product (GOP/s, single-schedule kernel).

Profiling: --timed-only runs nothing on the GPU but the chosen kernel's
warm-up and timed steps (no sweep, single launches, vendor rounds or copy),
so that a profiler's per-kernel figures describe exactly the timed region;
--summarize DIR reduces the CSV output of rocprofv3 written under DIR
(kernel trace and/or counters) to the markdown tables kept in profiles/.
--power samples the board power against its cap over about a second of
back-to-back launches after the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6   # 256 CUs x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
# int32 VALU: 4 SIMDs x 16 lanes per CU retire one full-rate instruction per
# lane per clock; counting one multiply-add (2 ops) per lane-slot gives
# 256 CUs x 64 x 2 x 2.4 GHz.  An upper bound for the int32 kernel, whose
# 32-bit multiply issues below the full rate.
PEAK_S32_TOPS = 256 * 64 * 2 * 2.4e9 / 1e12

WORKLOADS = {
    # name: (M, N, K, seed workload index, element type)
    "s32_nn_128x256x256": (128, 256, 256, 1, "s32"),
    "f16_nt_8192": (8192, 8192, 8192, 3, "f16"),
    "f16_nt_4096": (4096, 4096, 4096, 2, "f16"),
    "bf16_nt_ragged": (4095, 1000, 1000, 4, "bf16"),
    "f16_nt_skinny": (128, 8192, 16384, 5, "f16"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources that define the kernels' code (host planning and launch code
# do not change what a kernel moves)
KERNEL_SOURCES = ("device_common.hpp", "wave_mma.hpp", "kernels.hpp", "instances.hpp")


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines, each line stripped: what
    the compiler sees, so that a comment edit keeps a recorded hash."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", line).strip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash(csrc=None) -> str:
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "software_pipelined_tiled_pipeline_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str, stages: int):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    want = kernel_source_hash()
    for line in open(path):
        m = re.match(r"\s*traffic\s+(\S+)\s+(\S+)\s+S=(\d+)\s+src=(\S+)\s+bytes=(\d+)", line)
        if m and m.group(1) == kernel and m.group(2) == workload and int(m.group(3)) == stages \
                and m.group(4) == want:
            return int(m.group(5))
    return None


def time_launches(fn, reps, stream):
    """Average duration (ms) of `reps` back-to-back launches: HIP events on
    the launch stream before the first and after the last."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# ------------------------------------------------------------ board power

def _hwmon_files():
    """sysfs power files of the first amdgpu hwmon that has them (microwatts)."""
    import glob
    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        for name in ("power1_average", "power1_input"):
            f = os.path.join(d, name)
            if os.path.exists(f):
                cap = os.path.join(d, "power1_cap")
                return f, cap if os.path.exists(cap) else None
    return None, None


def _amdsmi_power():
    """(power W, cap W) from amd-smi, or (None, None)."""
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "-p", "--json"], capture_output=True, text=True, timeout=10).stdout
        data = json.loads(out)
    except Exception:
        return None, None
    found = {}

    def walk(x, path=""):
        if isinstance(x, dict):
            for k, v in x.items():
                walk(v, path + "/" + str(k).lower())
        elif isinstance(x, list):
            for v in x:
                walk(v, path)
        elif isinstance(x, (int, float)) and "power" in path:
            found.setdefault(path, float(x))
    walk(data)
    power = next((v for k, v in found.items() if "socket_power" in k and "limit" not in k and "cap" not in k), None)
    cap = next((v for k, v in found.items() if "cap" in k or "limit" in k), None)
    return power, cap


def sample_power(run_for_s, launch, stream):
    """Runs `launch` back to back for about `run_for_s` seconds while a
    thread samples the board power; returns the samples' statistics (the
    first quarter left out: clock settling) and the number of launches."""
    import threading
    import torch
    f, capf = _hwmon_files()
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            if f:
                try:
                    samples.append(int(open(f).read()) / 1e6)
                except OSError:
                    pass
                time.sleep(0.005)
            else:
                w, _ = _amdsmi_power()
                if w is not None:
                    samples.append(w)
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < run_for_s:
        for _ in range(20):
            launch()
        n += 20
        torch.cuda.synchronize()
    seconds = time.perf_counter() - t0
    stop.set()
    th.join()
    cap = None
    if capf:
        try:
            cap = int(open(capf).read()) / 1e6
        except OSError:
            cap = None
    if cap is None:
        cap = _amdsmi_power()[1]
    res = {"launches": n, "seconds": round(seconds, 3)}
    if samples:
        tail = samples[len(samples) // 4:]  # after the clock has settled
        res.update({"source": "sysfs " + os.path.basename(f) if f else "amd-smi metric -p",
                    "samples": len(samples), "mean_w": round(sum(tail) / len(tail), 1),
                    "max_w": round(max(samples), 1), "cap_w": round(cap, 1) if cap else None})
    else:
        res["source"] = "none available"
    return res


# ------------------------------------------------- rocprofv3 CSV reduction

def kernel_label(name):
    """A short label for a kernel name from a trace: the pgemm NT kernels as
    'nt_ws_kernel f16 256x256x64 S=4' (+ ' split', ' staged'), read from
    their mangled template arguments; other names cut at the argument list."""
    m = re.match(r"_ZN5pgemm\d+(\w+?_kernel)I(DF16_|DF16b)NS_6NtGeomI((?:Li\d+E)+)EE((?:Lb\dE)*)E", name)
    if m:
        ints = [int(x) for x in re.findall(r"Li(\d+)E", m.group(3))]
        flags = [int(x) for x in re.findall(r"Lb(\d)E", m.group(4) or "")]
        label = f"{m.group(1)} {'f16' if m.group(2) == 'DF16_' else 'bf16'} {ints[0]}x{ints[1]}x{ints[2]} S={ints[3]}"
        if len(flags) >= 1 and flags[0]:
            label += " split"
        if len(flags) >= 2 and flags[1]:
            label += " staged"
        return label
    m = re.match(r"_ZN5pgemm\d+(\w+?)I(DF16_|DF16b)", name)
    if m:
        return f"{m.group(1)} {'f16' if m.group(2) == 'DF16_' else 'bf16'}"
    m = re.match(r"_ZN5pgemm\d+(s32_nn_kernel)ILi(\d)E", name)
    if m:
        return f"{m.group(1)} S={m.group(2)}"
    name = re.sub(r"\(.*", "", name)
    for noise in ("pgemm::", "void ", "(anonymous namespace)::"):
        name = name.replace(noise, "")
    return name[:100]


def summarize(dirs, timed_steps=0):
    """Markdown tables from rocprofv3 CSV output: per kernel, the number of
    dispatches and their mean / min / max duration (kernel trace), and the
    mean over dispatches of each counter summed over its instances, with the
    derived shader clock (GRBM_GUI_ACTIVE per XCD over the duration), MFMA
    busy (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x cycles), LDS bank
    conflict rate (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE) and HBM bytes
    (FETCH_SIZE and WRITE_SIZE in KiB, scaled by what a plain copy of known
    size reads: see --calibrate-copy)."""
    import csv
    import glob
    from collections import defaultdict

    def short(name):
        return kernel_label(name)

    lines = []
    for d in dirs:
        lines.append(f"### {d}\n")
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            durs = defaultdict(list)
            for r in csv.DictReader(open(f)):
                durs[short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            lines.append(f"kernel trace `{os.path.relpath(f, d)}`\n")
            last = f" | mean of the last {timed_steps} us" if timed_steps else ""
            lines.append(f"| kernel | dispatches | mean us | min us | max us{last} |")
            lines.append("|---|---|---|---|---|" + ("---|" if timed_steps else ""))
            for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
                row = f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f}"
                if timed_steps:
                    tail = v[-timed_steps:]
                    row += f" | {sum(tail) / len(tail):.2f}"
                lines.append(row + " |")
            lines.append("")
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            per = defaultdict(float)
            meta = {}
            for r in csv.DictReader(open(f)):
                per[(r["Dispatch_Id"], r["Counter_Name"])] += float(r["Counter_Value"])
                meta[r["Dispatch_Id"]] = (short(r["Kernel_Name"]),
                                          (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            agg = defaultdict(lambda: defaultdict(list))
            for (disp, c), v in per.items():
                agg[meta[disp][0]][c].append(v)
            for disp, (k, us) in meta.items():
                agg[k]["__us"].append(us)
            lines.append(f"counters `{os.path.relpath(f, d)}` (mean per dispatch)\n")
            counters = sorted({c for k in agg for c in agg[k] if c != "__us"})
            head = ["kernel", "dispatches", "us"] + counters
            derived = []
            if "GRBM_GUI_ACTIVE" in counters:
                derived.append("sclk GHz")
                if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
                    derived.append("MFMA busy")
            if "SQ_LDS_BANK_CONFLICT" in counters and "SQ_LDS_IDX_ACTIVE" in counters:
                derived.append("LDS conflict / active")
            if "FETCH_SIZE" in counters:
                derived.append("FETCH bytes (x2.0)")
            if "WRITE_SIZE" in counters:
                derived.append("WRITE bytes (x1.0)")
            lines.append("| " + " | ".join(head + derived) + " |")
            lines.append("|" + "---|" * (len(head) + len(derived)))
            for k, cs in sorted(agg.items(), key=lambda kv: -sum(kv[1]["__us"])):
                mean = {c: sum(v) / len(v) for c, v in cs.items()}
                row = [k, str(len(cs["__us"])), f"{mean['__us']:.2f}"] + [f"{mean.get(c, float('nan')):.6g}"
                                                                          for c in counters]
                if "sclk GHz" in derived:
                    cyc = mean["GRBM_GUI_ACTIVE"] / 8  # one GRBM per XCD
                    row.append(f"{cyc / (mean['__us'] * 1e3):.3f}")
                    if "MFMA busy" in derived:
                        row.append(f"{100 * mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.1f} %")
                if "LDS conflict / active" in derived:
                    row.append(f"{100 * mean['SQ_LDS_BANK_CONFLICT'] / max(mean['SQ_LDS_IDX_ACTIVE'], 1):.2f} %")
                if "FETCH bytes (x2.0)" in derived:
                    row.append(f"{mean['FETCH_SIZE'] * 1024 * 2.0:.4g}")
                if "WRITE bytes (x1.0)" in derived:
                    row.append(f"{mean['WRITE_SIZE'] * 1024 * 1.0:.4g}")
                lines.append("| " + " | ".join(row) + " |")
            lines.append("")
    print("\n".join(lines))


def _counter_per_dispatch(d, counter):
    """[(kernel label, value summed over the counter's instances)] per
    dispatch, in dispatch order, from the rocprofv3 CSV output under d."""
    import csv
    import glob
    per, order = {}, []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            if key not in per:
                per[key] = [kernel_label(r["Kernel_Name"]), 0.0]
                order.append(key)
            per[key][1] += float(r["Counter_Value"])
    return [tuple(per[k]) for k in sorted(order)]


def reduce_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, args):
    """HBM-side bytes per call of the timed kernel (and, for a K split, its
    reduction) from FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch), scaled
    by what the same counters read for a plain 512 MiB device copy
    (--calibrate-copy: 512 MiB read and 512 MiB written).  Prints the line
    that recorded_traffic() reads back while the kernel sources are
    unchanged."""
    n = 512 << 20
    cf = [v for k, v in _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE") if "copyBuffer" in k]
    cw = [v for k, v in _counter_per_dispatch(copy_write_dir, "WRITE_SIZE") if "copyBuffer" in k]
    read_scale = n / 1024 / (sum(cf) / len(cf))
    write_scale = n / 1024 / (sum(cw) / len(cw))
    M, N, K, _, fmt = WORKLOADS[args.workload]
    kname = "nt_ws_kernel" if args.variant == "ws" else "nt_swap_kernel"

    def per_call(d, counter):
        rows = _counter_per_dispatch(d, counter)
        main = [v for k, v in rows if k.startswith(kname + " ")][-args.steps:]
        red = [v for k, v in rows if k.startswith("reduce_splits")][-args.steps:]
        return (sum(main) + sum(red)) / len(main), len(main), len(red)

    fetch, nf, nr = per_call(fetch_dir, "FETCH_SIZE")
    write, _, _ = per_call(write_dir, "WRITE_SIZE")
    rd, wr = fetch * 1024 * read_scale, write * 1024 * write_scale
    alg = (M * K + N * K) * 2 + M * N * 2
    print(f"# {args.workload} {kname} S={args.stages}: last {nf} calls{' (+ reduce_splits)' if nr else ''}; "
          f"read scale {read_scale:.4f}, write scale {write_scale:.4f}")
    print(f"#   FETCH_SIZE {fetch:.0f} KiB -> {rd:.4g} B read, WRITE_SIZE {write:.0f} KiB -> {wr:.4g} B written; "
          f"algorithmic {alg} B; traffic / algorithmic {(rd + wr) / alg:.2f}")
    print(f"traffic {kname} {args.workload} S={args.stages} src={kernel_source_hash()} bytes={int(rd + wr)}")


def cpu_baseline(fmt, A, B, M, N, K, budget_s: float, gpu_rows=None):
    """The oracle, as it stands, on a leading block of output rows; the rows
    it computed are then compared with the same rows of the library's output
    for the same operands (`gpu_rows(rows)`: uint16 bits), element by element
    within the oracle's bound."""
    import oracle
    rows = 2
    t = 0.0
    while True:
        t0 = time.perf_counter()
        ref, mag = oracle.gemm_nt(fmt, A[:rows], B)
        t = time.perf_counter() - t0
        if t * 4 > budget_s or rows * 4 > M:
            break
        rows *= 4
    flops = 2.0 * rows * N * K
    res = {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"first {rows} of {M} output rows ({rows}x{N}x{K}), {t:.1f} s",
    }
    if gpu_rows is not None:
        bad, worst = oracle.check_nt(fmt, gpu_rows(rows), ref, mag)
        res["parity"] = {"elements": rows * N, "violations": int(bad), "worst_err_over_bound": round(float(worst), 4)}
        if bad:
            raise RuntimeError(f"the library's output fails the oracle on {bad} of {rows * N} elements")
    return res


def run_s32(args, torch, np):
    """The int32 NN product: GOP/s of back-to-back launches, the per-launch
    duration distribution (median, min, p90 of 200 single launches), and the
    oracle timed on the whole product, whose result is then compared bit for
    bit with the timed output."""
    import ctypes
    from software_pipelined_tiled_pipeline_amd import inputs, pgemm

    M, N, K, widx, _ = WORKLOADS[args.workload]
    log(f"[bench] generating {args.workload} operands {M}x{N}x{K}")
    A, B = inputs.make_operands("s32_nn", M, N, K, inputs.workload_seed(widx))
    dev = torch.device("cuda:0")
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    out = torch.empty((M, N), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ops = 2.0 * M * N * K
    f = pgemm.lib().pgemm_s32_nn
    sptr = ctypes.c_void_p(stream.cuda_stream)
    pa, pb, po = (ctypes.c_void_p(t.data_ptr()) for t in (dA, dB, out))

    def launcher(s):
        def call():
            st = f(pa, pb, po, M, N, K, s, sptr)
            if st != 0:
                raise pgemm.PgemmError(st, "pgemm_s32_nn")
        return call

    sweep = {}
    if not args.timed_only:
        time_launches(launcher(2), 200, stream)
    for s in () if args.timed_only else (1, 2):
        call = launcher(s)
        time_launches(call, 20, stream)
        ms = time_launches(call, 200, stream)
        sweep[f"swap S={s}"] = round(ops / (ms * 1e-3) / 1e9, 1)
        log(f"[bench] sweep swap S={s}: {ms * 1e3:.2f} us, {sweep[f'swap S={s}']} GOP/s")
    stages = args.stages or (int(max(sweep, key=sweep.get).split("S=")[1]) if sweep else 2)
    step = launcher(stages)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps of swap S={stages}")
    t0 = time.perf_counter()
    kern_ms = time_launches(step, args.steps, stream)
    wall = time.perf_counter() - t0
    single = sorted(time_launches(step, 1, stream) for _ in range(0 if args.timed_only else 200))
    value = ops * args.steps / wall / 1e9
    achieved = ops / (kern_ms * 1e-3) / 1e12

    result = {
        "metric": f"GOP/s for s32 NN GEMM {M}x{N}x{K}, 1 MI355X",
        "value": round(value, 1),
        "unit": "GOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {
            "workload": f"s32 NN GEMM M={M} N={N} K={K}, operands integers -8..8, wrapping int32 "
                        "accumulation, single-schedule swap",
            "M": M, "N": N, "K": K,
            "variant": "swap",
            "stages": stages,
            "stage_sweep_gops": sweep,
            "single_launch_us": {"median": round(single[100] * 1e3, 2), "min": round(single[0] * 1e3, 2),
                                 "p90": round(single[180] * 1e3, 2), "launches": 200} if single else None,
        },
        "roofline": {
            "bound": "alu",
            "achieved": round(achieved, 4),
            "peak": round(PEAK_S32_TOPS, 1),
            "unit": "TOP/s",
            "frac": round(achieved / PEAK_S32_TOPS, 5),
            "traffic": None,
            "kernel": "s32_nn_kernel",
            "kernel_avg_us": round(kern_ms * 1e3, 2),
        },
    }
    if not args.no_cpu_baseline and not args.timed_only:
        # the oracle, timed on the whole product, and its result compared
        # bit for bit with the timed output
        import oracle
        log("[bench] timing the CPU oracle on the whole product")
        reps, t = 1, 0.0
        while True:
            t0 = time.perf_counter()
            for _ in range(reps):
                ref = oracle.gemm_s32_nn(A, B)
            t = time.perf_counter() - t0
            if t > min(2.0, args.cpu_budget) or reps >= 1 << 16:
                break
            reps *= 4
        bad = int(np.count_nonzero(out.cpu().numpy() != ref))
        if bad:
            raise RuntimeError(f"timed output differs from the oracle in {bad} elements")
        result["cpu_baseline"] = {"value": ops * reps / t / 1e9, "unit": "GOP/s", "cores": oracle.threads(),
                                  "kind": "oracle", "sample": f"the whole product, {reps} times, {t:.2f} s",
                                  "parity": {"elements": M * N, "mismatches": bad}}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="f16_nt_8192")
    ap.add_argument("--variant", choices=["ws", "swap"], default="ws")
    ap.add_argument("--stages", type=int, default=0, help="0: fastest of the sweep")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy three times (a known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--timed-only", action="store_true",
                    help="launch only the warm-up and timed steps of the chosen kernel (stages: --stages, else "
                         "the entry point's default), for profiling")
    ap.add_argument("--tile", type=int, default=0, choices=[0, 128, 256],
                    help="force the output tile of the NT workloads (pgemm_set_tiling; 0: planned)")
    ap.add_argument("--power", action="store_true",
                    help="sample board power over about 1 s of back-to-back steps after the timed region (on by "
                         "default except with --timed-only)")
    ap.add_argument("--no-power", action="store_true", help="skip the power sampling")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="HBM bytes per call of --workload/--variant/--stages (mean of the last --steps calls) "
                         "from FETCH_SIZE / WRITE_SIZE runs and the --calibrate-copy runs; no GPU")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="reduce rocprofv3 CSV output under DIR to markdown tables and exit (no GPU); with "
                         "--steps, the trace table adds the mean of each kernel's last --steps dispatches "
                         "(the timed steps of a --timed-only run)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.steps if "--steps" in sys.argv else 0)
        return
    if args.traffic:
        reduce_traffic(*args.traffic, args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(a multi-GPU run would split the output columns across GPUs; it is not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = 512 << 20
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 3}))
        return

    from software_pipelined_tiled_pipeline_amd import inputs, pgemm

    pgemm.lib()  # fails loudly if the HIP library is missing
    if args.tile:
        pgemm.pgemm_set_tiling(args.tile, 0)
    if WORKLOADS[args.workload][4] == "s32":
        run_s32(args, torch, np)
        return
    M, N, K, widx, fmt = WORKLOADS[args.workload]
    kind, tdt = ("f16_nt", torch.float16) if fmt == "f16" else ("bf16_nt", torch.bfloat16)
    log(f"[bench] generating {args.workload} operands {M}x{N}x{K}")
    A, B = inputs.make_operands(kind, M, N, K, inputs.workload_seed(widx))
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A.view(np.int16)).to(dev).view(tdt)
    dB = torch.from_numpy(B.view(np.int16)).to(dev).view(tdt)
    out = torch.empty((M, N), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream()
    flops = 2.0 * M * N * K
    # The skinny product streams a 256 MiB rhs, about the size of the
    # 256 MB Infinity Cache: launches alternate between two rhs sets so that
    # a launch cannot be served from what the previous one left in the cache.
    sets = [(A, B, dA, dB)]
    if args.workload == "f16_nt_skinny":
        A2, B2 = inputs.make_operands(kind, M, N, K, inputs.workload_seed(widx) + 1)
        sets.append((A2, B2, torch.from_numpy(A2.view(np.int16)).to(dev).view(tdt),
                     torch.from_numpy(B2.view(np.int16)).to(dev).view(tdt)))
    turn = [0]

    def operands():
        t = turn[0] % len(sets)
        turn[0] += 1
        return t, sets[t][2], sets[t][3]

    # Launches go straight to the C ABI with the pointers and the stream
    # handle resolved once, so that host-side argument marshalling does not
    # show up in the timing of short kernels.
    import ctypes
    L = pgemm.lib()
    names = {"ws": f"pgemm_{fmt}_nt_ws", "swap": f"pgemm_{fmt}_nt"}
    sptr = ctypes.c_void_p(stream.cuda_stream)
    ptrs = [(ctypes.c_void_p(x[2].data_ptr()), ctypes.c_void_p(x[3].data_ptr())) for x in sets]
    optr = ctypes.c_void_p(out.data_ptr())

    # a K-split plan keeps its partial sums in a workspace the caller owns
    for variant in ("ws", "swap"):
        for s in (1, 2, 3, 4):
            need = pgemm.pgemm_query("nt_" + variant, s, M, N, K)["workspace_bytes"]
            if need:
                pgemm.ensure_workspace(need, stream)

    def launcher(variant, s):
        f = getattr(L, names[variant])

        def call():
            t, _, _ = operands()
            st = f(ptrs[t][0], ptrs[t][1], optr, M, N, K, s, sptr)
            if st != 0:
                raise pgemm.PgemmError(st, names[variant])
            return t
        return call

    sweep = {}
    if not args.timed_only:
        # bring the clocks to their sustained state before anything is timed
        time_launches(launcher(args.variant, 0), 30, stream)
    for variant, stage_set in () if args.timed_only else (("ws", (1, 2, 3, 4)), ("swap", (1, 2, 3, 4))):
        for s in stage_set:
            call = launcher(variant, s)
            # at least ten launches and about 4 ms of them, so that short
            # products are ranked on more than a few tens of microseconds
            est = time_launches(call, 3, stream)
            ms = time_launches(call, max(10, int(4.0 / max(est, 1e-3))), stream)
            sweep[f"{variant} S={s}"] = round(flops / (ms * 1e-3) / 1e12, 1)
            log(f"[bench] sweep {variant} S={s}: {ms * 1e3:.1f} us, {sweep[f'{variant} S={s}']} TFLOP/s")
    stages = args.stages
    if stages == 0 and args.timed_only:
        stages = pgemm.pgemm_query("nt_" + args.variant, 0, M, N, K)["stages"]
    elif stages == 0:
        cands = {k: v for k, v in sweep.items() if k.startswith(args.variant + " ")}
        stages = int(max(cands, key=cands.get).split("S=")[1])
    timed = launcher(args.variant, stages)
    last = [0]

    def step():
        last[0] = timed()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps of {args.variant} S={stages}")
    t0 = time.perf_counter()
    kern_ms = time_launches(step, args.steps, stream)
    t1 = time.perf_counter()
    wall = t1 - t0
    if pgemm.pgemm_debug_status() != 0:
        raise RuntimeError("a credit wait gave up during the timed region")
    value = flops * args.steps / wall / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    want_power = (args.power or not args.timed_only) and not args.no_power
    power = sample_power(1.0, step, stream) if want_power else None
    # single launches, each between its own pair of events (they include the
    # event overhead and a launch from idle): median, min and p90
    n_single = 0 if args.timed_only else (200 if kern_ms < 0.05 else 20)
    single = sorted(time_launches(step, 1, stream) for _ in range(n_single))
    single_us = {"median": round(single[n_single // 2] * 1e3, 2), "min": round(single[0] * 1e3, 2),
                 "p90": round(single[(9 * n_single) // 10] * 1e3, 2), "launches": n_single} if single else None

    # the vendor library on the same operands and stream, for context:
    # torch.matmul (f16) or torch.mm (bf16: a plain 2-D product, not a
    # batched one) with the K-contiguous rhs as a transposed view, into the
    # same preallocated output, timed after our own timed region in three
    # alternating rounds,
    # medians reported.  In each round either side first runs untimed for
    # about two milliseconds: ten launches of a 0.1 ms product right after
    # the other side's ran measurably slower (the clock settles to each
    # kernel's power draw in about a millisecond).
    if fmt == "f16":
        call_name = "torch.matmul (hipBLASLt)"

        def ref_call():
            t, a_, b_ = operands()
            torch.matmul(a_, b_.t(), out=out)
    else:
        call_name = "torch.mm (hipBLASLt)"

        def ref_call():
            t, a_, b_ = operands()
            torch.mm(a_, b_.t(), out=out)
    settle = max(3, int(2.0 / max(kern_ms, 1e-3)))
    ref_ms, ours_ms = [], []
    for _ in range(0 if args.timed_only else 3):
        time_launches(ref_call, settle, stream)
        ref_ms.append(time_launches(ref_call, 10, stream))
        time_launches(step, settle, stream)
        ours_ms.append(time_launches(step, 10, stream))
    reference = None
    if ref_ms:
        ms_ref, ms_ours = float(np.median(ref_ms)), float(np.median(ours_ms))
        reference = {"call": call_name, "tflops": round(flops / (ms_ref * 1e-3) / 1e12, 1),
                     "ours_alternating_tflops": round(flops / (ms_ours * 1e-3) / 1e12, 1)}
        reference["ours_over_reference"] = round(ms_ref / ms_ours, 3)
        log(f"[bench] {call_name}: {ms_ref * 1e3:.1f} us, {reference['tflops']} TFLOP/s; ours alternating "
            f"with it {reference['ours_alternating_tflops']} TFLOP/s")

    kname = "nt_ws_kernel" if args.variant == "ws" else "nt_swap_kernel"
    traffic = recorded_traffic(kname, args.workload, stages)
    result = {
        "metric": "TFLOP/s (and % of MFMA peak) for f16 NT GEMM 8192^3, 1 MI355X"
        if args.workload == "f16_nt_8192" else f"TFLOP/s for {fmt} NT GEMM {M}x{N}x{K}, 1 MI355X",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fmt,
        "data": "synthetic",
        "config": {
            "workload": f"{fmt} NT GEMM M={M} N={N} K={K}, operands "
                        f"{'uniform[-1,1)' if fmt == 'f16' else 'normal(0,1)'}, fp32 accumulation, "
                        f"{'producer/consumer credits' if args.variant == 'ws' else 'single-schedule swap'}",
            "M": M, "N": N, "K": K,
            "variant": args.variant,
            "stages": stages,
            "tile": pgemm.pgemm_query("nt_" + args.variant, stages, M, N, K)["block_m"],
            "pct_of_mfma_peak": round(100.0 * value / PEAK_F16_TFLOPS, 1),
            "stage_sweep_tflops": sweep,
            "single_launch_us": single_us,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_F16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": kname,
            "kernel_avg_us": round(kern_ms * 1e3, 2),
        },
    }
    if reference:
        result["reference_library"] = reference
    if power:
        result["power"] = power
    if args.workload == "f16_nt_skinny":
        alg_bytes = (M * K + N * K + M * N) * 2
        achieved_gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
        result["roofline"].update({
            "bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved_gbs / PEAK_HBM_GBS, 4)})
    if args.workload == "f16_nt_skinny" and not args.timed_only:
        # what a plain device copy moves on this machine (read + write bytes per
        # second), beside the nominal 8 TB/s
        n = 512 << 20
        src = torch.ones(n // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        copy = lambda: dst.copy_(src)
        time_launches(copy, 3, stream)
        copy_ms = time_launches(copy, 5, stream)
        copy_gbs = 2 * n / (copy_ms * 1e-3) / 1e9
        result["roofline"]["measured_copy"] = {"bytes": 2 * n, "gbs": round(copy_gbs, 1),
                                               "frac_of_copy": round(achieved_gbs / copy_gbs, 4)}
        del src, dst
    if not args.no_cpu_baseline and not args.timed_only:
        log("[bench] timing the CPU oracle on a sample of the same product")

        def gpu_rows(rows):
            # the timed call once more (the vendor rounds wrote `out` since),
            # until it has run on the first operand set
            step()
            while last[0] != 0:
                step()
            torch.cuda.synchronize()
            return out[:rows].view(torch.int16).cpu().numpy().view(np.uint16)

        result["cpu_baseline"] = cpu_baseline(fmt, A, B, M, N, K, args.cpu_budget, gpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
