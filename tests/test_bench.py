"""bench.py's command-line contract: one JSON line with the fields the
measurement plan names, one GPU only."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run_bench(*args, timeout=150):
    return subprocess.run([sys.executable, "-u", BENCH, *args], cwd=ROOT, capture_output=True, text=True,
                          timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def json_line(r):
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


COMMON = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
          "vs_baseline", "dtype", "data", "config", "roofline"}


@pytest.mark.gpu
def test_int32_workload_line():
    j = json_line(run_bench("--workload", "s32_nn_128x256x256", "--steps", "20", "--warmup", "3",
                            "--cpu-budget", "1"))
    assert COMMON <= set(j)
    assert j["unit"] == "GOP/s" and j["dtype"] == "int32" and j["n_gpus"] == 1 and j["steps"] == 20
    assert j["value"] > 0 and j["vs_baseline"] is None
    lat = j["config"]["single_launch_us"]
    assert 0 < lat["min"] <= lat["median"] <= lat["p90"]
    roof = j["roofline"]
    assert roof["bound"] == "alu" and roof["unit"] == "TOP/s" and 0 < roof["frac"] < 1
    assert j["cpu_baseline"]["kind"] == "oracle" and j["cpu_baseline"]["value"] > 0
    # the oracle's result, compared bit for bit with the timed output
    assert j["cpu_baseline"]["parity"] == {"elements": 128 * 256, "mismatches": 0}


@pytest.mark.gpu
def test_ragged_workload_line():
    j = json_line(run_bench("--workload", "bf16_nt_ragged", "--steps", "20", "--warmup", "3", "--cpu-budget", "1"))
    assert COMMON <= set(j)
    assert j["unit"] == "TFLOP/s" and j["dtype"] == "bf16" and j["config"]["variant"] == "ws"
    # the oracle's sampled rows, compared with the library's same rows
    cpu = j["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["parity"]["violations"] == 0
    assert cpu["parity"]["elements"] >= 2 * 1000 and cpu["parity"]["elements"] % 1000 == 0
    lat = j["config"]["single_launch_us"]
    assert lat["launches"] == 200 and 0 < lat["min"] <= lat["median"] <= lat["p90"]
    assert set(j["config"]["stage_sweep_tflops"]) == {f"{v} S={s}" for v in ("ws", "swap") for s in (1, 2, 3, 4)}
    roof = j["roofline"]
    assert roof["bound"] == "mfma" and 0 < roof["frac"] < 1 and roof["kernel"] == "nt_ws_kernel"
    assert roof["achieved"] > 0 and roof["kernel_avg_us"] > 0
    ref = j["reference_library"]
    assert ref["call"].startswith("torch.mm") and ref["tflops"] > 0



def test_kernel_hash_ignores_comments_only(tmp_path):
    # the traffic record stays valid across comment edits, not code edits
    sys.path.insert(0, ROOT)
    import bench
    csrc = os.path.join(ROOT, "software_pipelined_tiled_pipeline_amd", "csrc")
    for name in bench.KERNEL_SOURCES:
        (tmp_path / name).write_text(open(os.path.join(csrc, name), encoding="utf-8").read(), encoding="utf-8")
    base = bench.kernel_source_hash(str(tmp_path))
    assert base == bench.kernel_source_hash()
    k = tmp_path / "kernels.hpp"
    text = k.read_text(encoding="utf-8")
    k.write_text("// a new comment\n\n" + text.replace("\n", "  // trailing\n", 3) + "\n/* block\n comment */\n",
                 encoding="utf-8")
    assert bench.kernel_source_hash(str(tmp_path)) == base
    k.write_text(text + "\nconstexpr int kCodeChange = 1;\n", encoding="utf-8")
    assert bench.kernel_source_hash(str(tmp_path)) != base


# ------------------------------------------------------------------------
# The reductions that turn rocprofv3 CSV output into the tables and the
# traffic record under profiles/, on small synthetic files whose expected
# figures are worked out by hand.

WS_NAME = "_ZN5pgemm12nt_ws_kernelIDF16_NS_6NtGeomILi256ELi256ELi32ELi4ELi2ELi4ELi4ELi1EEELb0ELb0EEEvPKtS4_PtiiiiiiiPfijiPj"
SPLIT_NAME = "_ZN5pgemm12nt_ws_kernelIDF16_NS_6NtGeomILi128ELi128ELi64ELi3ELi2ELi2ELi2ELi1EEELb1ELb0EEEvPKtS4_PtiiiiiiiPfijiPj"
RED_NAME = "_ZN5pgemm13reduce_splitsIDF16_EEvPKfPtiiii"
COPY_NAME = "__amd_rocclr_copyBuffer"


def write_trace(d, rows):
    """rows: (kernel name, start ns, end ns)"""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w") as f:
        f.write('"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for i, (name, s, e) in enumerate(rows, 1):
            f.write(f'"KERNEL_DISPATCH",{i},"{name}",{s},{e}\n')


def write_counters(d, rows):
    """rows: (dispatch id, kernel name, start ns, end ns, counter, value); a
    counter may appear on several rows of one dispatch (its instances)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
        for disp, name, s, e, c, v in rows:
            f.write(f'{disp},"{name}","{c}",{v},{s},{e}\n')


def test_kernel_labels():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.kernel_label(WS_NAME) == "nt_ws_kernel f16 256x256x32 S=4"
    assert bench.kernel_label(SPLIT_NAME) == "nt_ws_kernel f16 128x128x64 S=3 split"
    assert bench.kernel_label(RED_NAME) == "reduce_splits f16"
    assert bench.kernel_label(COPY_NAME) == COPY_NAME


def test_summarize_trace_and_counters(tmp_path):
    d = str(tmp_path / "run")
    # three dispatches of 800, 820 and 840 us, then a copy kernel
    write_trace(d, [(WS_NAME, 0, 800_000), (WS_NAME, 1_000_000, 1_820_000), (WS_NAME, 2_000_000, 2_840_000),
                    (COPY_NAME, 3_000_000, 3_002_000)])
    # one dispatch of 1000 us: GRBM_GUI_ACTIVE over 8 XCDs = 1.6e6 cycles each
    # (1.6 GHz), MFMA busy cycles summed over two instances = 0.75 of 1024
    # SIMDs x 1.6e6
    busy = 0.75 * 1024 * 1.6e6
    write_counters(d, [(1, WS_NAME, 0, 1_000_000, "GRBM_GUI_ACTIVE", 8 * 1.6e6),
                       (1, WS_NAME, 0, 1_000_000, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2),
                       (1, WS_NAME, 0, 1_000_000, "SQ_VALU_MFMA_BUSY_CYCLES", busy / 2)])
    r = run_bench("--summarize", d, "--steps", "2", timeout=60)
    assert r.returncode == 0, r.stderr
    rows = {l.split("|")[1].strip(): [c.strip() for c in l.split("|")[2:-1]]
            for l in r.stdout.splitlines() if l.startswith("| nt_") or l.startswith("| __amd")}
    trace = [l for l in r.stdout.splitlines() if l.startswith("| nt_ws_kernel")]
    # trace row: dispatches, mean, min, max, mean of the last two
    assert trace[0].split("|")[2:7] == [" 3 ", " 820.00 ", " 800.00 ", " 840.00 ", " 830.00 "]
    # counter row: ..., sclk 1.600, MFMA busy 75.0 %
    assert trace[1].rstrip(" |").endswith("| 1.600 | 75.0 %")
    assert rows[COPY_NAME][0] == "1"


def test_traffic_reduction(tmp_path):
    # a 512 MiB device copy reads FETCH_SIZE = 262144 KiB and writes
    # WRITE_SIZE = 524288 KiB: read scale 2, write scale 1
    cf, cw = str(tmp_path / "cf"), str(tmp_path / "cw")
    write_counters(cf, [(1, COPY_NAME, 0, 1, "FETCH_SIZE", 131072), (1, COPY_NAME, 0, 1, "FETCH_SIZE", 131072)])
    write_counters(cw, [(1, COPY_NAME, 0, 1, "WRITE_SIZE", 524288)])
    # two timed calls of a K-split product, each a GEMM dispatch and a
    # reduction, after one warm-up call that must be left out
    kf, kw = str(tmp_path / "kf"), str(tmp_path / "kw")
    seq = [(SPLIT_NAME, 999, 999), (RED_NAME, 999, 999), (SPLIT_NAME, 100_000, 8_000), (RED_NAME, 20_000, 2_000),
           (SPLIT_NAME, 102_000, 8_200), (RED_NAME, 20_000, 1_800)]
    write_counters(kf, [(i, n, 0, 1, "FETCH_SIZE", f) for i, (n, f, _) in enumerate(seq, 1)])
    write_counters(kw, [(i, n, 0, 1, "WRITE_SIZE", w) for i, (n, _, w) in enumerate(seq, 1)])
    r = run_bench("--traffic", kf, kw, cf, cw, "--workload", "f16_nt_skinny", "--variant", "ws", "--stages", "3",
                  "--steps", "2", timeout=60)
    assert r.returncode == 0, r.stderr
    line = [l for l in r.stdout.splitlines() if l.startswith("traffic ")]
    assert len(line) == 1
    # per call: fetch (100000 + 20000 + 102000 + 20000) / 2 KiB x 1024 x 2,
    # write (8000 + 2000 + 8200 + 1800) / 2 KiB x 1024 x 1
    expect = int(121000 * 1024 * 2 + 10000 * 1024)
    assert line[0].startswith("traffic nt_ws_kernel f16_nt_skinny S=3 src=")
    assert line[0].endswith(f"bytes={expect}")
