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
