"""bench.py end to end on the GPU, one short run per mode in a child process (as
the benchmark is run): each prints exactly one JSON line carrying the fields of
the benchmark contract, with consistent figures (value and roofline.achieved are
the same throughput, frac = achieved / peak, a positive step time), and the
fields that say what ran (entry point, workspace, cache state, bound, unit).
Runs that time the float64 oracle on the host also re-check the timed output
against it: the CPU baseline block names the oracle, its sample and its cores."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COMMON = ["--steps", "3", "--warmup", "2", "--no-clock"]
CONTRACT = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
            "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline")
ROOFLINE = ("bound", "achieved", "peak", "unit", "frac", "traffic")
C2 = ["--workload", "causal_b4_h16_n1024_d64_fp16", "--causal", "1"]
C5 = ["--workload", "ragged_b3_h8_n3000_d80_fp16", "--causal", "0"]


def run(args):
    print(f"\n[case] bench.py {' '.join(args)}", flush=True)
    p = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *COMMON, *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, p.stdout[-3000:]
    line = json.loads(lines[0])
    for key in CONTRACT:
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["warmup"] == 2
    assert line["higher_is_better"] is True and line["scaling"] == "weak" and line["vs_baseline"] is None
    assert line["ms_per_step"] > 0 and line["value"] > 0 and "workload" in line["config"]
    r = line["roofline"]
    for key in ROOFLINE:
        assert key in r, key
    assert r["unit"] == line["unit"]
    assert r["achieved"] == pytest.approx(line["value"], rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert 0 < r["frac"] < 1
    assert r["traffic"] is None or r["traffic"] > 0
    return line


def check_cpu_baseline(line):
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["unit"] == line["unit"]
    return cb


def test_headline_with_the_oracle_baseline(lib):
    line = run(["--cpu-seconds", "2"])
    cfg = line["config"]
    assert (cfg["workload"], cfg["entry"], cfg["l2"], cfg["workspace_bytes"]) == \
        ("causal_b2_h32_n4096_d128_bf16", "attn_fwd", "warm", 0)
    assert line["dtype"] == "bf16" and line["unit"] == "TFLOP/s" and line["roofline"]["bound"] == "mfma"
    assert line["roofline"]["peak"] == pytest.approx(2516.6)
    parity = check_cpu_baseline(line)["parity_of_timed_output"]
    assert parity["max_abs"] <= 1e-2 and parity["lse_max_abs"] <= 1e-3


def test_sliding_window(lib):
    line = run(C2 + ["--window", "256", "--no-cpu-baseline"])
    cfg = line["config"]
    assert cfg["entry"] == "attn_fwd_window" and cfg["window"] == 256 and cfg["workload"].endswith("-window256")
    assert line["cpu_baseline"] is None


def test_key_range_parts_and_the_plain_entry(lib):
    ws = run(C5 + ["--no-cpu-baseline"])
    plain = run(C5 + ["--no-cpu-baseline", "--entry", "attn_fwd"])
    assert ws["config"]["entry"] == "attn_fwd_ws" and ws["config"]["workspace_bytes"] > 0
    assert plain["config"]["entry"] == "attn_fwd" and plain["config"]["workspace_bytes"] == 0
    assert ws["dtype"] == plain["dtype"] == "fp16"


def test_cold_caches(lib):
    line = run(C2 + ["--cold-l2", "--no-cpu-baseline"])
    assert line["config"]["l2"] == "cold" and line["roofline"]["traffic"] is None


def test_backward(lib):
    line = run(C2 + ["--backward", "--cpu-seconds", "1"])
    assert line["config"]["workload"].endswith("-backward") and line["roofline"]["bound"] == "mfma"
    check_cpu_baseline(line)


def test_merge(lib):
    line = run(C2 + ["--merge", "3", "--cpu-seconds", "1"])
    assert line["unit"] == "GB/s" and line["roofline"]["bound"] == "hbm" and line["config"]["G"] == 3
    check_cpu_baseline(line)


def test_gemm(lib):
    line = run(["--workload", "gemm_kn_m4096_n4096_k4096_fp16_relu", "--cpu-seconds", "1"])
    assert line["unit"] == "TFLOP/s" and line["roofline"]["bound"] == "mfma" and line["dtype"] == "fp16"
    check_cpu_baseline(line)


def test_row_softmax(lib):
    line = run(["--workload", "softmax_rows4096_cols32768_bf16", "--cpu-seconds", "1"])
    assert line["unit"] == "GB/s" and line["roofline"]["bound"] == "hbm" and line["dtype"] == "bf16"
    check_cpu_baseline(line)
