"""Host-side measurement plumbing of bench.py (no GPU): the one-GPU guard, the HBM
traffic derived from rocprofv3 counter files, and the rule that a stored traffic
figure is only reported for the kernel source it was measured on."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def write_counters(directory, rows):
    """rows: (dispatch id, kernel name, counter, value) as rocprofv3 writes them."""
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout.strip() == ""                     # no JSON line


def test_traffic_summary_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    kib_copy = bench.COPY_BYTES // 1024
    # the copy kernel: FETCH_SIZE reads half the bytes it moves, WRITE_SIZE all of them;
    # a dispatch's value is the sum of its rows (one per XCD, say)
    write_counters(tmp_path / "cf", [(7, "elementwise_copy", "FETCH_SIZE", kib_copy / 4)] * 2)
    write_counters(tmp_path / "cw", [(7, "elementwise_copy", "WRITE_SIZE", kib_copy)])
    # three dispatches of the measured kernel: the median one counts; another kernel is ignored
    write_counters(tmp_path / "af", [(1, "attn_fwd_kernel<128>", "FETCH_SIZE", 900.0),
                                     (2, "attn_fwd_kernel<128>", "FETCH_SIZE", 1000.0),
                                     (3, "attn_fwd_kernel<128>", "FETCH_SIZE", 5000.0),
                                     (4, "other_kernel", "FETCH_SIZE", 1e9)])
    write_counters(tmp_path / "aw", [(1, "attn_fwd_kernel<128>", "WRITE_SIZE", 250.0),
                                     (1, "attn_fwd_kernel<128>", "WRITE_SIZE", 250.0)])
    bench.traffic_summary(str(tmp_path / "af"), str(tmp_path / "aw"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                          "wl", 1)
    entry = json.loads(traffic.read_text())["wl-causal1"]
    assert entry["fetch_scale"] == 2.0 and entry["write_scale"] == 1.0
    assert entry["read_bytes"] == 1000 * 1024 * 2
    assert entry["written_bytes"] == 500 * 1024
    assert entry["bytes_per_launch"] == 1000 * 1024 * 2 + 500 * 1024
    assert entry["source_sha256_16"] == bench.source_hash()


def test_stored_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\nint f() { return 1; }\n")
    traffic = tmp_path / "traffic.json"
    traffic.write_text(json.dumps({"wl-causal1": {"bytes_per_launch": 1234,
                                                  "source_sha256_16": bench.source_hash(str(src))}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    assert bench.measured_traffic("wl", 1, source=str(src)) == 1234
    # other workloads or masks have no entry
    assert bench.measured_traffic("wl", 0, source=str(src)) is None
    assert bench.measured_traffic("wl2", 1, source=str(src)) is None
    # a comment or whitespace edit keeps the figure
    src.write_text("// the same kernel, reworded\nint f()  {  return 1; }\n")
    assert bench.measured_traffic("wl", 1, source=str(src)) == 1234
    # a code change drops it
    src.write_text("// a kernel\nint f() { return 2; }\n")
    assert bench.measured_traffic("wl", 1, source=str(src)) is None


def test_the_flags_a_source_alone_is_compiled_with_are_part_of_its_hash(tmp_path, monkeypatch):
    import exact_tiled_attention_03_amd.build as build
    assert build.source_flags(bench.KERNEL_SOURCE) == ("-Xarch_device", "-fno-honor-nans")
    assert build.source_flags(bench.SOFTMAX_SOURCE) == () and build.source_flags(bench.BWD_SOURCE) == ()
    src = tmp_path / "attn_fwd.hip"
    src.write_text("int f() { return 1; }\n")
    flagged = bench.source_hash(str(src))
    monkeypatch.setattr(build, "SOURCE_FLAGS", {})
    assert bench.source_hash(str(src)) != flagged
