"""Benchmark of the fused exact-attention forward on one MI355X.

One step = one attn_fwd call over the whole workload (default: causal
B=2 H=32 N=4096 d=128 bf16), inputs resident in HBM before timing starts.
Prints ONE JSON line: TFLOP/s (4*B*H*N^2*d, halved for causal) with the
roofline of the kernel against the dense bf16/fp16 MFMA peak and the CPU
oracle's throughput on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--causal 0|1]
                    [--window W] [--no-cpu-baseline] [--cpu-seconds S]

--window W times attn_fwd_window (sliding window, key j kept for query i only if
i - W < j, and j < i + W when not causal) and credits 4*d FLOPs per kept pair.

--workload softmax_rows4096_cols32768_f32 (or another softmax workload) times the
standalone row softmax instead: effective bandwidth in GB/s, counting x read
once and y written once, against the 8 TB/s HBM roofline.

--backward times attn_bwd (dQ, dK, dV from the saved lse) on the attention
workload, crediting 2.5x the forward's FLOPs (the five N x N x d products of
the backward; recomputing S and dP in the dQ kernel is not credited).

--merge G times attn_lse_merge combining G key shards of the attention workload's
shape (o_parts [G, B, H, N, d], lse_parts [G, B, H, N]): effective bandwidth in
GB/s counting every part read once and the result written once, against the
8 TB/s HBM roofline.

--workload gemm_qkv_m8192_n12288_k4096_bf16 (or another gemm workload) times the
matrix product with its fused bias + activation epilogue: TFLOP/s counting
2*M*N*K, against the dense bf16/fp16 MFMA peak.

Warm-up: W untimed steps (default 100), continued until at least 0.25 s of
warm-up has passed so that the K timed steps see a settled GPU clock (a cold
start measured ~10% slower); the JSON line's warmup_detail says what was run.

Traffic calibration (run each under rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE):
    python bench.py --copy-calibration          # plain 256 MiB copy kernel, known bytes
    python bench.py --traffic-summary ATTN_FETCH ATTN_WRITE COPY_FETCH COPY_WRITE
        reads the four rocprofv3 output directories and writes profiles/traffic.json
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak, causal N=4096 d=128"
METRIC_BWD = "attention bwd TFLOP/s (2.5x the forward's 4*B*H*N^2*d, halved for causal) and % of bf16 MFMA peak"
METRIC_WINDOW = "sliding-window attention fwd TFLOP/s (4*d per kept query-key pair) and % of bf16 MFMA peak"
METRIC_SOFTMAX = "row softmax effective bandwidth GB/s (x read once + y written once)"
METRIC_MERGE = "key-shard merge effective bandwidth GB/s (G partial O and lse read once, merged O and lse written once)"
MFMA_PEAK_TFLOPS = 2516.6      # dense fp16/bf16: 256 CU x 4096 FLOP/clk x 2.4 GHz (the 2.5 PFLOP/s figure)
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
KERNEL_SOURCE = os.path.join(ROOT, "exact_tiled_attention_03_amd", "csrc", "attn_fwd.hip")
SOFTMAX_SOURCE = os.path.join(ROOT, "exact_tiled_attention_03_amd", "csrc", "softmax_rows.hip")
GEMM_SOURCE = os.path.join(ROOT, "exact_tiled_attention_03_amd", "csrc", "gemm.hip")
BWD_SOURCE = os.path.join(ROOT, "exact_tiled_attention_03_amd", "csrc", "attn_bwd.hip")
MERGE_SOURCE = os.path.join(ROOT, "exact_tiled_attention_03_amd", "csrc", "lse_merge.hip")
BWD_KERNELS = ("attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel")
METRIC_GEMM = "GEMM + bias + activation TFLOP/s (2*M*N*K) and % of bf16 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_hash(path: str = KERNEL_SOURCE) -> str:
    """Hash of a kernel source's code and of the flags it alone is compiled with:
    comments and whitespace are dropped, so that editing a comment does not
    invalidate counters taken on the same code."""
    import re
    from exact_tiled_attention_03_amd.build import source_flags
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split() + list(source_flags(path)))
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def traffic_key(workload: str, causal, window: int = 0) -> str:
    """Attention entries carry their mask (causal flag, window); the softmax has none."""
    if causal is None:
        return workload
    return f"{workload}-causal{causal}" + (f"-window{window}" if window > 0 else "")


def measured_traffic(workload: str, causal: int, window: int = 0, source: str = KERNEL_SOURCE, key=None):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when
    absent or when the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(key or traffic_key(workload, causal, window))
    if not entry or entry.get("source_sha256_16") != source_hash(source):
        return None
    return entry.get("bytes_per_launch")


COPY_BYTES = 256 << 20


def copy_calibration(steps: int):
    """A plain device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES) per launch."""
    import torch
    src = torch.randn(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "launches": steps}))


def _pmc_kib_per_dispatch(directory: str, counter: str, kernel_substr: str) -> float:
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for '{kernel_substr}' under {directory}")
    return statistics.median(vals.values())


def _has_kernel(directory: str, kernel_substr: str) -> bool:
    import csv
    import glob
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        if any(kernel_substr in r["Kernel_Name"] for r in csv.DictReader(open(f))):
            return True
    return False


def traffic_summary(attn_fetch, attn_write, copy_fetch, copy_write, workload, causal, window=0,
                    kernel_substr="attn_fwd_kernel", source=KERNEL_SOURCE, key=None):
    """HBM bytes per kernel launch: FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by
    the ratio of known bytes to what the same counter reads for the plain copy kernel.
    kernel_substr may be a tuple: the entry is then the sum over those kernels (the
    kernels of one entry-point call)."""
    f_copy = _pmc_kib_per_dispatch(copy_fetch, "FETCH_SIZE", "elementwise") * 1024
    w_copy = _pmc_kib_per_dispatch(copy_write, "WRITE_SIZE", "elementwise") * 1024
    names = kernel_substr if isinstance(kernel_substr, tuple) else (kernel_substr,)
    f_attn = sum(_pmc_kib_per_dispatch(attn_fetch, "FETCH_SIZE", n) for n in names) * 1024
    w_attn = sum(_pmc_kib_per_dispatch(attn_write, "WRITE_SIZE", n) for n in names) * 1024
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    entry = {"bytes_per_launch": round(f_attn * f_scale + w_attn * w_scale),
             "read_bytes": round(f_attn * f_scale), "written_bytes": round(w_attn * w_scale),
             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
             "raw_fetch_kib": f_attn / 1024, "raw_write_kib": w_attn / 1024,
             "source_sha256_16": source_hash(source)}
    if len(names) > 1:
        entry["per_kernel"] = {n: {"read_bytes": round(_pmc_kib_per_dispatch(attn_fetch, "FETCH_SIZE", n) * 1024 * f_scale),
                                   "written_bytes": round(_pmc_kib_per_dispatch(attn_write, "WRITE_SIZE", n) * 1024 * w_scale)}
                               for n in names}
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    key = key or traffic_key(workload, causal, window)
    table[key] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(json.dumps({key: entry}))


SETTLE_S = 0.25   # minimum untimed warm-up time: the GPU clock ramps up over the first ~100 ms of load


def warm_up(call, steps: int) -> dict:
    """Run `steps` untimed warm-up steps, then keep going until SETTLE_S seconds of
    warm-up have passed, so that the timed steps see a settled clock.  Returns what
    was done (reported in the JSON line)."""
    import torch
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(10):
            call()
        extra += 10
        torch.cuda.synchronize()
    return {"steps": steps, "extra_settle_steps": extra, "seconds": round(time.perf_counter() - t0, 3)}


class ClockUnderLoad:
    """The GPU clock and power while the timed kernel runs back to back.

    The driver's metrics table (amdsmi gpu metrics) is refreshed about once a
    second, so a few milliseconds of timed steps never show in it.  measure()
    keeps launching the same call after the timed steps until the table has
    been refreshed twice (the second refresh then covers a whole period of
    sustained load, at most ~3 s) and reports that snapshot: the graphics clock
    of every XCD (MHz) and the socket power (W)."""

    def __init__(self):
        self.error = None
        self._h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                raise RuntimeError("amdsmi sees no GPU")
            self._amdsmi, self._h = amdsmi, handles[0]
            self._read()
        except Exception as e:   # the clock is context; its absence must not stop the benchmark
            self.error = f"{type(e).__name__}: {e}"
            self._h = None

    def _read(self):
        return self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)

    def measure(self, call, max_s: float = 3.0) -> dict:
        if self._h is None:
            return {"median_mhz": None, "error": self.error}
        import torch
        try:
            stamp = self._read().get("system_clock_counter")
            refreshes, snap, t0 = 0, None, time.perf_counter()
            while refreshes < 2 and time.perf_counter() - t0 < max_s:
                for _ in range(4):
                    call()
                torch.cuda.synchronize()
                m = self._read()
                if m.get("system_clock_counter") != stamp:
                    stamp, refreshes, snap = m.get("system_clock_counter"), refreshes + 1, m
            if refreshes < 2:
                return {"median_mhz": None, "error": "metrics table not refreshed twice under load"}
            clks = [float(c) for c in (snap.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
            if not clks and isinstance(snap.get("current_gfxclk"), (int, float)):
                clks = [float(snap["current_gfxclk"])]
            power = snap.get("current_socket_power")
            return {"median_mhz": round(statistics.median(clks), 1) if clks else None,
                    "per_xcd_mhz": clks, "socket_power_w": power if isinstance(power, (int, float)) else None,
                    "source": "amdsmi gpu metrics (current_gfxclks, current_socket_power), the second table "
                              "refresh while the same launches ran back to back after the timed steps",
                    "seconds_under_load": round(time.perf_counter() - t0, 2)}
        except Exception as e:
            return {"median_mhz": None, "error": f"{type(e).__name__}: {e}"}


def time_steps(call, steps: int, stream) -> dict:
    """The K timed steps: one event before the first launch and one after the last,
    with a synchronize on both sides (ms_per_step = elapsed / K, nothing between the
    launches).  Each step is one call of the entry point, so ms_per_step is also the
    average launch duration the roofline divides by.  Then a separate loop of K
    launches, each between its own pair of events, for the spread of launch times
    (reported only: the event records between launches add a few microseconds to
    each one)."""
    import torch
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for _ in range(steps):
        call()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    return {"ms_per_step": total_ms / steps, "per_launch": per_launch, "launch_ms": statistics.mean(per_launch)}


COLD_L2_BYTES = 1 << 30   # written between cold-cache calls: past the 8 x 4 MB of L2 and the 256 MB Infinity Cache


def time_steps_cold(call, steps: int, stream, scratch) -> dict:
    """The K timed steps with cold caches: before each call the 1 GiB `scratch`
    buffer is overwritten (outside the timed region), so the call finds its
    inputs in HBM only.  Each call is timed between its own pair of events;
    ms_per_step is their mean (the event records add a few microseconds, as in
    time_steps' second loop)."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        scratch.fill_(i & 0xFF)
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    mean = statistics.mean(per_launch)
    return {"ms_per_step": mean, "per_launch": per_launch, "launch_ms": mean}


def launch_stats(t: dict) -> dict:
    pl = sorted(t["per_launch"])
    return {"launch_ms_mean": round(t["launch_ms"], 5), "launch_ms_median": round(statistics.median(pl), 5),
            "launch_ms_p95": round(pl[int(0.95 * (len(pl) - 1))], 5), "launch_ms_min": round(pl[0], 5)}


def kept_pairs(n: int, causal: int, window: int, rows=None) -> float:
    """Number of (query, key) pairs the mask keeps in one head (for the given query
    rows, default all): key j is kept for query i when j <= i (causal) and, with a
    window W >= 1, i - W < j (and j < i + W when not causal)."""
    import numpy as np
    i = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros_like(i)
    if causal:
        hi = i
    else:
        hi = np.minimum(n - 1, i + window - 1) if window > 0 else np.full_like(i, n - 1)
    return float((hi - lo + 1).sum())


def launch_flops(w, causal: int, window: int) -> float:
    """FLOPs credited to one launch: 4*B*H*N^2*d, halved when causal (the metric's
    convention); with a window, 4*d per kept (query, key) pair."""
    if window <= 0:
        return w.flops(causal)
    return 4.0 * w.d * w.B * w.H * kept_pairs(w.N, causal, window)


def cpu_baseline(w, causal, q, k, v, out, lse, budget_s: float, window: int = 0):
    """Time the float64 oracle on whole heads of the same workload until ~budget_s
    of CPU work; also re-check the GPU output of those heads against it."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
        oc, lc = out.cpu().double().numpy(), lse.cpu().double().numpy()
        flops_per_head = launch_flops(w, causal, window) / (w.B * w.H)
        heads, t0, max_err, lse_err = 0, time.perf_counter(), 0.0, 0.0
        rows = None
        if w.N > 8192:   # long sequences: the oracle's rows are sampled per head
            rows = np.sort(np.random.default_rng(w.seed + 11).choice(w.N, 256, replace=False))
        for idx in range(w.B * w.H):
            b, h = divmod(idx, w.H)
            O, L = oracle.attention(qc[b:b + 1, h:h + 1], kc[b:b + 1, h:h + 1], vc[b:b + 1, h:h + 1],
                                    causal, w.scale, rows=rows, window=window)
            sel = slice(None) if rows is None else rows
            max_err = max(max_err, float(np.abs(oc[b, h][sel] - O[0, 0]).max()))
            lse_err = max(lse_err, float(np.abs(lc[b, h][sel] - L[0, 0]).max()))
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    if rows is None:
        flops = heads * flops_per_head
        sample = f"{heads} of {w.B * w.H} heads, all {w.N} rows each"
    else:
        # rows cost in proportion to their kept key count
        keys = kept_pairs(w.N, causal, window, rows) if window > 0 else ((rows + 1).sum() if causal else len(rows) * w.N)
        flops = heads * 4.0 * keys * w.d
        sample = f"{heads} of {w.B * w.H} heads, {len(rows)} seeded rows each"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3), "host_cpus": cores,
            "parity_of_timed_output": {"max_abs": max_err, "lse_max_abs": lse_err}}


def softmax_cpu_baseline(w, x, y, budget_s: float):
    """Time the float64 oracle on blocks of 16 rows of the same workload until ~budget_s
    of CPU work; also re-check the GPU output of those rows against it."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        rows, t_work, max_rel = 0, 0.0, 0.0
        while rows < w.rows and t_work < budget_s:
            xc, yc = x[rows:rows + 16].cpu(), y[rows:rows + 16].cpu().double().numpy()
            t0 = time.perf_counter()
            ref = oracle.softmax_rows(xc)
            t_work += time.perf_counter() - t0
            max_rel = max(max_rel, float((np.abs(yc - ref) / np.maximum(ref, 1e-300)).max()))
            rows += xc.shape[0]
    es = 4 if w.dtype == "f32" else 2
    return {"value": 2.0 * rows * w.cols * es / t_work / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle", "sample": f"{rows} of {w.rows} rows (blocks of 16), all {w.cols} columns each",
            "seconds": round(t_work, 3), "host_cpus": cores,
            "parity_of_timed_output": {"max_rel": max_rel}}


def bench_softmax(args, w):
    """One step = one softmax_rows call over the whole [rows, cols] workload."""
    import torch
    import attn_workloads as aw
    import exact_tiled_attention_03_amd as eta

    dev = torch.device("cuda:0")
    x = aw.make_rows(w.rows, w.cols, w.dtype, w.seed, w.sigma).to(dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    warm = warm_up(lambda: eta.softmax_rows(x, y, stream=stream), args.warmup)
    t = time_steps(lambda: eta.softmax_rows(x, y, stream=stream), args.steps, stream)
    sclk = None if args.no_clock else ClockUnderLoad().measure(lambda: eta.softmax_rows(x, y, stream=stream))
    ms_per_step = t["ms_per_step"]
    nbytes = w.algorithmic_bytes()
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (ms_per_step * 1e-3) / 1e9
    kernel = "softmax_row_tiled_kernel" if w.cols > 65536 else "softmax_row_kernel"
    line = {
        "metric": METRIC_SOFTMAX,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_detail": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic (seeded iid N(0,{w.sigma:g}) x)",
        "config": {"workload": w.name, "rows": w.rows, "cols": w.cols, "layout": "[rows, cols] contiguous",
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2), **launch_stats(t), "sclk": sclk},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, None, 0, SOFTMAX_SOURCE),
                     "kernel": kernel, "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = softmax_cpu_baseline(w, x, y, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def gemm_cpu_baseline(w, a, b, bias, c, budget_s: float):
    """Time the float64 oracle on blocks of 8 rows of A (all of B) until ~budget_s of
    CPU work; also re-check the GPU output of those rows against it."""
    import numpy as np
    from oracle import gemm as og
    from threadpoolctl import threadpool_info, threadpool_limits

    acts = {"none": og.ACT_NONE, "relu": og.ACT_RELU, "gelu_tanh": og.ACT_GELU_TANH}
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        bl = b.cpu() if w.b_layout == "kn" else b.cpu().t()
        bc = bias.cpu() if w.bias else None
        rows, t_work, max_err = 0, 0.0, 0.0
        while rows < w.M and t_work < budget_s:
            ac, cc = a[rows:rows + 8].cpu(), c[rows:rows + 8].cpu().double().numpy()
            t0 = time.perf_counter()
            ref = og.gemm_bias_act(ac, bl, bc, acts[w.act])
            t_work += time.perf_counter() - t0
            max_err = max(max_err, float(np.abs(cc - ref).max()))
            rows += ac.shape[0]
    return {"value": 2.0 * rows * w.N * w.K / t_work / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle", "sample": f"{rows} of {w.M} rows of A (blocks of 8) against all of B",
            "seconds": round(t_work, 3), "host_cpus": cores, "parity_of_timed_output": {"max_abs": max_err}}


def bench_gemm(args, w):
    """One step = one gemm_bias_act call over the whole workload."""
    import torch
    import attn_workloads as aw
    import exact_tiled_attention_03_amd as eta

    dev = torch.device("cuda:0")
    a, b, bias = (t.to(dev) for t in aw.gemm_workload_inputs(w))
    bias = bias if w.bias else None
    c = torch.empty((w.M, w.N), dtype=a.dtype, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        eta.gemm_bias_act(a, b, bias, w.act, w.b_layout, c=c, stream=stream)

    warm = warm_up(call, args.warmup)
    t = time_steps(call, args.steps, stream)
    sclk = None if args.no_clock else ClockUnderLoad().measure(call)
    ms_per_step = t["ms_per_step"]
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": METRIC_GEMM,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_detail": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1) A, N(0,1/K) B, N(0,1) bias)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "b_layout": w.b_layout, "act": w.act,
                   "bias": w.bias, "pct_of_mfma_peak": round(100 * value / MFMA_PEAK_TFLOPS, 2), **launch_stats(t),
                   "sclk": sclk},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(w.name, None, 0, GEMM_SOURCE),
                     "kernel": f"gemm_kernel<{w.dtype},{w.b_layout}>",
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": w.algorithmic_bytes()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = gemm_cpu_baseline(w, a, b, bias, c, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def bench_backward(args, w, causal):
    """One step = one attn_bwd call (delta, dQ and dK/dV kernels) over the whole workload."""
    import torch
    import attn_workloads as aw
    import exact_tiled_attention_03_amd as eta

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in aw.workload_inputs(w))
    do = aw.make_inputs(w.shape, w.dtype, w.seed + 500)[0].to(dev)
    out, lse = eta.attention(q, k, v, bool(causal), w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        eta.attn_bwd(q, k, v, out, lse, do, dq, dk, dv, delta, causal=bool(causal), scale=w.scale, stream=stream)

    warm = warm_up(call, args.warmup)
    t = time_steps(call, args.steps, stream)
    sclk = None if args.no_clock else ClockUnderLoad().measure(call)
    ms_per_step = t["ms_per_step"]
    flops = 2.5 * w.flops(causal)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": METRIC_BWD,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_detail": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1) Q, K, V, dO)",
        "config": {"workload": w.name + "-backward", "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal,
                   "scale": w.scale, "pct_of_mfma_peak": round(100 * value / MFMA_PEAK_TFLOPS, 2), **launch_stats(t),
                   "sclk": sclk, "note": "one step = the dQ (with D) and dK/dV kernels of one attn_bwd call"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(w.name, causal, 0, BWD_SOURCE, key=f"{w.name}-causal{causal}-backward"),
                     "kernel": " + ".join(BWD_KERNELS),
                     "algorithmic_flops_per_launch": flops},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = backward_cpu_baseline(w, causal, q, k, v, do, dq, dk, dv, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def bench_merge(args, w, G):
    """One step = one attn_lse_merge call over G shards of the workload's rows."""
    import numpy as np
    import torch
    import attn_workloads as aw
    import exact_tiled_attention_03_amd as eta
    from oracle import backward as ob

    dev = torch.device("cuda:0")
    # seeded synthetic shard results of the workload's shape: the merge's cost does not
    # depend on the values (o_parts iid N(0, 1) in the workload's type, lse_parts N(5, 2^2))
    rng = np.random.default_rng(w.seed + 900)
    shape = (G, w.B, w.H, w.N, w.d)
    o_parts = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(aw.DTYPES[w.dtype]).to(dev)
    l_parts = torch.from_numpy(5.0 + 2.0 * rng.standard_normal(shape[:4], dtype=np.float32)).to(dev)
    o = torch.empty(shape[1:], dtype=o_parts.dtype, device=dev)
    lse = torch.empty(shape[1:4], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        eta.attn_lse_merge(o_parts, l_parts, o, lse, stream=stream)

    warm = warm_up(call, args.warmup)
    t = time_steps(call, args.steps, stream)
    sclk = None if args.no_clock else ClockUnderLoad().measure(call)
    ms_per_step = t["ms_per_step"]
    rows = w.B * w.H * w.N
    nbytes = G * rows * (w.d * 2 + 4) + rows * (w.d * 2 + 4)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC_MERGE, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_detail": warm, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded shard results: O_g iid N(0,1), lse_g iid N(5,4))",
        "config": {"workload": f"{w.name}-merge{G}", "G": G, "rows": rows, "d": w.d,
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2), **launch_stats(t), "sclk": sclk},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, None, 0, MERGE_SOURCE, key=f"{w.name}-merge{G}"),
                     "kernel": "lse_merge_kernel",
                     "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0))
        sl = slice(0, 4)   # 4 heads of batch 0
        op = o_parts[:, 0, sl].cpu().double().numpy()
        lp = l_parts[:, 0, sl].cpu().double().numpy()
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            ro, rl = ob.lse_merge(op, lp)
            reps += 1
        dt = time.perf_counter() - t0
        err = float(np.abs(o[0, sl].cpu().double().numpy() - ro).max())
        sample_rows = 4 * w.N
        line["cpu_baseline"] = {"value": reps * (G + 1) * sample_rows * (w.d * 2 + 4) / dt / 1e9, "unit": "GB/s",
                                "cores": 1, "kind": "oracle",
                                "sample": f"{sample_rows} of {rows} rows (4 heads), {reps} repetitions",
                                "seconds": round(dt, 3), "host_cpus": cores,
                                "parity_of_timed_output": {"max_abs": err}}
    print(json.dumps(line), flush=True)


def backward_cpu_baseline(w, causal, q, k, v, do, dq, dk, dv, budget_s: float):
    """Time the float64 gradient oracle on whole heads until ~budget_s of CPU work; also
    re-check the GPU gradients of those heads against it."""
    import numpy as np
    from oracle import backward as ob
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        heads, t_work, max_err = 0, 0.0, 0.0
        for idx in range(w.B * w.H):
            b, h = divmod(idx, w.H)
            sl = (slice(b, b + 1), slice(h, h + 1))
            args_ = [t[sl].cpu() for t in (q, k, v, do)]
            t0 = time.perf_counter()
            ref = ob.attention_bwd(*args_, causal, w.scale)
            t_work += time.perf_counter() - t0
            for g, r in zip((dq, dk, dv), ref):
                max_err = max(max_err, float(np.abs(g[sl].cpu().double().numpy() - r).max()))
            heads += 1
            if t_work >= budget_s:
                break
    flops = 2.5 * w.flops(causal) / (w.B * w.H) * heads
    return {"value": flops / t_work / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads, all {w.N} rows each", "seconds": round(t_work, 3),
            "host_cpus": cores, "parity_of_timed_output": {"max_abs": max_err}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline workload)")
    ap.add_argument("--causal", type=int, default=None)
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window W >= 1 (attn_fwd_window); FLOPs then count kept pairs x 4d")
    ap.add_argument("--backward", action="store_true", help="time attn_bwd on the attention workload")
    ap.add_argument("--merge", type=int, default=0, help="time attn_lse_merge over this many key shards")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--entry", choices=["auto", "attn_fwd"], default="auto",
                    help="forward entry point: auto uses attn_fwd_ws where it splits the last round")
    ap.add_argument("--cold-l2", action="store_true",
                    help="forward only: overwrite a 1 GiB buffer before each timed call (L2 and Infinity Cache "
                         "cold), each call timed between its own events")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock-under-load window (for profiler runs, which time every dispatch)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-summary", nargs=4, metavar="DIR")
    args = ap.parse_args()

    if args.traffic_summary:
        import attn_workloads as aw
        if args.workload and args.workload.startswith("softmax_"):
            traffic_summary(*args.traffic_summary, args.workload, None, 0, "softmax_row", SOFTMAX_SOURCE)
            return
        if args.workload and args.workload.startswith("gemm_"):
            traffic_summary(*args.traffic_summary, args.workload, None, 0, "gemm_kernel", GEMM_SOURCE)
            return
        w = aw.by_name(args.workload) if args.workload else aw.WORKLOADS[aw.HEADLINE]
        causal = w.causal_modes[0] if args.causal is None else args.causal
        if args.backward:
            traffic_summary(*args.traffic_summary, w.name, causal, 0, BWD_KERNELS, BWD_SOURCE,
                            key=f"{w.name}-causal{causal}-backward")
        elif args.merge > 0:
            traffic_summary(*args.traffic_summary, w.name, None, 0, "lse_merge_kernel", MERGE_SOURCE,
                            key=f"{w.name}-merge{args.merge}")
        elif _has_kernel(args.traffic_summary[0], "lse_merge_kernel"):
            # an attn_fwd_ws run: the forward with key-range parts and the merge
            traffic_summary(*args.traffic_summary, w.name, causal, 0, ("attn_fwd_kernel", "lse_merge_kernel"),
                            key=traffic_key(w.name, causal) + "-ws")
        else:
            traffic_summary(*args.traffic_summary, w.name, causal, args.window)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(heads or query tiles would shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import torch
    import attn_workloads as aw
    import exact_tiled_attention_03_amd as eta

    if args.workload and args.workload.startswith("softmax_"):
        bench_softmax(args, aw.softmax_by_name(args.workload))
        return
    if args.workload and args.workload.startswith("gemm_"):
        bench_gemm(args, aw.gemm_by_name(args.workload))
        return
    w = aw.by_name(args.workload) if args.workload else aw.WORKLOADS[aw.HEADLINE]
    causal = w.causal_modes[0] if args.causal is None else args.causal
    if args.backward:
        bench_backward(args, w, causal)
        return
    if args.merge > 0:
        bench_merge(args, w, args.merge)
        return
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in aw.workload_inputs(w))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # attn_fwd_ws where it splits a partial last round of query tiles (its
    # workspace allocated here, outside the timed region), else attn_fwd
    ws_bytes = 0 if args.window > 0 or args.entry == "attn_fwd" else eta.attn_fwd_workspace_bytes(w.B, w.H, w.N, w.d, causal)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes > 0 else None
    entry = "attn_fwd_ws" if workspace is not None else ("attn_fwd_window" if args.window > 0 else "attn_fwd")

    def call():
        if workspace is not None:
            eta.attn_fwd_ws(q, k, v, out, lse, causal, w.scale, workspace, stream=stream)
        else:
            eta.attn_fwd(q, k, v, out, lse, causal, w.scale, stream=stream, window=args.window)

    warm = warm_up(call, args.warmup)
    if args.cold_l2:
        scratch = torch.empty(COLD_L2_BYTES, dtype=torch.uint8, device=dev)
        t = time_steps_cold(call, args.steps, stream, scratch)
    else:
        t = time_steps(call, args.steps, stream)
    sclk = None if args.no_clock else ClockUnderLoad().measure(call)
    ms_per_step = t["ms_per_step"]
    flops = launch_flops(w, causal, args.window)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (ms_per_step * 1e-3) / 1e12

    line = {
        "metric": METRIC if args.window <= 0 else METRIC_WINDOW,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_detail": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1) Q, K, V)",
        "config": {"workload": w.name + (f"-window{args.window}" if args.window > 0 else ""),
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal, "window": args.window,
                   "scale": w.scale, "layout": "[B,H,N,d] contiguous", "entry": entry, "workspace_bytes": ws_bytes,
                   "pct_of_mfma_peak": round(100 * value / MFMA_PEAK_TFLOPS, 2),
                   **launch_stats(t), "sclk": sclk,
                   "pct_of_peak_at_sclk": (round(100 * achieved / (MFMA_PEAK_TFLOPS * sclk["median_mhz"] / 2400.0), 2)
                                           if sclk and sclk.get("median_mhz") else None),
                   "l2": "cold" if args.cold_l2 else "warm",
                   "timing": ("ms_per_step: the mean of the K calls, each between its own events after a 1 GiB "
                              "buffer was overwritten (outside the events); launch_ms_*: the same calls")
                             if args.cold_l2 else
                             ("ms_per_step: one event pair around the K timed steps (also the roofline's launch "
                              "duration); launch_ms_*: a second loop of K launches, each between its own events "
                              "(those records add a few microseconds per launch)")},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     # the committed counters were taken with warm caches
                     "traffic": None if args.cold_l2 else measured_traffic(
                         w.name, causal, args.window,
                         key=(traffic_key(w.name, causal) + "-ws") if workspace is not None else None),
                     "kernel": f"attn_fwd_kernel<{w.d},{'bf16' if w.dtype == 'bf16' else 'f16'},{'causal' if causal else 'full'}>"
                               + (" with key-range parts, then lse_merge_kernel (achieved over both)" if workspace is not None else ""),
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": w.algorithmic_bytes()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, causal, q, k, v, out, lse, args.cpu_seconds, args.window)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
