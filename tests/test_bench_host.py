"""Host-side logic of bench.py (no GPU): the FLOPs credited per launch."""
import bench
import attn_workloads as aw


def brute_pairs(n, causal, window):
    return sum(1 for i in range(n) for j in range(n)
               if (not causal or j <= i) and (window == 0 or (i - window < j and (causal or j < i + window))))


def test_kept_pairs_matches_enumeration():
    for n in (1, 2, 7, 33):
        for causal in (0, 1):
            for window in (0, 1, 2, 5, 32, 33, 100):
                assert bench.kept_pairs(n, causal, window) == brute_pairs(n, causal, window)


def test_kept_pairs_on_rows_subset():
    rows = [0, 3, 9]
    assert bench.kept_pairs(10, 1, 4, rows) == 1 + 4 + 4
    assert bench.kept_pairs(10, 0, 4, rows) == 4 + 7 + 4


def test_launch_flops_conventions():
    w = aw.WORKLOADS[aw.HEADLINE]
    assert bench.launch_flops(w, 1, 0) == w.flops(1) == 2.0 * w.B * w.H * w.N ** 2 * w.d
    # a window of N keeps every causal pair: N(N+1)/2 per head, not the N^2/2 convention
    assert bench.launch_flops(w, 1, w.N) == 4.0 * w.d * w.B * w.H * w.N * (w.N + 1) / 2
    assert bench.launch_flops(w, 0, 1) == 4.0 * w.d * w.B * w.H * w.N


def test_every_name_bench_reads_is_defined():
    """Each name that bench.py loads is bound somewhere in it or is a builtin, so no
    run of the benchmark stops on a NameError."""
    import ast
    import builtins
    tree = ast.parse(open(bench.__file__).read())
    bound = set(dir(builtins)) | {"__file__", "__name__", "__doc__"}
    for node in ast.walk(tree):
        if isinstance(node, (ast.FunctionDef, ast.ClassDef, ast.AsyncFunctionDef)):
            bound.add(node.name)
        elif isinstance(node, ast.arg):
            bound.add(node.arg)
        elif isinstance(node, ast.Name) and isinstance(node.ctx, (ast.Store, ast.Del)):
            bound.add(node.id)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            bound.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, ast.ExceptHandler) and node.name:
            bound.add(node.name)
    loaded = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
    assert loaded <= bound, sorted(loaded - bound)


def test_clock_reading_never_raises_without_a_gpu():
    calls = []
    r = bench.ClockUnderLoad().measure(lambda: calls.append(1), max_s=0.1)
    assert "median_mhz" in r
    if r["median_mhz"] is None:
        assert r.get("error")


def test_cold_cache_buffer_exceeds_the_caches():
    """--cold-l2 overwrites more bytes than MI355X's caches hold between calls: eight
    4 MB L2s and the 256 MB Infinity Cache."""
    assert bench.COLD_L2_BYTES >= 2 * (8 * 4 * 2 ** 20 + 256 * 2 ** 20)


def test_cold_cache_timing_flushes_outside_the_events():
    """time_steps_cold overwrites the buffer before each call's start event, so the
    flush is never inside a timed interval (checked on the order of the calls it
    makes, with stand-ins for the stream events)."""
    import sys
    import types

    log = []

    class Event:
        def __init__(self, enable_timing=False):
            self.t = None

        def record(self, stream=None):
            log.append("record")
            self.t = len(log)

        def elapsed_time(self, other):
            return float(other.t - self.t)

    class Scratch:
        def fill_(self, v):
            log.append("flush")

    fake = types.SimpleNamespace(cuda=types.SimpleNamespace(Event=Event, synchronize=lambda: None))
    real = sys.modules.get("torch")
    sys.modules["torch"] = fake
    try:
        t = bench.time_steps_cold(lambda: log.append("call"), 3, None, Scratch())
    finally:
        if real is not None:
            sys.modules["torch"] = real
        else:
            del sys.modules["torch"]
    assert log == ["flush", "record", "call", "record"] * 3
    assert t["per_launch"] == [2.0, 2.0, 2.0] and t["ms_per_step"] == 2.0
