"""GPU parity of the standalone row softmax (softmax_rows, include/softmax.h)
against the float64 oracle (oracle/softmax.py, pinned in
test_oracle_softmax_pins.py), element by element, with the bar derived below.

Bar.  The kernel computes in fp32: y = exp2(fma(x, log2e, -max*log2e)) * (1/sum).
With u = 2^-24 the relative error of one output is at most about
  * u (2|x| + 3|max|)  from rounding the exp2 argument (log2e, the product
    max*log2e and the fma each round once; ln2 * log2e = 1 turns the log2-unit
    error into a relative one),
  * 4u                 for v_exp_f32 (documented at 1 ulp, i.e. 2u) with margin,
  * 130u               for the sum of positive terms: at most 64 sequential
    additions per thread and two reduction trees (1024 threads, 16 waves) when
    the row fits in registers; for longer rows at most 32 additions per tile and
    a compensated running sum, whose error does not grow with the tile count,
  * 4u per rescale of a running sum (longer rows only), at most one per tile of
    16384 elements,
  * 3u                 for the reciprocal and the product,
and a 16-bit y adds its own rounding to nearest even (u_out = 2^-8 bf16, 2^-11
fp16).  Outputs below the normal range may be flushed: absolute slack 2^-126
(fp32, bf16) or half an fp16 subnormal step, 2^-25.  Every element must satisfy
|y - y_oracle| <= rel * y_oracle + atol.
"""
import numpy as np
import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
import oracle

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
U_OUT = {"f32": 0.0, "bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
ATOL = {"f32": 2.0 ** -126, "bf16": 2.0 ** -126, "fp16": 2.0 ** -25}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def rescales(cols: int) -> int:
    """Upper bound on the running-sum rescales of one thread: none when the row fits in
    registers (65536 elements), else at most one per tile of 16384 or more elements."""
    return 0 if cols <= 65536 else -(-cols // 16384)


def rel_bound(abs_x, abs_max, cols: int, dtype: str):
    return U32 * (2 * abs_x + 3 * abs_max + 4 + 130 + 4 * rescales(cols) + 3) + U_OUT[dtype]


def bound(x64: np.ndarray, y_ref: np.ndarray, dtype: str) -> np.ndarray:
    finite = np.where(np.isfinite(x64), x64, -np.inf)
    m = np.abs(finite.max(axis=1, keepdims=True))
    xa = np.where(np.isfinite(x64), np.abs(x64), 0.0)
    return rel_bound(xa, m, x64.shape[1], dtype) * y_ref + ATOL[dtype]


def check(y_gpu: torch.Tensor, x_cpu: torch.Tensor, dtype: str, label: str, rows=None):
    """Compare y (GPU or CPU tensor) with the oracle on x (CPU), optionally on a row subset."""
    x = x_cpu if rows is None else x_cpu[rows]
    y = (y_gpu if rows is None else y_gpu[rows]).double().cpu().numpy()
    with np.errstate(invalid="ignore"):
        ref = oracle.softmax_rows(x)
    x64 = x.double().numpy()
    nan_ref, nan_got = np.isnan(ref), np.isnan(y)
    assert (nan_ref == nan_got).all(), f"{label}: NaN pattern differs at {np.argwhere(nan_ref != nan_got)[:5]}"
    ok = ~nan_ref
    with np.errstate(invalid="ignore"):
        b = bound(x64, np.where(ok, ref, 0.0), dtype)
    err = np.where(ok, np.abs(y - np.where(ok, ref, 0.0)), 0.0)
    if (err > b).any():
        i = np.unravel_index(np.argmax(err - b), err.shape)
        raise AssertionError(f"{label}: |y - ref| = {err[i]:.3e} > bound {b[i]:.3e} at {i} "
                             f"(y={y[i]!r}, ref={ref[i]!r})")


def run(x_cpu: torch.Tensor) -> torch.Tensor:
    """x copied to the GPU as it is (contiguous: rows 16-byte aligned only when
    cols * element size is a multiple of 16)."""
    y = eta.softmax_rows(x_cpu.cuda())
    torch.cuda.synchronize()
    return y


def run_padded(x_cpu: torch.Tensor) -> torch.Tensor:
    """x on the GPU with its row stride padded to 16 bytes (the vectorised kernels);
    y gets the same padded stride."""
    rows, cols = x_cpu.shape
    per16 = 16 // x_cpu.element_size()
    xs = -(-cols // per16) * per16
    big = torch.empty((rows, xs), dtype=x_cpu.dtype, device="cuda")
    big[:, :cols] = x_cpu.cuda()
    y = eta.softmax_rows(big[:, :cols])
    torch.cuda.synchronize()
    assert y.stride(0) == xs
    return y


# column counts around every vector, work-group and tile boundary of both kernels:
# 4/8-element vectors, 64/256/1024-thread groups, up to 64 values per thread in
# registers (65536 elements), tiles of 16384 (fp32) or 32768 (16-bit) beyond that
COLS = [1, 2, 3, 7, 8, 9, 63, 64, 65, 255, 256, 257, 1000, 1023, 1024, 1025, 4095, 4096, 4097, 8200, 16384,
        16385, 32767, 32768, 32769, 65535, 65536, 65537, 100003]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp16"])
@pytest.mark.parametrize("layout", ["contiguous", "padded"])
def test_softmax_parity_column_counts(lib, dtype, layout):
    for i, cols in enumerate(COLS):
        rows = 33 if cols <= 4097 else 5
        print(f"\n[case] softmax {dtype} {layout} rows={rows} cols={cols}", flush=True)
        x = aw.make_rows(rows, cols, dtype, 3000 + i, sigma=2.0)
        y = run(x) if layout == "contiguous" else run_padded(x)
        check(y, x, dtype, f"{dtype} {layout} cols={cols}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [4096, 65536, 65537, 100003])
def test_softmax_dominant_element_positions(lib, dtype, cols):
    """One large entry per row at vector, group and tile edges (first, last, ...):
    the row's max and most of its sum sit in that one element."""
    positions = sorted({p for p in (0, 1, 7, 8, 1023, 1024, 4095, 4096, 16383, 16384, 32767, 32768, 65535,
                                    65536, cols - 2, cols - 1) if 0 <= p < cols})
    x = aw.make_rows(len(positions), cols, dtype, 3100 + cols)
    for r, p in enumerate(positions):
        x[r, p] = 12.0
    print(f"\n[case] softmax dominant {dtype} cols={cols} positions={positions}", flush=True)
    check(run_padded(x), x, dtype, f"dominant {dtype} cols={cols}")
    check(run(x), x, dtype, f"dominant {dtype} cols={cols}")


@pytest.mark.parametrize("cols", [3, 300, 65536, 70001])
def test_softmax_masked_entries_and_specials(lib, cols):
    """-inf entries (masked positions) get exactly 0; rows with +inf or NaN, or with
    every entry -inf, are NaN throughout in IEEE arithmetic, as in the oracle."""
    x = aw.make_rows(8, cols, "f32", 3200 + cols)
    g = np.random.default_rng(cols)
    x[0, torch.from_numpy(g.random(cols) < 0.5)] = -float("inf")
    x[0, cols // 2] = 0.5                                   # never all masked
    x[1, :] = -float("inf")
    x[1, cols - 1] = -3.0                                   # a single survivor, at the tail
    x[2, :] = -float("inf")                                 # all masked -> NaN
    x[3, cols // 3] = float("inf")                          # +inf -> NaN
    x[4, cols - 1] = float("nan")                           # NaN -> NaN
    x[5, :] = 1.25                                          # constant row: 1/cols everywhere
    for y in (run(x), run_padded(x)):
        print(f"\n[case] softmax specials cols={cols} row stride {y.stride(0)}", flush=True)
        check(y, x, "f32", f"specials cols={cols}")
        yc = y.cpu()
        assert (yc[0][x[0] == -float("inf")] == 0).all()
        assert (yc[1, :cols - 1] == 0).all() and abs(float(yc[1, cols - 1]) - 1.0) <= 4 * U32
        for r in (2, 3, 4):
            assert torch.isnan(yc[r]).all(), r


@pytest.mark.parametrize("dtype", ["f32", "fp16"])
@pytest.mark.parametrize("cols", [37, 4100, 70001])
def test_softmax_strided_rows_and_offsets(lib, dtype, cols):
    """x and y with padded row strides of their own, x starting at an aligned offset."""
    per16 = 4 if dtype == "f32" else 8
    xs = (cols + per16 - 1) // per16 * per16 + 3 * per16
    ys = (cols + per16 - 1) // per16 * per16 + per16
    rows = 9
    big = aw.make_rows(rows + 1, xs, dtype, 3300 + cols)
    xd = big.cuda()[1:, per16:per16 + cols]                # aligned: row stride xs, offset xs + per16
    assert xd.stride(0) == xs and xd.data_ptr() % 16 == 0
    yd_big = torch.full((rows, ys), 7.0, dtype=TORCH[dtype], device="cuda")
    yd = yd_big[:, :cols]
    print(f"\n[case] softmax strided {dtype} cols={cols} xs={xs} ys={ys}", flush=True)
    eta.softmax_rows(xd, yd)
    torch.cuda.synchronize()
    check(yd, big[1:, per16:per16 + cols].contiguous(), dtype, f"strided {dtype} cols={cols}")
    assert (yd_big[:, cols:].cpu() == 7.0).all(), "padding between rows was written"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols", [100, 32768, 100003])
def test_softmax_in_place(lib, dtype, cols):
    x = aw.make_rows(6, cols, dtype, 3400 + cols, sigma=3.0)
    xd = x.cuda()
    out = eta.softmax_rows(xd, xd)
    torch.cuda.synchronize()
    assert out.data_ptr() == xd.data_ptr()
    check(xd, x, dtype, f"in place {dtype} cols={cols}")


def test_softmax_more_rows_than_groups(lib):
    """More rows than the 65536 work-groups of one launch: the grid strides over rows."""
    for rows, cols, dt in ((70001, 5, "f32"), (131075, 3, "bf16"), (65537, 1, "fp16")):
        print(f"\n[case] softmax many rows {rows}x{cols} {dt}", flush=True)
        x = aw.make_rows(rows, cols, dt, 3500 + rows)
        check(run(x), x, dt, f"rows={rows} cols={cols}")


def test_softmax_empty_is_a_no_op(lib):
    for shape in ((0, 5), (3, 0)):
        x = torch.empty(shape, device="cuda")
        assert eta.softmax_rows(x).shape == shape


def test_softmax_rejects_overlap_unless_in_place(lib):
    y = torch.zeros(4, 12, device="cuda")        # 48-byte rows
    with pytest.raises(eta.AttnError) as e:
        eta.softmax_rows(y[:, 4:12], y[:, :8])  # overlapping spans, not in place
    assert e.value.status == 10
    x = aw.make_rows(4, 12, "f32", 3600)
    yd = x.cuda()
    eta.softmax_rows(yd[:, :8], yd[:, :8])       # in place on a strided view
    torch.cuda.synchronize()
    check(yd[:, :8], x[:, :8].contiguous(), "f32", "strided in place")
    assert torch.equal(yd[:, 8:].cpu(), x[:, 8:])


@pytest.mark.parametrize("name", [w.name for w in aw.SOFTMAX_WORKLOADS])
def test_softmax_full_size_workloads(lib, name):
    """The benchmark's shapes at full size, launched exactly as bench.py launches
    them: every row's sum is 1 within the bar, and 64 sampled rows (first and last
    included) match the oracle element by element."""
    w = aw.softmax_by_name(name)
    print(f"\n[case] softmax workload {name}", flush=True)
    x = aw.make_rows(w.rows, w.cols, w.dtype, w.seed, w.sigma)
    xd = x.cuda()
    y = eta.softmax_rows(xd)
    torch.cuda.synchronize()
    s = y.double().sum(dim=1).cpu().numpy()
    xmax = float(x.abs().max())
    slack = rel_bound(xmax, xmax, w.cols, w.dtype) + w.cols * ATOL[w.dtype]
    assert np.abs(s - 1.0).max() <= slack, f"row sums off by {np.abs(s - 1.0).max():.3e} > {slack:.3e}"
    rows = np.unique(np.concatenate([[0, w.rows - 1], np.random.default_rng(w.seed).choice(w.rows, 62, False)]))
    check(y, x, w.dtype, name, rows=torch.from_numpy(rows))


@pytest.mark.parametrize("rows,cols,dtype", [(2, (1 << 30) + 5, "f32"), (1, (1 << 31) - 1, "bf16")])
def test_softmax_maximum_sizes_closed_form(lib, rows, cols, dtype):
    """Rows whose byte offsets pass 2^31 and 2^32, checked against a closed form: with
    x_j = 0.5 (j mod 7) - r the softmax is exp(0.5 (j mod 7)) / sum_k c_k exp(0.5 k),
    c_k the number of j < cols with j mod 7 = k (the row shift r cancels).  Every
    thread's first tile already holds the row maximum 3 - r, so no running sum is
    ever rescaled."""
    if torch.cuda.get_device_properties(0).total_memory < 64 << 30:
        pytest.skip("needs a device with tens of GB")
    el = 4 if dtype == "f32" else 2
    xs = -(-cols // (16 // el)) * (16 // el)
    print(f"\n[case] softmax max size rows={rows} cols={cols} {dtype} ({rows * xs * el / 2**30:.1f} GiB each)",
          flush=True)
    x = torch.empty((rows, xs), dtype=TORCH[dtype], device="cuda")[:, :cols]
    chunk = 1 << 26
    for c0 in range(0, cols, chunk):
        j = torch.arange(c0, min(cols, c0 + chunk), device="cuda", dtype=torch.int64)
        for r in range(rows):
            x[r, c0:c0 + j.numel()] = ((j % 7).to(torch.float32) * 0.5 - r).to(TORCH[dtype])
    y = eta.softmax_rows(x)
    torch.cuda.synchronize()
    assert rows == 1 or y.stride(0) == xs
    del x
    counts = [(cols - k + 6) // 7 for k in range(7)]
    z = sum(c * np.exp(0.5 * k) for k, c in enumerate(counts))
    expect = torch.tensor([np.exp(0.5 * k) / z for k in range(7)], dtype=torch.float64, device="cuda")
    rel = U32 * (2 * 3.0 + 3 * 3.0 + 4 + 130 + 3) + U_OUT[dtype]
    for c0 in range(0, cols, chunk):
        j = torch.arange(c0, min(cols, c0 + chunk), device="cuda", dtype=torch.int64)
        ref = expect[j % 7]
        for r in range(rows):
            err = (y[r, c0:c0 + j.numel()].double() - ref).abs() / ref
            assert float(err.max()) <= rel, f"row {r} cols {c0}..: rel err {float(err.max()):.3e} > {rel:.3e}"
