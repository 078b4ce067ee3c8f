"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same rows, and measure the errors the acceptance bar is stated in."""
from __future__ import annotations

import numpy as np
import torch

import attn_workloads as aw
import oracle

# Acceptance bar for fp16/bf16 outputs against the float64 oracle.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def run_gpu(q, k, v, causal, scale, with_lse=True, stream=None, window=0):
    """q, k, v: CPU tensors.  Returns (out, lse) as CPU tensors (lse None if skipped).
    window > 0 goes through attn_fwd_window."""
    import exact_tiled_attention_03_amd as eta
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(qd)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda") if with_lse else None
    eta.attn_fwd(qd, kd, vd, out, lse, causal, scale, stream=stream, window=window)
    torch.cuda.synchronize()
    return out.cpu(), (lse.cpu() if with_lse else None)


def gather_rows(x: np.ndarray, rows):
    """x [B, H, N, ...] -> [B, H, R, ...] for rows None, [R] or [B, H, R]."""
    if rows is None:
        return x
    rows = np.asarray(rows)
    if rows.ndim == 1:
        return x[:, :, rows]
    B, H = x.shape[:2]
    return np.stack([np.stack([x[b, h, rows[b, h]] for h in range(H)]) for b in range(B)])


def errors(out, lse, q, k, v, causal, scale, rows=None, window=0):
    """Max-abs / mean-abs error of out and max-abs error of lse against the oracle."""
    O, L = oracle.attention(q, k, v, causal, scale, rows=rows, window=window)
    og = gather_rows(out.double().numpy(), rows)
    e = np.abs(og - O)
    res = {"max_abs": float(e.max()), "mean_abs": float(e.mean())}
    if lse is not None:
        lg = gather_rows(lse.double().numpy(), rows)
        res["lse_max_abs"] = float(np.abs(lg - L).max())
    return res


def assert_within_bar(err, label=""):
    assert err["max_abs"] <= MAX_ABS, f"{label} max_abs {err['max_abs']:.3e} > {MAX_ABS}"
    assert err["mean_abs"] <= MEAN_ABS, f"{label} mean_abs {err['mean_abs']:.3e} > {MEAN_ABS}"
    if "lse_max_abs" in err:
        assert err["lse_max_abs"] <= LSE_ABS, f"{label} lse error {err['lse_max_abs']:.3e} > {LSE_ABS}"


def unit_roundoff(dtype) -> float:
    """2^-p for a p-bit significand: bf16 has 8 bits, fp16 11."""
    return 2.0 ** -8 if dtype in ("bf16", torch.bfloat16) else 2.0 ** -11


def assert_within_derived_bound(out, lse, q, k, v, causal, scale, rows=None, label="", window=0,
                                partial_roundings=0):
    """Bar for shapes beyond the five workloads.

    The method rounds the probabilities to the input type before P V and the
    output to the input type at the end ("Triton in depth" 3.3 casts p to v's
    dtype; the store casts the fp32 accumulator).  With unit roundoff u these
    two roundings alone can move an output element by up to
        u * sum_j w_j |v_j|  +  u * (|O| + u * sum_j w_j |v_j|),
    which exceeds 1e-2 for bf16 when a few keys with large |v| dominate a row
    (early causal rows).  Each element must be within max(1e-2, that bound plus
    1e-5 * (1 + sum_j w_j |v_j|) of fp32 accumulation slack); the mean error must
    be within max(1e-3, the mean of the same bound), since with very few keys the
    output rounding alone averages about 1e-3 in bf16; lse keeps the plain bar.

    partial_roundings = 1 for results merged from key-range parts whose O was
    rounded to the input type before the merge: the merge weights sum to 1, so
    that rounding adds at most u * (1 + u) * sum_j w_j |v_j|."""
    u = unit_roundoff(q.dtype)
    O, L = oracle.attention(q, k, v, causal, scale, rows=rows, window=window)
    A, _ = oracle.attention(q, k, v.abs(), causal, scale, rows=rows, window=window)
    og = gather_rows(out.double().numpy(), rows)
    e = np.abs(og - O)
    derived = u * A + u * (np.abs(O) + u * A) + 1e-5 * (1.0 + A) + partial_roundings * u * (1 + u) * A
    bound = np.maximum(MAX_ABS, derived)
    worst = np.unravel_index(np.argmax(e - bound), e.shape)
    assert (e <= bound).all(), f"{label} error {e[worst]:.3e} > bound {bound[worst]:.3e} at {worst}"
    mean_bar = max(MEAN_ABS, float(derived.mean()))
    assert e.mean() <= mean_bar, f"{label} mean_abs {e.mean():.3e} > {mean_bar:.3e}"
    if lse is not None:
        lerr = np.abs(gather_rows(lse.double().numpy(), rows) - L).max()
        assert lerr <= LSE_ABS, f"{label} lse error {lerr:.3e} > {LSE_ABS}"


def workload_rows(w: aw.Workload):
    """Rows the oracle checks at a workload's full size: every row, except where the
    workload states a per-head sample (512 seeded rows per head, rows 0 and N-1
    always included)."""
    if w.sample_rows is None:
        return None
    return aw.sample_rows(w.B, w.H, w.N, w.sample_rows, w.seed + 7)
