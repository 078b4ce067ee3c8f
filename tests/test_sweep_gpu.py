"""Seeded random configurations: the other parity tests pick their shapes by hand,
one property at a time; these draw shape, head dim, type, mask, window, scale and
outliers together from a fixed-seed generator, per schedule the library selects
(4-wave, 4-wave unpaired causal, 8-wave, 8-wave key split, key-range parts
through attn_fwd_ws), plus the backward, the matrix product, the row softmax
and the merge of key shards.  Each case is checked against the float64 oracle
with the bars of the other tests (forward: the derived per-element and mean
bounds, lse; backward: the gradient bound; the others: their own files' bars),
on every row or on a seeded sample of rows per head where a case has hundreds
of heads.

The draw is fixed by SEED: a case's id names its shape and parameters, so a
failure is reproduced by running that id alone."""
import math

import numpy as np
import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
from parity_util import assert_within_derived_bound
from test_bwd_gpu import bwd_inputs, check_bwd, run_bwd

pytestmark = pytest.mark.gpu

SEED = 20261202
D_CHOICES = (64, 80, 128)


def _scale(rng, d):
    """Mostly 1/sqrt(d) times a factor in [0.3, 3]; sometimes 0 (uniform weights)
    or negative (the mask's largest scores become the smallest)."""
    u = rng.random()
    if u < 0.1:
        return 0.0
    if u < 0.25:
        return -float(rng.uniform(0.05, 0.5))
    return float(rng.uniform(0.3, 3.0)) / math.sqrt(d)


def _length(rng, hi):
    """Half the draws log-uniform over [1, hi] (the short, ragged tiles), half
    uniform over [64, hi] (several tiles)."""
    if rng.random() < 0.5:
        return int(round(math.exp(rng.uniform(0.0, math.log(hi)))))
    return int(rng.integers(64, hi + 1))


def _split_bh(rng, bh):
    B = int(rng.integers(1, 5))
    return B, -(-bh // B)


def _outliers(rng):
    return (0.01, float(rng.uniform(4.0, 30.0))) if rng.random() < 0.3 else (0.0, 1.0)


def _forward_cases():
    rng = np.random.default_rng(SEED)
    cases = []

    def add(kind, B, H, N, d, causal, window=0, sample=None):
        frac, factor = _outliers(rng)
        cases.append(dict(kind=kind, B=B, H=H, N=N, d=d, dtype=("fp16", "bf16")[int(rng.integers(2))],
                          causal=causal, window=window, scale=_scale(rng, d), outlier_fraction=frac,
                          outlier_factor=factor, sample=sample, seed=int(rng.integers(1 << 30))))

    for _ in range(24):      # 4-wave: few heads, any length below the key split's
        N = _length(rng, 1600)
        window = int(rng.integers(1, N + 41)) if rng.random() < 0.4 else 0
        add("small", int(rng.integers(1, 3)), int(rng.integers(1, 5)), N, int(rng.choice(D_CHOICES)),
            int(rng.integers(2)), window)
    for _ in range(10):      # 8-wave: at least 512 work-groups of 256 queries
        N = int(rng.integers(100, 521))
        causal = int(rng.integers(2))
        nqt = -(-N // 256)
        groups = (nqt + 1) // 2 if causal else nqt
        B, H = _split_bh(rng, -(-512 // groups) + int(rng.integers(0, 17)))
        window = int(rng.integers(1, N + 41)) if rng.random() < 0.3 else 0
        add("wide", B, H, N, int(rng.choice(D_CHOICES)), causal, window, sample=40)
    for causal in (0, 0, 0, 1, 1, 1):   # 8-wave key split: d = 64, long rows, few work-groups
        if causal:
            N = int(rng.integers(4096, 4601))
            bh = int(rng.integers(1, 4))
        else:
            N = int(rng.integers(2048, 3601))
            bh = int(rng.integers(1, min(6, 511 // -(-N // 128)) + 1))
        add("split", 1, bh, N, 64, causal, sample=64)
    for _ in range(8):       # 4-wave causal, one query tile per work-group, unpaired
        N = int(rng.integers(200, 2001))
        nqt = -(-N // 128)
        bh = int(rng.integers(1, min(12, 512 // nqt) + 1))
        add("unpaired", 1, bh, N, int(rng.choice((80, 128))) if N >= 2048 else int(rng.choice(D_CHOICES)), 1)
    for _ in range(10):      # attn_fwd_ws: the key-range parts of the chip's last round, merged
        N = int(rng.integers(300, 3001))
        add("ws", 1, int(rng.integers(1, 25)), N, int(rng.choice(D_CHOICES)), 0)
    return cases


def _case_id(i, c):
    w = f"-w{c['window']}" if c["window"] else ""
    return (f"f{i:02d}-{c['kind']}-{c['B']}x{c['H']}x{c['N']}x{c['d']}-{c['dtype']}-c{c['causal']}{w}"
            f"-s{c['scale']:.3g}" + ("-outl" if c["outlier_fraction"] else ""))


FWD = _forward_cases()


def _rows(c):
    if c["sample"] is None:
        return None
    return aw.sample_rows(c["B"], c["H"], c["N"], c["sample"], c["seed"] + 1)


@pytest.mark.parametrize("c", FWD, ids=[_case_id(i, c) for i, c in enumerate(FWD)])
def test_forward_sweep(lib, c):
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    print(f"\n[case] {c}", flush=True)
    q, k, v = aw.make_inputs((B, H, N, d), c["dtype"], c["seed"], c["outlier_fraction"], c["outlier_factor"])
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    partial = 0
    if c["kind"] == "ws":
        need = eta.attn_fwd_workspace_bytes(B, H, N, d, False)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        eta.attn_fwd_ws(qd, kd, vd, out, lse, False, c["scale"], ws)
        partial = 1 if need else 0
    else:
        eta.attn_fwd(qd, kd, vd, out, lse, bool(c["causal"]), c["scale"], window=c["window"])
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert_within_derived_bound(out, lse, q, k, v, c["causal"], c["scale"], rows=_rows(c), label=str(c),
                                window=c["window"], partial_roundings=partial)


def test_forward_sweep_covers_every_schedule(lib):
    """The draw above reaches each schedule: asked of the library for each case."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    want = {"small": lib.ATTN_SCHEDULE_SMALL, "unpaired": lib.ATTN_SCHEDULE_SMALL,
            "wide": lib.ATTN_SCHEDULE_WIDE, "split": lib.ATTN_SCHEDULE_SPLIT}
    split_parts = 0
    for i, c in enumerate(FWD):
        s = lib.attn_fwd_schedule(c["B"], c["H"], c["N"], c["d"], c["causal"])
        if c["kind"] == "ws":
            split_parts += eta.attn_fwd_workspace_bytes(c["B"], c["H"], c["N"], c["d"], False) > 0
            continue
        assert s == want[c["kind"]], _case_id(i, c)
        if c["kind"] == "unpaired" and cus >= 256:
            # one round of two 4-wave work-groups per CU: the unpaired grid
            assert -(-c["N"] // 128) * c["B"] * c["H"] <= 2 * cus, _case_id(i, c)
    assert split_parts >= 5, "too few attn_fwd_ws cases split into key-range parts on this device"


def _backward_cases():
    rng = np.random.default_rng(SEED + 1)
    cases = []
    for _ in range(24):
        d = int(rng.choice(D_CHOICES))
        cases.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), N=_length(rng, 1000),
                          d=d, dtype=("fp16", "bf16")[int(rng.integers(2))], causal=int(rng.integers(2)),
                          scale=_scale(rng, d), seed=int(rng.integers(1 << 30))))
    return cases


BWD = _backward_cases()


@pytest.mark.parametrize("c", BWD, ids=[f"b{i:02d}-{c['B']}x{c['H']}x{c['N']}x{c['d']}-{c['dtype']}-c{c['causal']}"
                                         f"-s{c['scale']:.3g}" for i, c in enumerate(BWD)])
def test_backward_sweep(lib, c):
    print(f"\n[case] {c}", flush=True)
    shape = (c["B"], c["H"], c["N"], c["d"])
    q, k, v, do, out, lse = bwd_inputs(shape, c["dtype"], c["seed"], c["causal"], c["scale"])
    dq, dk, dv, _ = run_bwd(q, k, v, do, out, lse, c["causal"], c["scale"])
    check_bwd((dq, dk, dv), q, k, v, do, c["causal"], c["scale"], c["dtype"], str(c))


# --- the later rows: matrix product, row softmax, merge of key shards ----------

def _gemm_cases():
    rng = np.random.default_rng(SEED + 2)
    cases = []
    for _ in range(16):
        cases.append(dict(M=_length(rng, 1200), N=_length(rng, 1200), K=_length(rng, 600),
                          b_layout=("kn", "nk")[int(rng.integers(2))],
                          act=("none", "relu", "gelu_tanh")[int(rng.integers(3))],
                          bias=bool(rng.random() < 0.75), dtype=("fp16", "bf16")[int(rng.integers(2))],
                          seed=int(rng.integers(1 << 30))))
    return cases


GEMM = _gemm_cases()


@pytest.mark.parametrize("c", GEMM, ids=[f"g{i:02d}-{c['M']}x{c['N']}x{c['K']}-{c['b_layout']}-{c['act']}"
                                          f"{'-bias' if c['bias'] else ''}-{c['dtype']}" for i, c in enumerate(GEMM)])
def test_gemm_sweep(lib, c):
    """M, N, K drawn around and between the 256-row tiles, the 64-wide k steps and the
    8-element chunks (K not a multiple of 8 goes through the binding's zero padding)."""
    from test_gemm_gpu import check as check_gemm
    print(f"\n[case] {c}", flush=True)
    a, b, bias = aw.make_gemm(c["M"], c["N"], c["K"], c["dtype"], c["b_layout"], c["seed"])
    bias = bias if c["bias"] else None
    out = eta.gemm_bias_act(a.cuda(), b.cuda(), None if bias is None else bias.cuda(), c["act"], c["b_layout"])
    torch.cuda.synchronize()
    check_gemm(out.cpu(), a, b, bias, c["act"], c["b_layout"], c["dtype"], str(c))


def _softmax_cases():
    rng = np.random.default_rng(SEED + 3)
    cases = []
    for _ in range(12):
        if rng.random() < 0.5:
            cols = int(round(math.exp(rng.uniform(0.0, math.log(200000)))))
        else:
            cols = int(rng.integers(30000, 200001))
        rows = int(rng.integers(1, max(2, min(300, 4_000_000 // cols)) + 1))
        cases.append(dict(rows=rows, cols=cols, dtype=("f32", "bf16", "fp16")[int(rng.integers(3))],
                          sigma=float(rng.choice((0.5, 1.0, 4.0, 20.0))), masked=float(rng.choice((0.0, 0.0, 0.3))),
                          seed=int(rng.integers(1 << 30))))
    return cases


SOFTMAX = _softmax_cases()


@pytest.mark.parametrize("c", SOFTMAX, ids=[f"s{i:02d}-{c['rows']}x{c['cols']}-{c['dtype']}-sigma{c['sigma']:g}"
                                             f"{'-masked' if c['masked'] else ''}" for i, c in enumerate(SOFTMAX)])
def test_softmax_sweep(lib, c):
    """Row lengths from 1 to 2e5 (in registers up to 65536, tiled beyond), score
    spreads up to sigma = 20, and rows with a share of -inf (masked) entries."""
    from test_softmax_gpu import check as check_softmax
    print(f"\n[case] {c}", flush=True)
    x = aw.make_rows(c["rows"], c["cols"], c["dtype"], c["seed"], c["sigma"])
    if c["masked"]:
        keep = np.random.default_rng(c["seed"] + 1).random((c["rows"], c["cols"])) >= c["masked"]
        keep[:, 0] = True                                   # every row keeps one entry
        x = x.masked_fill(torch.from_numpy(~keep), -float("inf"))
    y = eta.softmax_rows(x.cuda())
    torch.cuda.synchronize()
    check_softmax(y, x, c["dtype"], str(c))


def _merge_cases():
    rng = np.random.default_rng(SEED + 4)
    cases = []
    for _ in range(10):
        cases.append(dict(G=int(rng.integers(1, 11)), R=_length(rng, 40000), d=int(rng.choice(D_CHOICES)),
                          dtype=("fp16", "bf16")[int(rng.integers(2))], empty=float(rng.choice((0.0, 0.2, 0.6))),
                          seed=int(rng.integers(1 << 30))))
    return cases


MERGE = _merge_cases()


@pytest.mark.parametrize("c", MERGE, ids=[f"m{i:02d}-G{c['G']}-R{c['R']}-d{c['d']}-{c['dtype']}-empty{c['empty']:g}"
                                          for i, c in enumerate(MERGE)])
def test_merge_sweep(lib, c):
    """G from 1 to 10 shards (past the eight read per round), lse spread over
    about 20 nats, and a share of -inf entries (shards with no key for a row),
    which leaves some rows with every shard empty."""
    from oracle import backward as ob
    from test_bwd_gpu import U_OUT
    print(f"\n[case] {c}", flush=True)
    G, R, d = c["G"], c["R"], c["d"]
    g = np.random.default_rng(c["seed"])
    o_parts = torch.from_numpy(g.standard_normal((G, R, d)).astype(np.float32)).to(aw.DTYPES[c["dtype"]])
    l_np = (g.standard_normal((G, R)) * 5.0 + 3.0).astype(np.float32)
    l_np[g.random((G, R)) < c["empty"]] = -np.inf
    l_parts = torch.from_numpy(l_np)
    o, lse = eta.attn_lse_merge(o_parts.cuda(), l_parts.cuda())
    torch.cuda.synchronize()
    ro, rl = ob.lse_merge(o_parts.double().numpy(), l_parts.double().numpy())
    got_o, got_l = o.cpu().double().numpy(), lse.cpu().double().numpy()
    empty = ~np.isfinite(rl)
    assert (np.isneginf(got_l) == empty).all()
    assert (got_o[empty] == 0).all()
    ok = ~empty
    big = np.abs(o_parts.double().numpy()).max(axis=0)
    assert (np.abs(got_o - ro)[ok] <= (U_OUT[c["dtype"]] * np.abs(ro) + 1e-5 * (1 + big))[ok]).all()
    assert (np.abs(got_l[ok] - rl[ok]) <= 1e-5 * (1 + np.abs(rl[ok]))).all()
