"""attn_fwd_ws through the C ABI: the forward whose last, incomplete round of query
tiles is cut into key ranges run on otherwise idle CUs and merged, against the
float64 oracle on the same seeded inputs, and against attn_fwd where the two
must agree exactly."""
import math

import numpy as np
import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
from parity_util import assert_within_bar, assert_within_derived_bound, errors, run_gpu

pytestmark = pytest.mark.gpu


def resident_groups():
    return torch.cuda.get_device_properties(0).multi_processor_count & ~7


def documented_plan(B, H, N, d, causal):
    """The split include/attn.h describes, computed here from its text: None when
    attn_fwd_ws does not split, else the cut tiles' first row, row count, part
    count and workspace size."""
    S = resident_groups()
    nqt = -(-N // 256)
    items = nqt * B * H
    r = items % S
    if causal or r == 0:
        return None
    P = min(S // r, (-(-N // 64)) // 2)
    if P < 2:
        return None
    whole = items - r
    row0 = (whole // nqt) * N + (whole % nqt) * 256
    rows = B * H * N - row0

    def up(x):
        return -(-x // 256) * 256

    return {"row0": row0, "rows": rows, "P": P, "bytes": up(P * rows * d * 2) + up(P * rows * 4) + up(rows * 4)}


def run_ws(q, k, v, causal, scale, with_lse=True, workspace="auto"):
    """q, k, v: CPU tensors.  workspace "auto" allocates attn_fwd_workspace_bytes."""
    B, H, N, d = q.shape
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(qd)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda") if with_lse else None
    if isinstance(workspace, str):
        need = eta.attn_fwd_workspace_bytes(B, H, N, d, causal)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    eta.attn_fwd_ws(qd, kd, vd, out, lse, causal, scale, workspace)
    torch.cuda.synchronize()
    return out.cpu(), (lse.cpu() if with_lse else None)


def cut_rows(B, H, N, plan):
    """[B, H, R] rows of every head that lie in the cut tiles (row >= row0 of [BH*N])."""
    flat = np.arange(B * H * N).reshape(B, H, N)
    return [(b, h) for b in range(B) for h in range(H) if flat[b, h, -1] >= plan["row0"]]


SHAPES = [  # (B, H, N, d, dtype): each leaves a last round of at most half the CUs
    (3, 8, 3000, 80, "fp16"),   # the ragged workload: 288 tiles, 32 cut
    (1, 9, 8192, 128, "bf16"),
    (1, 20, 3500, 64, "fp16"),
    (1, 2, 1000, 64, "bf16"),   # fewer tiles than CUs: every tile is cut
    (1, 43, 3000, 80, "bf16"),  # attn_fwd runs the same 8-wave kernel on the whole tiles
]


def test_workspace_bytes_follow_the_documented_plan(lib):
    for B, H, N, d, _ in SHAPES + [(2, 32, 4096, 128, "bf16"), (1, 16, 32768, 128, "bf16"), (4, 16, 1024, 64, "fp16")]:
        for causal in (0, 1):
            plan = documented_plan(B, H, N, d, causal)
            got = eta.attn_fwd_workspace_bytes(B, H, N, d, causal)
            assert got == (plan["bytes"] if plan else 0), (B, H, N, d, causal)
    # the shapes above that are meant to split do split on a 256-CU device
    if resident_groups() == 256:
        for B, H, N, d, _ in SHAPES:
            assert documented_plan(B, H, N, d, 0) is not None, (B, H, N, d)


def test_ragged_workload_parity(lib):
    w = aw.by_name("ragged_b3_h8_n3000_d80_fp16")
    print(f"\n[case] attn_fwd_ws {w.name} shape={w.shape}", flush=True)
    q, k, v = aw.workload_inputs(w)
    out, lse = run_ws(q, k, v, 0, w.scale)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    err = errors(out, lse, q, k, v, 0, w.scale)
    print(f"[err] {err}", flush=True)
    assert_within_bar(err, "attn_fwd_ws " + w.name)


@pytest.mark.parametrize("B,H,N,d,dtype", SHAPES[1:], ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}-{s[4]}" for s in SHAPES[1:]])
def test_split_shapes_within_derived_bound(lib, B, H, N, d, dtype):
    print(f"\n[case] attn_fwd_ws B={B} H={H} N={N} d={d} {dtype}", flush=True)
    q, k, v = aw.make_inputs((B, H, N, d), dtype, 9100 + N + d)
    scale = 1.0 / math.sqrt(d)
    out, lse = run_ws(q, k, v, 0, scale)
    plan = documented_plan(B, H, N, d, 0)
    rng = np.random.default_rng(N)
    # every head: the first and last 32 rows and a sample, plus the rows around the cut
    rows = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N), rng.choice(N, min(N, 128), replace=False),
                                     np.arange(max(0, plan["row0"] % N - 16), min(N, plan["row0"] % N + 16))]))
    assert_within_derived_bound(out, lse, q, k, v, 0, scale, rows=rows, partial_roundings=1,
                                label=f"B={B} H={H} N={N} d={d} {dtype}")
    # the heads that hold cut tiles: every row (every third beyond 4096 rows)
    dense = np.arange(N) if N <= 4096 else np.unique(np.concatenate([np.arange(0, N, 3), np.arange(N - 64, N)]))
    for b, h in cut_rows(B, H, N, plan)[:2]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        assert_within_derived_bound(out[sl], lse[sl], q[sl], k[sl], v[sl], 0, scale, rows=dense, partial_roundings=1,
                                    label=f"head ({b},{h})")


def test_whole_tiles_match_attn_fwd_bitwise(lib):
    """B=1 H=43 N=3000: attn_fwd uses the 8-wave kernel too, so every row before
    the cut tiles is the same computation and must match bit for bit."""
    B, H, N, d = 1, 43, 3000, 80
    q, k, v = aw.make_inputs((B, H, N, d), "bf16", 9200)
    out_ws, lse_ws = run_ws(q, k, v, 0, 0.11)
    out, lse = run_gpu(q, k, v, 0, 0.11)
    plan = documented_plan(B, H, N, d, 0)
    n0 = plan["row0"]
    flat_ws, flat = out_ws.reshape(-1, d), out.reshape(-1, d)
    assert torch.equal(flat_ws[:n0].view(torch.int16), flat[:n0].view(torch.int16))
    assert torch.equal(lse_ws.reshape(-1)[:n0], lse.reshape(-1)[:n0])
    # the cut rows differ from attn_fwd by at most the extra rounding of the parts
    diff = (flat_ws[n0:].float() - flat[n0:].float()).abs().max().item()
    assert diff <= 2.0 ** -7, diff


def test_null_workspace_and_causal_are_attn_fwd(lib):
    q, k, v = aw.make_inputs((3, 8, 3000, 80), "fp16", 9300)
    for causal in (0, 1):
        ref, ref_l = run_gpu(q, k, v, causal, 0.1)
        for ws in (None, "auto"):
            if ws == "auto" and not causal:
                continue   # that one splits
            out, lse = run_ws(q, k, v, causal, 0.1, workspace=ws)
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (causal, ws)
            assert torch.equal(lse, ref_l), (causal, ws)
    assert eta.attn_fwd_workspace_bytes(3, 8, 3000, 80, 1) == 0


def test_without_lse_and_repeatable(lib):
    q, k, v = aw.make_inputs((1, 20, 3500, 64), "fp16", 9400)
    a, la = run_ws(q, k, v, 0, 0.125)
    b, _ = run_ws(q, k, v, 0, 0.125, with_lse=False)
    c, lc = run_ws(q, k, v, 0, 0.125)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16)) and torch.equal(la, lc)


def test_workspace_errors(lib):
    """Rejected before any launch: out keeps its sentinel."""
    B, H, N, d = 3, 8, 3000, 80
    q, k, v = (t.cuda() for t in aw.make_inputs((B, H, N, d), "fp16", 9500))
    need = eta.attn_fwd_workspace_bytes(B, H, N, d, 0)
    assert need > 0
    out = torch.full_like(q, 7.0)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    big = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    cases = [(big[:need - 256], 13), (big[16:16 + need], 6)]
    for ws, code in cases:
        with pytest.raises(eta.AttnError) as e:
            eta.attn_fwd_ws(q, k, v, out, lse, 0, 0.1, ws)
        assert e.value.status == code
    # out's own memory as the workspace
    ws_alias = out.view(-1).view(torch.uint8)[:need]
    with pytest.raises(eta.AttnError) as e:
        eta.attn_fwd_ws(q, k, v, out, lse, 0, 0.1, ws_alias)
    assert e.value.status == 10
    torch.cuda.synchronize()
    assert (out == 7.0).all()
