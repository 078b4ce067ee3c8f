"""GPU parity: the HIP path through the C ABI against the float64 oracle on the same
seeded inputs, plus on-device properties that hold at any size.

Bar for the five workloads (fp16/bf16 outputs): max-abs <= 1e-2, mean-abs <= 1e-3,
lse max-abs <= 1e-3.  Other shapes use assert_within_derived_bound: per element
max(1e-2, the error the method's two roundings to the input type allow), with the
same mean-abs and lse bars.
"""
import math

import numpy as np
import pytest
import torch

import attn_workloads as aw
import oracle
from parity_util import assert_within_bar, assert_within_derived_bound, errors, run_gpu, workload_rows

pytestmark = pytest.mark.gpu


def _case_id(w, causal):
    return f"{w.name}-causal{causal}"


CASES = [(w, c) for w in aw.WORKLOADS for c in w.causal_modes]


@pytest.mark.parametrize("w,causal", CASES, ids=[_case_id(w, c) for w, c in CASES])
def test_workload_parity(lib, w, causal):
    print(f"\n[case] {_case_id(w, causal)} shape={w.shape} dtype={w.dtype}", flush=True)
    q, k, v = aw.workload_inputs(w)
    out, lse = run_gpu(q, k, v, causal, w.scale)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = workload_rows(w)
    err = errors(out, lse, q, k, v, causal, w.scale, rows=rows)
    print(f"[err] {err}", flush=True)
    assert_within_bar(err, _case_id(w, causal))
    if rows is not None and causal:
        # the first rows carry the largest |O| under a causal mask
        err0 = errors(out, lse, q, k, v, causal, w.scale, rows=np.arange(64))
        print(f"[err first 64 rows] {err0}", flush=True)
        assert_within_bar(err0, _case_id(w, causal) + " rows 0..63")


EDGE_N = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 255, 257]


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [0, 1])
def test_edge_shapes(lib, d, dtype, causal):
    for N in EDGE_N:
        q, k, v = aw.make_inputs((1, 2, N, d), dtype, 7000 + N + d)
        scale = 1.0 / math.sqrt(d)
        out, lse = run_gpu(q, k, v, causal, scale)
        assert_within_derived_bound(out, lse, q, k, v, causal, scale, label=f"N={N} d={d} {dtype} causal={causal}")


def test_many_heads_small_n(lib):
    q, k, v = aw.make_inputs((3, 5, 70, 64), "fp16", 11)
    for causal in (0, 1):
        out, lse = run_gpu(q, k, v, causal, 0.125)
        assert_within_derived_bound(out, lse, q, k, v, causal, 0.125, label=f"causal={causal}")


def test_single_head_long_sequence(lib):
    q, k, v = aw.make_inputs((1, 1, 8192, 128), "bf16", 12)
    out, lse = run_gpu(q, k, v, 1, 1 / math.sqrt(128))
    rows = np.unique(np.concatenate([np.arange(64), np.random.default_rng(3).choice(8192, 256, replace=False), [8191]]))
    assert_within_derived_bound(out, lse, q, k, v, 1, 1 / math.sqrt(128), rows=rows)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_causal_row0_is_v0_bitwise(lib, dtype):
    q, k, v = aw.make_inputs((2, 3, 200, 128), dtype, 13)
    out, lse = run_gpu(q, k, v, 1, 0.3)
    assert torch.equal(out[:, :, 0].view(torch.int16), v[:, :, 0].view(torch.int16))
    s64 = np.float64(np.float32(0.3))
    want = s64 * np.einsum("bhd,bhd->bh", q[:, :, 0].double().numpy(), k[:, :, 0].double().numpy())
    assert np.abs(lse[:, :, 0].double().numpy() - want).max() <= 1e-3


@pytest.mark.parametrize("causal", [0, 1])
def test_constant_v_gives_constant_output(lib, causal):
    q, k, _ = aw.make_inputs((1, 4, 300, 80), "fp16", 14)
    c = torch.linspace(-3, 3, 80, dtype=torch.float16)
    v = c.expand(1, 4, 300, 80).contiguous()
    out, _ = run_gpu(q, k, v, causal, 1 / math.sqrt(80))
    tol = 2.0 ** -8 * c.abs().double().numpy() + 1e-6
    assert (np.abs(out.double().numpy() - c.double().numpy()) <= tol).all()


def test_zero_q_gives_prefix_means(lib):
    _, k, v = aw.make_inputs((1, 2, 130, 64), "fp16", 15)
    q = torch.zeros_like(k)
    for causal in (0, 1):
        out, lse = run_gpu(q, k, v, causal, 0.125)
        vv = v.double().numpy()
        cnt = np.arange(1, 131)[None, None, :]
        want = np.cumsum(vv, axis=2) / cnt[..., None] if causal else vv.mean(axis=2, keepdims=True)
        assert np.abs(out.double().numpy() - want).max() <= 1e-2
        want_lse = np.log(cnt) if causal else np.full(cnt.shape, math.log(130))
        assert np.abs(lse.double().numpy() - want_lse).max() <= 1e-3


def test_key_value_permutation_invariance(lib):
    q, k, v = aw.make_inputs((1, 2, 257, 128), "bf16", 16)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(257))
    o1, l1 = run_gpu(q, k, v, 0, 0.09)
    o2, l2 = run_gpu(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), 0, 0.09)
    assert (o1.double() - o2.double()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("scale", [0.0, -0.125, 2.5])
def test_unusual_scales(lib, scale):
    q, k, v = aw.make_inputs((1, 2, 100, 64), "fp16", 17)
    for causal in (0, 1):
        out, lse = run_gpu(q, k, v, causal, scale)
        assert_within_derived_bound(out, lse, q, k, v, causal, scale, label=f"scale={scale} causal={causal}")


def test_outliers_stress_rescaling(lib):
    q, k, v = aw.make_inputs((1, 2, 1000, 128), "bf16", 18, outlier_fraction=0.02, outlier_factor=30.0)
    for causal in (0, 1):
        out, lse = run_gpu(q, k, v, causal, 1 / math.sqrt(128))
        assert_within_derived_bound(out, lse, q, k, v, causal, 1 / math.sqrt(128), label=f"causal={causal}")


def test_deterministic(lib):
    q, k, v = aw.make_inputs((2, 4, 1000, 128), "bf16", 19)
    o1, l1 = run_gpu(q, k, v, 1, 0.088)
    o2, l2 = run_gpu(q, k, v, 1, 0.088)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_lse_optional(lib):
    q, k, v = aw.make_inputs((1, 2, 150, 64), "bf16", 20)
    o1, l1 = run_gpu(q, k, v, 1, 0.125)
    o2, l2 = run_gpu(q, k, v, 1, 0.125, with_lse=False)
    assert l2 is None and torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("causal", [0, 1])
def test_guard_bands_untouched(lib, causal):
    import exact_tiled_attention_03_amd as eta
    B, H, N, d = 1, 3, 333, 80
    q, k, v = (t.cuda() for t in aw.make_inputs((B, H, N, d), "fp16", 21))
    n = B * H * N * d
    pad = 4096
    obuf = torch.full((n + 2 * pad,), 7.25, dtype=torch.float16, device="cuda")
    lbuf = torch.full((B * H * N + 2 * pad,), -3.5, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n].view(B, H, N, d)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    eta.attn_fwd(q, k, v, out, lse, causal, 0.11)
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7.25).all() and (obuf[pad + n:] == 7.25).all()
    assert (lbuf[:pad] == -3.5).all() and (lbuf[pad + B * H * N:] == -3.5).all()
    assert_within_derived_bound(out.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(), causal, 0.11)


def test_non_default_stream(lib):
    import exact_tiled_attention_03_amd as eta
    q, k, v = (t.cuda() for t in aw.make_inputs((2, 2, 500, 128), "bf16", 22))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], device="cuda")
        eta.attn_fwd(q, k, v, out, lse, True, 0.088, stream=s)
    s.synchronize()
    assert_within_derived_bound(out.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(), 1, 0.088)


def test_rejects_misaligned_and_leaves_output(lib):
    import exact_tiled_attention_03_amd as eta
    q, k, v = (t.cuda() for t in aw.make_inputs((1, 1, 64, 64), "fp16", 23))
    big = torch.full((64 * 64 + 8,), 1.5, dtype=torch.float16, device="cuda")
    out = big[1:1 + 64 * 64].view(1, 1, 64, 64)   # 2-byte offset: not 16-byte aligned
    with pytest.raises(eta.AttnError) as ei:
        eta.attn_fwd(q, k, v, out, None, True, 0.125)
    assert ei.value.status == 6
    torch.cuda.synchronize()
    assert (big == 1.5).all()


# Shapes with 512 heads select the 8-wave schedule even for short sequences,
# so its masking, ragged tails and head dims are covered at small N.
PP_N = [1, 65, 200, 256, 257, 300, 513]


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [0, 1])
def test_wide_schedule_edge_shapes(lib, d, dtype, causal):
    for N in PP_N:
        assert lib.attn_fwd_schedule(8, 64, N, d, causal) == lib.ATTN_SCHEDULE_WIDE
        q, k, v = aw.make_inputs((8, 64, N, d), dtype, 9000 + N + d)
        scale = 1.0 / math.sqrt(d)
        out, lse = run_gpu(q, k, v, causal, scale)
        assert_within_derived_bound(out, lse, q, k, v, causal, scale, label=f"wide N={N} d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("scale", [0.0, -0.125])
def test_wide_schedule_unusual_scales(lib, scale):
    q, k, v = aw.make_inputs((8, 64, 130, 64), "bf16", 31)
    for causal in (0, 1):
        assert lib.attn_fwd_schedule(8, 64, 130, 64, causal) == lib.ATTN_SCHEDULE_WIDE
        out, lse = run_gpu(q, k, v, causal, scale)
        assert_within_derived_bound(out, lse, q, k, v, causal, scale, label=f"wide scale={scale} causal={causal}")


def test_wide_schedule_long_causal_rows_and_outliers(lib):
    q, k, v = aw.make_inputs((4, 128, 600, 128), "bf16", 32, outlier_fraction=0.02, outlier_factor=30.0)
    assert lib.attn_fwd_schedule(4, 128, 600, 128, 1) == lib.ATTN_SCHEDULE_WIDE
    out, lse = run_gpu(q, k, v, 1, 1 / math.sqrt(128))
    assert_within_derived_bound(out, lse, q, k, v, 1, 1 / math.sqrt(128))
    assert torch.equal(out[:, :, 0].view(torch.int16), v[:, :, 0].view(torch.int16))


# d = 64 shapes with N >= 2048 (causal: N >= 4096) and fewer than 512 work-groups
# of 128 queries take the key-split form of the 8-wave schedule: waves w and w+4
# hold the same rows, each over one half of the query tile's key tiles, merged at
# the end.  The shapes give items with one tile (second half empty), odd counts
# (halves differ by one) and even counts, ragged N and rows past N.
SPLIT_SHAPES = {0: [(1, 1, 2048), (1, 2, 2049), (2, 1, 2111), (1, 1, 3000)],
                1: [(1, 1, 4096), (1, 2, 4097), (2, 1, 4159), (1, 1, 4500)]}


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [0, 1])
def test_key_split_schedule(lib, dtype, causal):
    for B, H, N in SPLIT_SHAPES[causal]:
        assert lib.attn_fwd_schedule(B, H, N, 64, causal) == lib.ATTN_SCHEDULE_SPLIT
        print(f"\n[case] split B={B} H={H} N={N} {dtype} causal={causal}", flush=True)
        q, k, v = aw.make_inputs((B, H, N, 64), dtype, 9500 + N)
        out, lse = run_gpu(q, k, v, causal, 0.125)
        assert_within_derived_bound(out, lse, q, k, v, causal, 0.125, label=f"split N={N} {dtype} causal={causal}")
        if causal:
            assert torch.equal(out[:, :, 0].view(torch.int16), v[:, :, 0].view(torch.int16))


def test_key_split_merge_with_outliers(lib):
    # the two halves reach very different row maxima: the merge rescales both
    for causal, N in ((0, 2100), (1, 4200)):
        q, k, v = aw.make_inputs((2, 3, N, 64), "fp16", 9600, outlier_fraction=0.02, outlier_factor=30.0)
        assert lib.attn_fwd_schedule(2, 3, N, 64, causal) == lib.ATTN_SCHEDULE_SPLIT
        for scale in (0.125, -0.2):
            out, lse = run_gpu(q, k, v, causal, scale)
            rows = np.unique(np.concatenate([np.arange(200), np.random.default_rng(5).choice(N, 300, replace=False), [N - 1]]))
            assert_within_derived_bound(out, lse, q, k, v, causal, scale, rows=rows,
                                        label=f"split outliers causal={causal} scale={scale}")


# Causal 4-wave grids whose single query tiles fit one round of two work-groups
# per CU run them unpaired, longest first from both ends of one list: tile counts
# that are odd or end inside a tile index's run of heads must still give every
# tile to exactly one work-group (a missed tile leaves its rows unwritten).
UNPAIRED_SHAPES = [(1, 3, 640, 64, "fp16"), (2, 5, 1100, 80, "bf16"), (1, 7, 1000, 128, "fp16"), (1, 1, 300, 64, "bf16")]


@pytest.mark.parametrize("B,H,N,d,dtype", UNPAIRED_SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}-{s[4]}" for s in UNPAIRED_SHAPES])
def test_unpaired_causal_tiles(lib, B, H, N, d, dtype):
    assert lib.attn_fwd_schedule(B, H, N, d, 1) == lib.ATTN_SCHEDULE_SMALL
    print(f"\n[case] unpaired B={B} H={H} N={N} d={d} {dtype}", flush=True)
    q, k, v = aw.make_inputs((B, H, N, d), dtype, 9800 + N + d)
    out, lse = run_gpu(q, k, v, 1, 1.0 / math.sqrt(d))
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert_within_derived_bound(out, lse, q, k, v, 1, 1.0 / math.sqrt(d), label=f"unpaired B={B} H={H} N={N} d={d}")


def test_small_schedule_d64(lib):
    # 512 work-groups of 128 queries: the 4-wave schedule without the key split
    for causal, (B, H, N) in ((1, (8, 32, 512)), (0, (4, 32, 512))):
        assert lib.attn_fwd_schedule(B, H, N, 64, causal) == lib.ATTN_SCHEDULE_SMALL
        q, k, v = aw.make_inputs((B, H, N, 64), "bf16", 9700 + causal)
        out, lse = run_gpu(q, k, v, causal, 0.125)
        rows = np.unique(np.concatenate([np.arange(70), np.arange(N - 70, N)]))
        assert_within_derived_bound(out, lse, q, k, v, causal, 0.125, rows=rows, label=f"small d64 causal={causal}")
