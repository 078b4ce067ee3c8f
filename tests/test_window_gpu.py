"""GPU parity of the sliding-window entry point attn_fwd_window against the
float64 oracle (same window reading, pinned in test_oracle_window_pins.py), with
the derived per-element bar of parity_util, plus exact properties of the band."""
import math

import numpy as np
import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
from parity_util import assert_within_derived_bound, run_gpu

pytestmark = pytest.mark.gpu

WINDOWS = [1, 2, 17, 63, 64, 65, 128, 200, 299, 300, 1000]


@pytest.mark.parametrize("d,dtype", [(64, "fp16"), (80, "fp16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [0, 1])
def test_window_parity_small_schedule(lib, d, dtype, causal):
    N = 300
    q, k, v = aw.make_inputs((1, 2, N, d), dtype, 9100 + d)
    scale = 1.0 / math.sqrt(d)
    for w in WINDOWS:
        print(f"\n[case] window N={N} d={d} {dtype} causal={causal} W={w}", flush=True)
        out, lse = run_gpu(q, k, v, causal, scale, window=w)
        assert_within_derived_bound(out, lse, q, k, v, causal, scale, window=w,
                                    label=f"N={N} d={d} {dtype} causal={causal} W={w}")


@pytest.mark.parametrize("causal", [0, 1])
def test_window_parity_wide_schedule(lib, causal):
    # 8 x 64 heads of 300 rows: 512 groups of 256 queries -> the 8-wave schedule
    B, H, N, d = 8, 64, 300, 128
    assert eta.attn_fwd_schedule(B, H, N, d, causal) == eta.ATTN_SCHEDULE_WIDE
    q, k, v = aw.make_inputs((B, H, N, d), "bf16", 9200 + causal)
    rows = np.unique(np.concatenate([np.arange(8), np.random.default_rng(5).choice(N, 40, replace=False), [N - 1]]))
    for w in (1, 33, 100, 257):
        print(f"\n[case] wide window causal={causal} W={w}", flush=True)
        out, lse = run_gpu(q, k, v, causal, 1 / math.sqrt(d), window=w)
        assert_within_derived_bound(out, lse, q, k, v, causal, 1 / math.sqrt(d), rows=rows, window=w,
                                    label=f"wide causal={causal} W={w}")


@pytest.mark.parametrize("causal", [0, 1])
def test_window_long_sequence_sampled_rows(lib, causal):
    N, d, w = 4096, 128, 512
    q, k, v = aw.make_inputs((1, 4, N, d), "bf16", 9300 + causal)
    rows = np.unique(np.concatenate([np.arange(4), np.random.default_rng(6).choice(N, 200, replace=False),
                                     np.arange(w - 3, w + 3), [N - 1]]))
    out, lse = run_gpu(q, k, v, causal, 1 / math.sqrt(d), window=w)
    assert_within_derived_bound(out, lse, q, k, v, causal, 1 / math.sqrt(d), rows=rows, window=w,
                                label=f"N={N} causal={causal} W={w}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [0, 1])
def test_window_one_is_v_bitwise(lib, dtype, causal):
    q, k, v = aw.make_inputs((2, 3, 150, 64), dtype, 9400)
    out, lse = run_gpu(q, k, v, causal, 0.3, window=1)
    assert torch.equal(out.view(torch.int16), v.view(torch.int16))
    s64 = np.float64(np.float32(0.3))
    want = s64 * np.einsum("bhnd,bhnd->bhn", q.double().numpy(), k.double().numpy())
    assert np.abs(lse.double().numpy() - want).max() <= 1e-3


@pytest.mark.parametrize("causal", [0, 1])
def test_window_at_least_n_equals_full_attention(lib, causal):
    q, k, v = aw.make_inputs((2, 2, 333, 128), "bf16", 9500)
    full, lfull = run_gpu(q, k, v, causal, 0.09)
    for w in (333, 334, 100000):
        out, lse = run_gpu(q, k, v, causal, 0.09, window=w)
        assert torch.equal(out.view(torch.int16), full.view(torch.int16))
        assert torch.equal(lse, lfull)


@pytest.mark.parametrize("causal", [0, 1])
def test_window_band_locality(lib, causal):
    # moving K/V rows just outside row i's band leaves row i bit-identical
    N, w, i = 512, 100, 300
    q, k, v = aw.make_inputs((1, 1, N, 64), "fp16", 9600)
    out, lse = run_gpu(q, k, v, causal, 0.125, window=w)
    k2, v2 = k.clone(), v.clone()
    outside = [i - w] + ([] if causal else [i + w])
    for j in outside:
        k2[0, 0, j] = -k2[0, 0, j]
        v2[0, 0, j] = 2 * v2[0, 0, j]
    out2, lse2 = run_gpu(q, k2, v2, causal, 0.125, window=w)
    assert torch.equal(out2[0, 0, i].view(torch.int16), out[0, 0, i].view(torch.int16))
    assert lse2[0, 0, i] == lse[0, 0, i]


def test_window_outliers_and_rescale(lib):
    q, k, v = aw.make_inputs((2, 4, 1111, 80), "fp16", 9700, outlier_fraction=0.01, outlier_factor=20.0)
    for causal in (0, 1):
        for w in (50, 300):
            out, lse = run_gpu(q, k, v, causal, 1 / math.sqrt(80), window=w)
            assert_within_derived_bound(out, lse, q, k, v, causal, 1 / math.sqrt(80), window=w,
                                        label=f"outliers causal={causal} W={w}")


def test_window_negative_rejected(lib):
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(eta.AttnError) as ei:
        eta.attn_fwd(q, q, q, out, None, True, 0.1, window=-3)
    assert ei.value.status == 11
    torch.cuda.synchronize()
    assert (out == 7.0).all()


# Causal windowed problems give every query tile its own work unit (no causal
# pairs): odd tile counts, for both launch shapes, every row of the checked heads.
@pytest.mark.parametrize("B,H,N,d,w", [(8, 64, 5 * 256 - 3, 64, 300), (1, 3, 7 * 128 - 5, 80, 200)],
                         ids=["wide-5-tiles", "small-7-tiles"])
def test_window_causal_every_tile_of_odd_counts(lib, B, H, N, d, w):
    want = eta.ATTN_SCHEDULE_WIDE if B * H >= 512 else eta.ATTN_SCHEDULE_SMALL
    assert eta.attn_fwd_schedule(B, H, N, d, 1) == want
    print(f"\n[case] window causal B={B} H={H} N={N} d={d} W={w}", flush=True)
    q, k, v = aw.make_inputs((B, H, N, d), "fp16", 9700 + N)
    out, lse = run_gpu(q, k, v, 1, 1 / math.sqrt(d), window=w)
    heads = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        assert_within_derived_bound(out[sl], lse[sl], q[sl], k[sl], v[sl], 1, 1 / math.sqrt(d), window=w,
                                    label=f"head ({b},{h}) N={N} W={w}")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
