"""The seeded input recipe: deterministic, shaped as stated, outliers where stated."""
import numpy as np
import torch

import attn_workloads as aw


def test_same_seed_same_bytes():
    a = aw.make_inputs((1, 2, 33, 16), "bf16", 7)
    b = aw.make_inputs((1, 2, 33, 16), "bf16", 7)
    c = aw.make_inputs((1, 2, 33, 16), "bf16", 8)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a[0], c[0])


def test_cast_is_round_to_nearest_even_of_the_fp32_draw():
    q32, _, _ = aw.draw_fp32((2, 3, 5, 8), 11)
    q16, _, _ = aw.make_inputs((2, 3, 5, 8), "fp16", 11)
    assert q16.dtype == torch.float16 and q16.is_contiguous()
    assert np.array_equal(q16.numpy(), q32.astype(np.float16))


def test_workload_table():
    assert len(aw.WORKLOADS) == 5
    h = aw.WORKLOADS[aw.HEADLINE]
    assert (h.B, h.H, h.N, h.d, h.dtype, h.causal_modes) == (2, 32, 4096, 128, "bf16", (1,))
    assert abs(h.flops(1) - 274.877906944e9) < 1.0
    assert [w.seed for w in aw.WORKLOADS] == [1000, 1001, 1002, 1003, 1004]


def test_outlier_fraction_and_factor():
    shape = (2, 2, 300, 80)
    q, k, v = aw.draw_fp32(shape, 5, 0.01, 20.0)
    q0, k0, v0 = aw.draw_fp32(shape, 5)
    rq = np.abs(q / q0)
    scaled = np.isclose(rq, 20.0)
    assert np.all(np.isclose(rq, 1.0) | scaled)
    frac = scaled.mean()
    assert 0.007 < frac < 0.013
    assert np.array_equal(v, v0)


def test_sample_rows():
    r = aw.sample_rows(1, 3, 1000, 64, 3)
    assert r.shape == (1, 3, 64)
    for h in range(3):
        row = r[0, h]
        assert row[0] == 0 and row[-1] == 999
        assert np.all(np.diff(row) > 0)
    assert np.array_equal(r, aw.sample_rows(1, 3, 1000, 64, 3))
