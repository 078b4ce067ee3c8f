"""GPU check of attn_bwd_noalloc (include/attn_bwd.h), the backward entry point for
callers that cannot allocate: through the C ABI it must give exactly what attn_bwd
gives with a caller-provided delta workspace (the same kernels, so bit for bit),
on two calls in a row where the second is smaller than the first (the device
array then still holds the first call's rows past the second's), and stay within
the backward's bar against the float64 oracle."""
import math

import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
from test_bwd_gpu import bwd_inputs, check_bwd

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def both_entry_points(shape, dtype, seed, causal):
    scale = 1.0 / math.sqrt(shape[3])
    q, k, v, do, out, lse = bwd_inputs(shape, dtype, seed, causal, scale)
    g = [t.cuda() for t in (q, k, v, out, lse, do)]
    ref = eta.attn_bwd(*g, causal=causal, scale=scale)[:3]
    got = tuple(torch.full_like(g[0], float("nan")) for _ in range(3))
    eta.attn_bwd_noalloc(*g, *got, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, do, scale), ref, got


@pytest.mark.parametrize("first,second", [
    (((2, 4, 700, 128), "bf16", 1), ((1, 2, 300, 64), "fp16", 0)),
    (((1, 3, 1000, 80), "fp16", 0), ((2, 1, 129, 128), "bf16", 1)),
])
def test_noalloc_matches_attn_bwd_on_two_calls(lib, first, second):
    for i, (shape, dtype, causal) in enumerate((first, second)):
        print(f"\n[case] bwd_noalloc call {i + 1}: {shape} {dtype} causal={causal}", flush=True)
        (q, k, v, do, scale), ref, got = both_entry_points(shape, dtype, 6100 + 10 * i + shape[2], causal)
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(r.view(torch.int16), g.view(torch.int16)), f"{name} differs from attn_bwd"
        check_bwd(tuple(t.cpu() for t in got), q, k, v, do, causal, scale, dtype, f"noalloc {shape} {dtype}")


def test_noalloc_rejects_rows_past_its_array(lib):
    # the row limit is checked on the host before any device work
    rows = 4194304
    base = 0x10000
    sz = 1 << 24
    l = eta.load_library()
    ptrs = [base + i * sz for i in range(9)]
    assert l.attn_bwd_noalloc(*ptrs, 1, 1, rows + 1, 64, 1, 0.125, eta.ATTN_BF16, None) == 2
    assert l.attn_bwd_noalloc(*ptrs, 2, 2, rows // 4 + 1, 64, 1, 0.125, eta.ATTN_BF16, None) == 2
