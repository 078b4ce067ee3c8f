"""The derived per-element bound used for shapes beyond the five workloads admits
the rounding the method prescribes and still rejects plausible kernel mistakes.

A numpy model of the kernel arithmetic (fp32 scores, exp2 with the scale folded,
P rounded to the input type before P V, fp32 accumulation, one division by l,
output rounded to the input type) stands in for the GPU output here."""
import math

import numpy as np
import pytest
import torch

import attn_workloads as aw
from parity_util import assert_within_derived_bound


def model_kernel(q, k, v, causal, scale, *, drop_diag=False, scale_err=0.0, skip_last_key=False):
    dt = q.dtype
    B, H, N, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(B, H, N)
    c = np.float32(scale * (1 + scale_err)) * np.float32(1.4426950408889634)
    for b in range(B):
        for h in range(H):
            s = (q[b, h].float() @ k[b, h].float().T).numpy()
            j = np.arange(N)[None, :]
            i = np.arange(N)[:, None]
            bad = np.zeros((N, N), bool)
            if causal:
                bad = (j >= i) & (j > 0) if drop_diag else j > i
            if skip_last_key:
                bad = bad | (j == N - 1)
            t = np.where(bad, -np.inf, s * c).astype(np.float32)
            m = t.max(1)
            p = np.exp2(t - m[:, None]).astype(np.float32)
            pr = torch.from_numpy(p).to(dt).float().numpy()
            acc = pr @ v[b, h].float().numpy()
            out[b, h] = torch.from_numpy(acc / p.sum(1)[:, None]).to(dt)
            lse[b, h] = torch.from_numpy((m + np.log2(p.sum(1))) * np.float32(math.log(2)))
    return out, lse


def case():
    N, d = 255, 64
    q, k, v = aw.make_inputs((1, 2, N, d), "bf16", 7000 + N + d)
    return q, k, v, 1.0 / math.sqrt(d)


def test_method_rounding_passes_derived_bound_but_not_plain_bar():
    q, k, v, scale = case()
    out, lse = model_kernel(q, k, v, 1, scale)
    assert_within_derived_bound(out, lse, q, k, v, 1, scale)
    import oracle
    O, _ = oracle.attention(q, k, v, 1, scale)
    assert np.abs(out.double().numpy() - O).max() > 1e-2   # the plain bar alone would reject it


@pytest.mark.parametrize("mistake", [dict(drop_diag=True), dict(scale_err=0.01), dict(skip_last_key=True)],
                         ids=["diagonal_dropped", "scale_off_1pct", "last_key_dropped"])
def test_derived_bound_rejects_mistakes(mistake):
    q, k, v, scale = case()
    out, lse = model_kernel(q, k, v, 1 if "drop_diag" in mistake else 0, scale, **mistake)
    with pytest.raises(AssertionError):
        assert_within_derived_bound(out, lse, q, k, v, 1 if "drop_diag" in mistake else 0, scale)
