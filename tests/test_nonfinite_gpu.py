"""Non-finite inputs.  The header leaves unspecified the rows whose scores meet a
NaN or an infinite element of q, k or v; the call must still succeed, and every
row whose scores and values are all finite must match the oracle: the running
max, sum and rescale are kept per query row, and nothing is shared across rows
of a wave.  The expected rows are checked against the oracle on the clean inputs,
which give those rows exactly the same scores and values."""
import math

import numpy as np
import pytest

import attn_workloads as aw
from parity_util import assert_within_derived_bound, run_gpu

pytestmark = pytest.mark.gpu

BAD = {"nan": math.nan, "+inf": math.inf, "-inf": -math.inf}
N = 700


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (80, "fp16"), (64, "fp16")])
@pytest.mark.parametrize("bad", list(BAD))
def test_causal_rows_before_a_bad_key(lib, d, dtype, bad):
    """Key j of head 1 holds a non-finite element: under the causal mask rows 0..j-1
    never see it, and head 0 does not hold it at all."""
    j = 333
    print(f"\n[case] causal B=1 H=2 N={N} d={d} {dtype}, k[0,1,{j},5] = {bad}", flush=True)
    q, k, v = aw.make_inputs((1, 2, N, d), dtype, 8100 + d)
    k_bad = k.clone()
    k_bad[0, 1, j, 5] = BAD[bad]
    scale = 1.0 / math.sqrt(d)
    out, lse = run_gpu(q, k_bad, v, 1, scale)
    assert_within_derived_bound(out[:, :1], lse[:, :1], q[:, :1], k[:, :1], v[:, :1], 1, scale,
                                label=f"head 0, {bad}")
    assert_within_derived_bound(out[:, 1:], lse[:, 1:], q[:, 1:], k[:, 1:], v[:, 1:], 1, scale,
                                rows=np.arange(j), label=f"head 1 rows before {j}, {bad}")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (80, "fp16")])
@pytest.mark.parametrize("bad", list(BAD))
def test_unmasked_rows_beside_a_bad_query(lib, d, dtype, bad):
    """Query row i of head 1 holds a non-finite element: only that row's scores meet
    it, so every other row, including the rows of its own wave, stays exact."""
    i = 290
    print(f"\n[case] non-causal B=1 H=2 N={N} d={d} {dtype}, q[0,1,{i},7] = {bad}", flush=True)
    q, k, v = aw.make_inputs((1, 2, N, d), dtype, 8200 + d)
    q_bad = q.clone()
    q_bad[0, 1, i, 7] = BAD[bad]
    scale = 1.0 / math.sqrt(d)
    out, lse = run_gpu(q_bad, k, v, 0, scale)
    keep = np.array([r for r in range(N) if r != i])
    assert_within_derived_bound(out, lse, q, k, v, 0, scale, rows=keep, label=f"rows other than {i}, {bad}")
