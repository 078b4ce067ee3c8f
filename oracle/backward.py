"""Gradients of the exact attention forward, and the merge of attention results
computed over disjoint key shards, in float64 on the CPU: the oracles of the
backward kernels and of the merge kernel.

TEST INFRASTRUCTURE ONLY.  It is imported by the tests, by the smoke check and
by the benchmark's CPU-baseline leg, and by nothing else; the HIP library and
its binding never call it and share no code with it.

The pages name fused backward operators only in passing ("Triton: CUDA-level
operators in Python", section on why Triton) and give no algorithm, so this is
the derivative of the forward definition ("Triton in depth" 3.1), written out:
with S = scale * Q K^T (masked entries -inf), P = softmax_rows(S), O = P V and
an upstream gradient dO,

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - D),   D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic
    dQ = scale * dS K
    dK = scale * dS^T Q

(the softmax Jacobian applied row by row; masked entries have P = 0, so they
receive no gradient).  The forward's lse is not needed here: P is rebuilt from
the definition.

The merge follows from the definition of lse (reading R9 of the forward,
lse_i = ln sum_j exp(S_ij)): if key set J is split into shards J_g with partial
results (O_g, lse_g), then lse = ln sum_g exp(lse_g) and
O = sum_g exp(lse_g - lse) O_g.  A shard with no kept key for a row has
lse_g = -inf and weight 0.

Pinned by tests/test_oracle_bwd_pins.py; no function here is unpinned.
"""
from __future__ import annotations

import numpy as np

from .attention import softmax_weights


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def attention_bwd(q, k, v, do, causal: int, scale: float, window: int = 0):
    """q, k, v, do: [B, H, N, d].  Returns float64 (dq, dk, dv), each [B, H, N, d]."""
    Q, K, V, dO = (_f64(t) for t in (q, k, v, do))
    P = softmax_weights(Q, K, causal, scale, window=window)      # [B, H, N, N], float64
    O = P @ V
    dV = np.swapaxes(P, -1, -2) @ dO
    dP = dO @ np.swapaxes(V, -1, -2)
    D = (dO * O).sum(axis=-1, keepdims=True)
    dS = P * (dP - D)
    s = float(np.float32(scale))
    dQ = s * (dS @ K)
    dK = s * (np.swapaxes(dS, -1, -2) @ Q)
    return dQ, dK, dV


def lse_merge(o_parts, lse_parts):
    """o_parts: [G, ..., N, d]; lse_parts: [G, ..., N] (natural log, -inf for an empty
    shard).  Returns float64 (o [..., N, d], lse [..., N])."""
    Og, Lg = _f64(o_parts), _f64(lse_parts)
    m = Lg.max(axis=0)
    finite = np.isfinite(m)
    mm = np.where(finite, m, 0.0)
    w = np.exp(Lg - mm[None])                                     # exp(-inf) = 0 for empty shards
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(finite, mm + np.log(tot), -np.inf)
        o = (w[..., None] * Og).sum(axis=0) / tot[..., None]
    return o, lse
