"""Exact attention forward in float64 on the CPU: the oracle.

TEST INFRASTRUCTURE ONLY.  It is imported by the tests, by the smoke check and
by the benchmark's CPU-baseline leg, and by nothing else; the HIP library and
its binding never call it and share no code with it.

What it computes is the plain definition of the forward pass that the tiled
method reaches exactly (the pages: "Triton in depth", section 3.1 gives
softmax(Q K^T / sqrt(d)) V; section 3.2 states that tiling with online
statistics (m, l) yields the exact result without storing the N x N matrix;
"CS336 Lecture 6", Level 1 softmax, gives the max-subtracted softmax):

    S      = scale * Q K^T                      (N x N, materialised here)
    S[i,j] = -inf  where causal and j > i       ("Triton in depth" 3.3: a key is
                                                 kept when its index <= the query's)
    m_i    = max_j S[i,j]
    P      = exp(S - m)                         (masked entries give exp(-inf) = 0,
                                                 Level 1 softmax padding rule)
    l_i    = sum_j P[i,j]
    O_i    = (sum_j P[i,j] V_j) / l_i
    lse_i  = m_i + ln(l_i)                      (natural log of sum_j exp(S[i,j]))

Sliding window (the pages name sliding-window attention among the custom
attention variants a tiled kernel is suited to, "Triton: CUDA-level operators
in Python", section "when to use Triton", without defining it; the reading
taken here is the usual local band).  With window W >= 1 a key j is kept for
query i only if, in addition to the causal rule,

    i - W < j                (the W most recent keys, the diagonal included)
    j < i + W                (non-causal only: the symmetric band |i - j| < W)

and W = 0 means no window.  Every row keeps at least key i.

All arithmetic is float64 on the exact input values (fp16/bf16 upcast).  The
scale is taken as float64(float32(scale)), i.e. exactly the float32 value the
library receives.  The logsumexp output is not on the pages; it is the natural
log of the row's softmax denominator over the scaled scores.

Pinned by tests/test_oracle_pins.py (brute force, closed forms, invariants and
a library special case); no function here is unpinned.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """torch tensor (any float dtype, CPU) or ndarray -> float64 ndarray."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _scale64(scale: float) -> np.float64:
    return np.float64(np.float32(scale))


def _head(qh, kh, vh, causal: bool, scale64, rows, window: int = 0):
    """One (b, h): qh [N, d], kh [N, d], vh [N, d]; rows = query indices to produce.

    Returns O [R, d], lse [R], W [R, N] (the normalised softmax weights)."""
    s = scale64 * (qh[rows] @ kh.T)                       # [R, N]
    j = np.arange(kh.shape[0])[None, :]
    i = rows[:, None]
    if causal:
        s = np.where(j > i, -np.inf, s)
    if window > 0:
        s = np.where(j <= i - window, -np.inf, s)
        if not causal:
            s = np.where(j >= i + window, -np.inf, s)
    m = s.max(axis=1)                                     # every row keeps key i, so m is finite
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (p @ vh) / l[:, None]
    lse = m + np.log(l)
    return o, lse, p / l[:, None]


def _rows_for(rows, b, h, n):
    if rows is None:
        return np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    return rows if rows.ndim == 1 else rows[b, h]


def attention(q, k, v, causal, scale, rows=None, window=0):
    """Exact attention forward.

    q, k, v : [B, H, N, d] (torch CPU tensors or arrays, any float dtype)
    causal  : truthy for the causal mask (key j kept iff j <= i)
    scale   : the score scale (used as float64(float32(scale)))
    rows    : None for every query row, an int array [R] of rows used for every
              head, or [B, H, R] per head
    window  : 0 for none, else W >= 1: key j also needs i - W < j (and j < i + W
              when not causal)
    returns : O [B, H, R, d] float64, lse [B, H, R] float64 (natural log)
    """
    window = int(window)
    if window < 0:
        raise ValueError("window must be >= 0")
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    s64 = _scale64(scale)
    R = N if rows is None else np.asarray(rows).shape[-1]
    O = np.empty((B, H, R, d))
    L = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            r = _rows_for(rows, b, h, N)
            O[b, h], L[b, h], _ = _head(q[b, h], k[b, h], v[b, h], bool(causal), s64, r, window)
    return O, L


def softmax_weights(q, k, causal, scale, window=0):
    """The normalised weights P/l [B, H, N, N] of the definition (small shapes only)."""
    q, k = _f64(q), _f64(k)
    B, H, N, d = q.shape
    s64 = _scale64(scale)
    W = np.empty((B, H, N, N))
    zeros = np.zeros((N, 1))
    for b in range(B):
        for h in range(H):
            _, _, W[b, h] = _head(q[b, h], k[b, h], zeros, bool(causal), s64, np.arange(N), int(window))
    return W
