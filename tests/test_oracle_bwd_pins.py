"""Pins for the attention-gradient and shard-merge oracles (oracle/backward.py),
from facts the definition fixes:

  B1  torch.autograd in CPU float64 through the forward definition, causal and
      not, with and without a window (library derivative, independent of the
      written-out formulas)
  B2  central finite differences of L = sum(O * dO) computed by the forward
      oracle, on a tiny head
  B3  N = 1: dV = dO and dQ = dK = 0
  B4  invariants: rows of P sum to 1, so the column sums of dV equal those of dO,
      and rows of dS sum to 0, so the column sums of dK are 0
  B5  all rows of V equal: O does not depend on Q or K, so dQ = dK = 0
  B6  causal row 0 sees only key 0: dQ_0 = 0
  M1  keys split into shards, each shard's (O, lse) from the forward oracle,
      merged, equals the unsplit forward oracle
  M2  one shard merges to itself; two identical shards add ln 2 to lse
  M3  an empty shard (lse = -inf) contributes nothing

test_bwd_mutants_are_caught plants plausible mistakes in a copy of the formulas
and asserts that some pin rejects each.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def torch_grads(q, k, v, do, causal, scale, window=0):
    Q, K, V = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = float(np.float32(scale))
    S = s * (Q @ K.transpose(-1, -2))
    N = q.shape[-2]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    keep = torch.ones(N, N, dtype=torch.bool)
    if causal:
        keep &= j <= i
    if window > 0:
        keep &= j > i - window
        if not causal:
            keep &= j < i + window
    S = S.masked_fill(~keep, -math.inf)
    O = torch.softmax(S, dim=-1) @ V
    (O * torch.tensor(do)).sum().backward()
    return Q.grad.numpy(), K.grad.numpy(), V.grad.numpy()


def pin_b1(bwd):
    for n, (causal, window) in enumerate([(0, 0), (1, 0), (1, 5), (0, 4)]):
        q, k, v, do = (rnd((2, 3, 17, 8), 10 * n + i) for i in range(4))
        got = bwd(q, k, v, do, causal, 0.3, window)
        want = torch_grads(q, k, v, do, causal, 0.3, window)
        for g, w_ in zip(got, want):
            assert np.allclose(g, w_, rtol=1e-11, atol=1e-12), (causal, window)


def pin_b2(bwd):
    q, k, v, do = (rnd((1, 1, 5, 3), 50 + i) for i in range(4))
    scale = 0.7

    def loss(q_, k_, v_):
        O, _ = oracle.attention(q_, k_, v_, 1, scale)
        return float((O * do).sum())

    grads = bwd(q, k, v, do, 1, scale, 0)
    h = 1e-6
    for which, g in enumerate(grads):
        fd = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-8), which


def pin_b3(bwd):
    q, k, v, do = (rnd((2, 2, 1, 6), 60 + i) for i in range(4))
    dq, dk, dv = bwd(q, k, v, do, 1, 0.5, 0)
    assert np.allclose(dv, do, rtol=0, atol=1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15


def pin_b4(bwd):
    for causal in (0, 1):
        q, k, v, do = (rnd((2, 2, 23, 5), 70 + i) for i in range(4))
        dq, dk, dv = bwd(q, k, v, do, causal, 0.4, 0)
        assert np.allclose(dv.sum(axis=-2), do.sum(axis=-2), rtol=0, atol=1e-12)
        assert np.abs(dk.sum(axis=-2)).max() < 1e-12


def pin_b5(bwd):
    q, k, do = (rnd((1, 2, 11, 4), 80 + i) for i in range(3))
    v = np.broadcast_to(rnd((1, 2, 1, 4), 84), (1, 2, 11, 4)).copy()
    dq, dk, dv = bwd(q, k, v, do, 0, 0.9, 0)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def pin_b6(bwd):
    q, k, v, do = (rnd((1, 1, 9, 4), 90 + i) for i in range(4))
    dq, _, _ = bwd(q, k, v, do, 1, 0.6, 0)
    assert np.abs(dq[0, 0, 0]).max() < 1e-15


def pin_m1(merge):
    q, k, v = (rnd((2, 2, 40, 8), 100 + i) for i in range(3))
    scale = 0.35
    full_o, full_l = oracle.attention(q, k, v, 0, scale)
    cuts = [0, 7, 8, 25, 40]
    parts = [oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0, scale) for a, b in zip(cuts, cuts[1:])]
    o, lse = merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.allclose(o, full_o, rtol=1e-12, atol=1e-13) and np.allclose(lse, full_l, rtol=1e-13, atol=1e-13)


def pin_m2(merge):
    o, l = rnd((2, 3, 9, 5), 110), rnd((2, 3, 9), 111)
    o1, l1 = merge(o[None], l[None])
    assert np.allclose(o1, o, rtol=1e-15, atol=1e-15) and np.allclose(l1, l, rtol=1e-15, atol=1e-15)
    o2, l2 = merge(np.stack([o, o]), np.stack([l, l]))
    assert np.allclose(o2, o, rtol=1e-14, atol=1e-15) and np.allclose(l2, l + math.log(2.0), rtol=1e-14, atol=1e-14)


def pin_m3(merge):
    o, l = rnd((1, 2, 6, 4), 120), rnd((1, 2, 6), 121)
    empty_o, empty_l = np.zeros_like(o), np.full_like(l, -np.inf)
    om, lm = merge(np.stack([empty_o, o, empty_o]), np.stack([empty_l, l, empty_l]))
    assert np.allclose(om, o, rtol=1e-15, atol=1e-15) and np.allclose(lm, l, rtol=1e-15, atol=1e-15)


BWD_PINS = [pin_b1, pin_b2, pin_b3, pin_b4, pin_b5, pin_b6]
MERGE_PINS = [pin_m1, pin_m2, pin_m3]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_oracle_pin(pin):
    pin(ob.attention_bwd)


@pytest.mark.parametrize("pin", MERGE_PINS, ids=lambda f: f.__name__)
def test_merge_oracle_pin(pin):
    pin(ob.lse_merge)


# ----------------------------------------------------------------------------- mutants

def _bwd(q, k, v, do, causal, scale, window=0, *, no_delta=False, dk_unscaled=False, dq_uses_v=False,
         dv_not_transposed=False, delta_from_dp=False):
    P = oracle.softmax_weights(q, k, causal, scale, window=window)
    Q, K, V, dO = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    O = P @ V
    dV = (P if dv_not_transposed else np.swapaxes(P, -1, -2)) @ dO
    dP = dO @ np.swapaxes(V, -1, -2)
    D = dP.sum(axis=-1, keepdims=True) if delta_from_dp else (dO * O).sum(axis=-1, keepdims=True)
    dS = P * dP if no_delta else P * (dP - D)
    s = float(np.float32(scale))
    dQ = s * (dS @ (V if dq_uses_v else K))
    dK = (1.0 if dk_unscaled else s) * (np.swapaxes(dS, -1, -2) @ Q)
    return dQ, dK, dV


def _merge(o_parts, lse_parts, *, unnormalised=False, lse_is_max=False):
    Og, Lg = np.asarray(o_parts, dtype=np.float64), np.asarray(lse_parts, dtype=np.float64)
    m = Lg.max(axis=0)
    w = np.exp(Lg - m[None])
    tot = w.sum(axis=0)
    lse = m if lse_is_max else m + np.log(tot)
    o = (w[..., None] * Og).sum(axis=0)
    return (o if unnormalised else o / tot[..., None]), lse


BWD_MUTANTS = {
    "delta_term_dropped": dict(no_delta=True),
    "dk_scale_dropped": dict(dk_unscaled=True),
    "dq_multiplies_v": dict(dq_uses_v=True),
    "dv_from_p_not_p_transposed": dict(dv_not_transposed=True),
    "delta_as_row_sum_of_dp": dict(delta_from_dp=True),
}
MERGE_MUTANTS = {"weights_not_normalised": dict(unnormalised=True), "lse_is_the_max_only": dict(lse_is_max=True)}


def test_copies_pass_all_pins():
    for pin in BWD_PINS:
        pin(_bwd)
    for pin in MERGE_PINS:
        pin(_merge)


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutants_are_caught(name):
    caught = []
    for pin in BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda *a, **kw: _bwd(*a, **kw, **BWD_MUTANTS[name]))
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every backward pin"


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_mutants_are_caught(name):
    caught = []
    for pin in MERGE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda *a: _merge(*a, **MERGE_MUTANTS[name]))
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every merge pin"
