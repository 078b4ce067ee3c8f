"""Pins for the float64 oracle: checks against facts the pages and mathematics fix,
none of which re-types the oracle's own formula.

  P1  softmax rows sum to 1                    (normalisation, Level 1 softmax)
  P2  causal row 0: O_0 = V_0, lse_0 = s*q0.k0  (causal rule, "Triton in depth" 3.3)
  P3  V constant per column -> O constant       (convex combination)
  P4  non-causal: joint K/V row permutation leaves O, lse unchanged
  P5  brute force with scalar loops, math.fsum, on tiny odd shapes
  P6  Q = 0: O_i = mean of allowed V rows, lse_i = ln(#allowed)
  P7  non-causal key shift K_j += u: O unchanged, lse_i += s*q_i.u
  P8  N = 2 closed form of the two-term online update
  P9  torch scaled_dot_product_attention in CPU float64 (library special case)
  PG  the pages' worked tiled-reduction example (tests/golden/)

test_mutants_are_caught plants one plausible mistake at a time in a copy of the
definition and asserts that some pin rejects it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ----------------------------------------------------------------------------- pins
# Each pin takes an implementation impl(q, k, v, causal, scale) -> (O, lse) and
# raises AssertionError when it does not hold.

def pin_p2(impl):
    q, k, v = rnd((2, 3, 7, 5), 1), rnd((2, 3, 7, 5), 2), rnd((2, 3, 7, 5), 3)
    s = 0.37
    O, L = impl(q, k, v, 1, s)
    assert np.array_equal(O[:, :, 0], v[:, :, 0]), "causal row 0 must be V_0 exactly"
    s64 = np.float64(np.float32(s))
    want = s64 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.allclose(L[:, :, 0], want, rtol=0, atol=1e-12)


def pin_p3(impl):
    for causal in (0, 1):
        q, k = rnd((1, 2, 9, 4), 4), rnd((1, 2, 9, 4), 5)
        c = np.array([1.5, -2.0, 0.25, 7.0])
        v = np.broadcast_to(c, (1, 2, 9, 4)).copy()
        O, _ = impl(q, k, v, causal, 0.8)
        assert np.allclose(O, c, rtol=0, atol=1e-12)


def pin_p4(impl):
    q, k, v = rnd((1, 2, 11, 6), 6), rnd((1, 2, 11, 6), 7), rnd((1, 2, 11, 6), 8)
    perm = np.random.default_rng(9).permutation(11)
    O1, L1 = impl(q, k, v, 0, 0.5)
    O2, L2 = impl(q, k[:, :, perm], v[:, :, perm], 0, 0.5)
    assert np.allclose(O1, O2, rtol=0, atol=1e-12)
    assert np.allclose(L1, L2, rtol=0, atol=1e-12)


def brute(q, k, v, causal, scale):
    """Scalar-loop definition: plain Python floats, math.exp, math.fsum."""
    s64 = float(np.float32(scale))
    B, H, N, d = np.shape(q)
    O = [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if (not causal) or j <= i]
                sc = [s64 * math.fsum(float(q[b][h][i][c]) * float(k[b][h][j][c]) for c in range(d))
                      for j in keys]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = math.fsum(e)
                for c in range(d):
                    O[b][h][i][c] = math.fsum(e[t] * float(v[b][h][j][c]) for t, j in enumerate(keys)) / tot
                L[b][h][i] = mx + math.log(tot)
    return np.array(O), np.array(L)


def pin_p5(impl):
    shapes = [(1, 1, 1, 1), (1, 1, 2, 3), (2, 1, 5, 2), (1, 2, 9, 5), (2, 2, 7, 3)]
    for n, shp in enumerate(shapes):
        for causal in (0, 1):
            q, k, v = rnd(shp, 10 + n), rnd(shp, 20 + n, 2.0), rnd(shp, 30 + n)
            O, L = impl(q, k, v, causal, 0.61)
            Ob, Lb = brute(q, k, v, causal, 0.61)
            assert np.allclose(O, Ob, rtol=0, atol=1e-12)
            assert np.allclose(L, Lb, rtol=0, atol=1e-12)


def pin_p6(impl):
    v = rnd((2, 2, 8, 3), 40)
    k = rnd((2, 2, 8, 3), 41)
    q = np.zeros((2, 2, 8, 3))
    O, L = impl(q, k, v, 1, 0.9)
    cnt = np.arange(1, 9)
    assert np.allclose(O, np.cumsum(v, axis=2) / cnt[None, None, :, None], rtol=0, atol=1e-12)
    assert np.allclose(L, np.log(cnt)[None, None, :], rtol=0, atol=1e-12)
    O, L = impl(q, k, v, 0, 0.9)
    assert np.allclose(O, v.mean(axis=2, keepdims=True).repeat(8, axis=2), rtol=0, atol=1e-12)
    assert np.allclose(L, math.log(8), rtol=0, atol=1e-12)


def pin_p7(impl):
    q, k, v = rnd((1, 3, 10, 4), 50), rnd((1, 3, 10, 4), 51), rnd((1, 3, 10, 4), 52)
    u = np.array([0.5, -1.0, 2.0, 0.25])
    s = 0.7
    O1, L1 = impl(q, k, v, 0, s)
    O2, L2 = impl(q, k + u, v, 0, s)
    s64 = np.float64(np.float32(s))
    assert np.allclose(O1, O2, rtol=0, atol=1e-10)
    assert np.allclose(L2 - L1, s64 * (q @ u), rtol=0, atol=1e-10)


def pin_p8(impl):
    q, k, v = rnd((1, 1, 2, 3), 60), rnd((1, 1, 2, 3), 61), rnd((1, 1, 2, 3), 62)
    s = 1.3
    s64 = np.float64(np.float32(s))
    for causal in (0, 1):
        O, L = impl(q, k, v, causal, s)
        s10 = s64 * float(q[0, 0, 1] @ k[0, 0, 0])
        s11 = s64 * float(q[0, 0, 1] @ k[0, 0, 1])
        e0, e1 = math.exp(s10), math.exp(s11)
        assert np.allclose(O[0, 0, 1], (e0 * v[0, 0, 0] + e1 * v[0, 0, 1]) / (e0 + e1), rtol=0, atol=1e-12)
        assert abs(L[0, 0, 1] - math.log(e0 + e1)) < 1e-12
        s00 = s64 * float(q[0, 0, 0] @ k[0, 0, 0])
        s01 = s64 * float(q[0, 0, 0] @ k[0, 0, 1])
        if causal:
            assert np.allclose(O[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-12)
            assert abs(L[0, 0, 0] - s00) < 1e-12
        else:
            f0, f1 = math.exp(s00), math.exp(s01)
            assert np.allclose(O[0, 0, 0], (f0 * v[0, 0, 0] + f1 * v[0, 0, 1]) / (f0 + f1), rtol=0, atol=1e-12)


def pin_p9(impl):
    for causal in (0, 1):
        for shp in [(2, 3, 33, 16), (1, 2, 70, 8)]:
            q, k, v = rnd(shp, 70), rnd(shp, 71), rnd(shp, 72)
            s = 0.25
            s64 = float(np.float32(s))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                is_causal=bool(causal), scale=s64).numpy()
            O, _ = impl(q, k, v, causal, s)
            assert np.allclose(O, ref, rtol=0, atol=1e-10)


PINS = [pin_p2, pin_p3, pin_p4, pin_p5, pin_p6, pin_p7, pin_p8, pin_p9]


def oracle_impl(q, k, v, causal, scale):
    return oracle.attention(q, k, v, causal, scale)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl)


def test_p1_rows_sum_to_one():
    for causal in (0, 1):
        q, k = rnd((2, 2, 13, 4), 80, 3.0), rnd((2, 2, 13, 4), 81, 3.0)
        W = oracle.softmax_weights(q, k, causal, 0.9)
        assert np.allclose(W.sum(axis=-1), 1.0, rtol=0, atol=1e-12 * 13)
        assert (W >= 0).all()
        if causal:
            assert (np.triu(W, k=1) == 0).all(), "weights above the diagonal must be exactly 0"


def test_rows_argument_matches_full():
    q, k, v = rnd((2, 2, 20, 4), 90), rnd((2, 2, 20, 4), 91), rnd((2, 2, 20, 4), 92)
    Of, Lf = oracle.attention(q, k, v, 1, 0.5)
    rows = np.array([0, 3, 19])
    Or, Lr = oracle.attention(q, k, v, 1, 0.5, rows=rows)
    assert np.array_equal(Or, Of[:, :, rows]) and np.array_equal(Lr, Lf[:, :, rows])
    per_head = np.array([[[1, 2], [5, 7]], [[0, 19], [4, 4]]])
    Op, Lp = oracle.attention(q, k, v, 1, 0.5, rows=per_head)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(Op[b, h], Of[b, h, per_head[b, h]])


def test_large_scores_stay_finite():
    """Scores of several hundred (outlier inputs) must not overflow: the max is subtracted."""
    q, k, v = rnd((1, 1, 6, 4), 93, 30.0), rnd((1, 1, 6, 4), 94, 30.0), rnd((1, 1, 6, 4), 95)
    O, L = oracle.attention(q, k, v, 0, 1.0)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    Ob, Lb = brute(q, k, v, 0, 1.0)
    assert np.allclose(O, Ob, rtol=0, atol=1e-9)
    assert np.allclose(L, Lb, rtol=1e-13, atol=0)


def test_golden_pages_tiled_reduction_example():
    """Page "CS336 Lecture 6", Level 2 row sum: a row split into tiles of four, where the
    per-thread accumulators after the second tile read 8 (= 3 + 5) and 10 (= 1 + 9).

    With Q = 0 every allowed key has weight 1, so causal row i of the attention output is
    the mean of V_0..V_i: the row sum of that example divided by the count."""
    with open(os.path.join(GOLDEN, "pages_rowsum_example.json")) as f:
        g = json.load(f)
    vals = np.array(g["row_values"], dtype=np.float64)
    n = vals.size
    v = vals.reshape(1, 1, n, 1)
    q = np.zeros((1, 1, n, 2))
    k = rnd((1, 1, n, 2), 96)
    O, L = oracle.attention(q, k, v, 1, 1.0)
    acc = g["thread_accumulators_after_tile1"]
    tile = g["block_size"]
    # threads 0 and 1 hold vals[0]+vals[4] and vals[1]+vals[5]; threads 2, 3 hold vals[2], vals[3]
    total = acc["thread0"] + acc["thread1"] + vals[2] + vals[3]
    assert tile == 4 and n == 6
    assert abs(O[0, 0, n - 1, 0] * n - total) < 1e-12
    for i in range(n):
        assert abs(O[0, 0, i, 0] - vals[: i + 1].mean()) < 1e-12
        assert abs(L[0, 0, i] - math.log(i + 1)) < 1e-12


def test_golden_oracle_regression():
    """Stored outputs written by tests/golden/make_oracle_fixtures.py (oracle only)."""
    with open(os.path.join(GOLDEN, "oracle_small.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        q = np.array(case["q"]); k = np.array(case["k"]); v = np.array(case["v"])
        O, L = oracle.attention(q, k, v, case["causal"], case["scale"])
        assert np.allclose(O, np.array(case["O"]), rtol=0, atol=1e-14)
        assert np.allclose(L, np.array(case["lse"]), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- mutants

def _definition(q, k, v, causal, scale, *, drop_scale=False, strict_mask=False, anti_mask=False,
                transpose_qk=False, lse_log2=False, lse_unscaled=False, page1_double_scale=False,
                norm_axis0=False, ignore_f32_scale=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s64 = np.float64(scale) if ignore_f32_scale else np.float64(np.float32(scale))
    B, H, N, d = q.shape
    O = np.empty_like(q)
    L = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, h], k[b, h], v[b, h]
            raw = (kh @ qh.T) if transpose_qk else (qh @ kh.T)
            s = raw if drop_scale else s64 * raw
            if causal:
                i = np.arange(N)[:, None]
                j = np.arange(N)[None, :]
                bad = (j >= i) & (j > 0) if strict_mask else ((j < i) if anti_mask else (j > i))
                s = np.where(bad, -np.inf, s)
            m = s.max(axis=1)
            if page1_double_scale:
                # the block-wise update of the simplified page-1 kernel, applied over 2-key blocks
                acc = np.zeros((N, vh.shape[1])); tot = np.zeros(N); mx = np.full(N, -np.inf)
                for st in range(0, N, 2):
                    blk = s[:, st:st + 2]
                    bm = blk.max(axis=1)
                    nm = np.maximum(mx, bm)
                    so = np.where(np.isfinite(mx), np.exp(mx - nm), 0.0)
                    sn = np.exp(bm - nm)
                    e = np.exp(blk - nm[:, None])
                    tot = tot * so + e.sum(axis=1) * sn
                    acc = acc * so[:, None] + (e @ vh[st:st + 2]) * sn[:, None]
                    mx = nm
                O[b, h] = acc / tot[:, None]
                L[b, h] = mx + np.log(tot)
                continue
            p = np.exp(s - m[:, None])
            if norm_axis0:
                l = p.sum(axis=0)
                O[b, h] = (p / l[None, :]) @ vh
            else:
                l = p.sum(axis=1)
                O[b, h] = (p @ vh) / l[:, None]
            lse = m + np.log(l)
            if lse_log2:
                lse = lse / math.log(2)
            if lse_unscaled:
                lse = lse / s64
            L[b, h] = lse
    return O, L


MUTANTS = {
    "drop_scale": dict(drop_scale=True),
    "diagonal_masked": dict(strict_mask=True),
    "mask_flipped": dict(anti_mask=True),
    "scores_transposed": dict(transpose_qk=True),
    "lse_in_log2": dict(lse_log2=True),
    "lse_unscaled": dict(lse_unscaled=True),
    "page1_double_scaling": dict(page1_double_scale=True),
    "normalised_over_queries": dict(norm_axis0=True),
    "scale_not_rounded_to_f32": dict(ignore_f32_scale=True),
}


def test_definition_copy_passes_all_pins():
    for pin in PINS:
        pin(lambda q, k, v, c, s: _definition(q, k, v, c, s))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name):
    kw = MUTANTS[name]
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda q, k, v, c, s: _definition(q, k, v, c, s, **kw))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
