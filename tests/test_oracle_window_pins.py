"""Pins for the oracle's sliding window, from facts the window's definition
fixes and that do not re-type the oracle's masking code:

  W1  W >= N changes nothing: the result equals the unwindowed oracle
  W2  W = 1 keeps only the diagonal: O_i = V_i exactly, lse_i = s*q_i.k_i
  W3  brute force with scalar loops and an explicit key list per row
  W4  Q = 0: O_i = mean of V over the kept band, lse_i = ln(band size), with
      the band sizes counted by hand for a small case
  W5  locality: changing the K/V row just outside row i's band leaves row i
      unchanged, changing the row at the band's edge changes it
  W6  torch scaled_dot_product_attention in CPU float64 with a boolean mask
      built from the explicit key lists of W3 (library special case)

test_window_mutants_are_caught plants plausible window mistakes in a copy of the
definition and asserts that some pin rejects each.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def keys_for(i, n, causal, w):
    """Kept key indices of row i, listed by walking the band, not by a formula on j."""
    if w == 0:
        hi = i if causal else n - 1
        return list(range(0, hi + 1))
    lo = max(0, i - w + 1)
    hi = i if causal else min(n - 1, i + w - 1)
    return list(range(lo, hi + 1))


def brute(q, k, v, causal, scale, w):
    s64 = float(np.float32(scale))
    B, H, N, d = np.shape(q)
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = keys_for(i, N, causal, w)
                sc = [s64 * math.fsum(float(q[b][h][i][c]) * float(k[b][h][j][c]) for c in range(d)) for j in keys]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = math.fsum(e)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(e[t] * float(v[b][h][j][c]) for t, j in enumerate(keys)) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


# Each pin takes impl(q, k, v, causal, scale, window) -> (O, lse).

def pin_w1(impl):
    q, k, v = rnd((2, 2, 13, 5), 1), rnd((2, 2, 13, 5), 2), rnd((2, 2, 13, 5), 3)
    for causal in (0, 1):
        O0, L0 = oracle.attention(q, k, v, causal, 0.4)
        for w in (13, 14, 100):
            O, L = impl(q, k, v, causal, 0.4, w)
            assert np.array_equal(O, O0) and np.array_equal(L, L0)


def pin_w2(impl):
    q, k, v = rnd((1, 3, 9, 4), 4), rnd((1, 3, 9, 4), 5), rnd((1, 3, 9, 4), 6)
    s64 = np.float64(np.float32(0.9))
    for causal in (0, 1):
        O, L = impl(q, k, v, causal, 0.9, 1)
        assert np.array_equal(O, v), "W = 1 keeps only the diagonal"
        assert np.allclose(L, s64 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-12)


def pin_w3(impl):
    for n, (shp, w) in enumerate([((1, 1, 6, 3), 2), ((2, 1, 9, 2), 3), ((1, 2, 11, 4), 5), ((1, 1, 7, 3), 6)]):
        for causal in (0, 1):
            q, k, v = rnd(shp, 10 + n), rnd(shp, 20 + n, 2.0), rnd(shp, 30 + n)
            O, L = impl(q, k, v, causal, 0.55, w)
            Ob, Lb = brute(q, k, v, causal, 0.55, w)
            assert np.allclose(O, Ob, rtol=0, atol=1e-12)
            assert np.allclose(L, Lb, rtol=0, atol=1e-12)


def pin_w4(impl):
    N, w = 7, 3
    v = rnd((1, 1, N, 2), 40)
    q = np.zeros((1, 1, N, 2))
    k = rnd((1, 1, N, 2), 41)
    # band sizes counted by hand for N = 7, W = 3
    causal_cnt = [1, 2, 3, 3, 3, 3, 3]
    causal_lo = [0, 0, 0, 1, 2, 3, 4]
    band_cnt = [3, 4, 5, 5, 5, 4, 3]
    band_lo = [0, 0, 0, 1, 2, 3, 4]
    for causal, cnt, lo in ((1, causal_cnt, causal_lo), (0, band_cnt, band_lo)):
        O, L = impl(q, k, v, causal, 0.7, w)
        for i in range(N):
            want = v[0, 0, lo[i]:lo[i] + cnt[i]].mean(axis=0)
            assert np.allclose(O[0, 0, i], want, rtol=0, atol=1e-12)
            assert abs(L[0, 0, i] - math.log(cnt[i])) < 1e-12


def pin_w5(impl):
    N, w, i = 14, 4, 8
    q, k, v = rnd((1, 1, N, 3), 50), rnd((1, 1, N, 3), 51), rnd((1, 1, N, 3), 52)
    for causal in (0, 1):
        O, L = impl(q, k, v, causal, 0.8, w)
        outside = [i - w] + ([] if causal else [i + w])
        edge = [i - w + 1] + ([] if causal else [i + w - 1])
        for j in outside:
            k2, v2 = k.copy(), v.copy()
            k2[0, 0, j] += 3.0
            v2[0, 0, j] -= 5.0
            O2, L2 = impl(q, k2, v2, causal, 0.8, w)
            assert np.array_equal(O2[0, 0, i], O[0, 0, i]) and L2[0, 0, i] == L[0, 0, i], f"key {j} is outside row {i}'s band"
        for j in edge:
            v2 = v.copy()
            v2[0, 0, j] -= 5.0
            O2, _ = impl(q, k, v2, causal, 0.8, w)
            assert not np.allclose(O2[0, 0, i], O[0, 0, i], rtol=0, atol=1e-6), f"key {j} is inside row {i}'s band"


def pin_w6(impl):
    for causal in (0, 1):
        for shp, w in [((2, 2, 40, 8), 7), ((1, 3, 65, 4), 16)]:
            q, k, v = rnd(shp, 60), rnd(shp, 61), rnd(shp, 62)
            N = shp[2]
            mask = torch.zeros(N, N, dtype=torch.bool)
            for i in range(N):
                mask[i, keys_for(i, N, causal, w)] = True
            s64 = float(np.float32(0.3))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=s64).numpy()
            O, _ = impl(q, k, v, causal, 0.3, w)
            assert np.allclose(O, ref, rtol=0, atol=1e-10)


PINS = [pin_w1, pin_w2, pin_w3, pin_w4, pin_w5, pin_w6]


def oracle_impl(q, k, v, causal, scale, w):
    return oracle.attention(q, k, v, causal, scale, window=w)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_window_pin(pin):
    pin(oracle_impl)


def test_window_rejects_negative():
    q = rnd((1, 1, 4, 2), 1)
    with pytest.raises(ValueError):
        oracle.attention(q, q, q, 1, 0.5, window=-1)


def test_window_weights_rows_sum_to_one():
    q, k = rnd((1, 2, 10, 3), 70), rnd((1, 2, 10, 3), 71)
    for causal in (0, 1):
        W = oracle.softmax_weights(q, k, causal, 0.6, window=3)
        assert np.allclose(W.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
        for i in range(10):
            kept = set(keys_for(i, 10, causal, 3))
            assert all((W[0, :, i, j] == 0).all() for j in range(10) if j not in kept)


# ----------------------------------------------------------------------------- mutants

def _definition(q, k, v, causal, scale, w, *, lo_off=0, hi_off=0, ignore=False, causal_band=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    s64 = np.float64(np.float32(scale))
    B, H, N, d = q.shape
    O = np.empty_like(q)
    L = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            s = s64 * (q[b, h] @ k[b, h].T)
            i = np.arange(N)[:, None]
            j = np.arange(N)[None, :]
            keep = np.ones((N, N), dtype=bool)
            if causal:
                keep &= j <= i
            if w > 0 and not ignore:
                keep &= j > i - w + lo_off
                if not causal or causal_band:
                    keep &= j < i + w + hi_off
            s = np.where(keep, s, -np.inf)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            l = p.sum(axis=1)
            O[b, h] = (p @ v[b, h]) / l[:, None]
            L[b, h] = m + np.log(l)
    return O, L


MUTANTS = {
    "window_one_too_wide": dict(lo_off=-1),
    "window_one_too_narrow": dict(lo_off=1),
    "band_upper_edge_off_by_one": dict(hi_off=1),
    "window_ignored": dict(ignore=True),
}


def test_definition_copy_passes_all_window_pins():
    for pin in PINS:
        pin(lambda q, k, v, c, s, w: _definition(q, k, v, c, s, w))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_window_mutants_are_caught(name):
    kw = MUTANTS[name]
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda q, k, v, c, s, w: _definition(q, k, v, c, s, w, **kw))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every window pin"
