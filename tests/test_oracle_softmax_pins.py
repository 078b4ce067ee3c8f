"""Pins for the row-softmax oracle, from facts the definition fixes:

  S1  rows sum to 1 and every entry lies in (0, 1]
  S2  shift invariance: adding a constant to a row leaves it unchanged
  S3  two columns: the closed form 1 / (1 + exp(x1 - x0)) (the logistic function)
  S4  a constant row gives 1 / cols exactly
  S5  brute force with scalar loops, math.exp and math.fsum, on small ragged shapes
  S6  torch.softmax in CPU float64 (library special case)
  S7  a dominant entry: x0 = x_j + 800 makes y0 = 1 and the rest underflow to 0
  S8  the pages' worked row [3, 1, 4, 1, 5, 9, ...] of the tiled row-sum example:
      the softmax of [3, 1, 4, 1] (the first tile) from the exponential sums

test_softmax_mutants_are_caught plants plausible mistakes in a copy of the
definition and asserts that some pin rejects each.
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


def pin_s1(impl):
    x = rnd((7, 33), 1, 3.0)
    y = impl(x)
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert (y > 0).all() and (y <= 1).all()


def pin_s2(impl):
    x = rnd((5, 17), 2)
    y0 = impl(x)
    y1 = impl(x + np.array([[3.5], [-100.0], [0.25], [1e3], [-7.0]]))
    assert np.allclose(y0, y1, rtol=1e-12, atol=1e-15)


def pin_s3(impl):
    x = rnd((9, 2), 3, 4.0)
    y = impl(x)
    want0 = 1.0 / (1.0 + np.exp(x[:, 1] - x[:, 0]))
    assert np.allclose(y[:, 0], want0, rtol=1e-13, atol=0)
    assert np.allclose(y[:, 1], 1.0 - want0, rtol=1e-12, atol=1e-15)


def pin_s4(impl):
    for cols in (1, 3, 64, 1000):
        y = impl(np.full((2, cols), -2.5))
        assert (y == 1.0 / cols).all()


def brute(x):
    out = []
    for row in np.asarray(x).tolist():
        mx = max(row)
        e = [math.exp(v - mx) for v in row]
        s = math.fsum(e)
        out.append([v / s for v in e])
    return np.array(out)


def pin_s5(impl):
    for n, shp in enumerate([(1, 1), (3, 5), (4, 31), (2, 129)]):
        x = rnd(shp, 10 + n, 5.0)
        assert np.allclose(impl(x), brute(x), rtol=1e-13, atol=1e-300)


def pin_s6(impl):
    x = rnd((6, 257), 20, 2.0)
    ref = torch.softmax(torch.from_numpy(x), dim=1).numpy()
    assert np.allclose(impl(x), ref, rtol=1e-12, atol=1e-300)


def pin_s7(impl):
    x = rnd((3, 40), 30)
    x[:, 0] = x[:, 1:].max(axis=1) + 800.0
    y = impl(x)
    assert (y[:, 0] == 1.0).all() and (y[:, 1:] == 0.0).all()


def pin_s8(impl):
    case = json.load(open(os.path.join(GOLDEN, "pages_rowsum_example.json")))
    tile = np.array([case["row_values"][:4]], dtype=np.float64)   # first tile of the pages' row
    y = impl(tile)
    e = np.exp(tile - tile.max())
    assert np.allclose(y, e / e.sum(), rtol=1e-14, atol=0)
    # the largest entry of [3, 1, 4, 1] is 4, and exp(0) / (e^-1 + e^-3 + 1 + e^-3)
    assert abs(y[0, 2] - 1.0 / (1.0 + math.exp(-1) + 2 * math.exp(-3))) < 1e-15


PINS = [pin_s1, pin_s2, pin_s3, pin_s4, pin_s5, pin_s6, pin_s7, pin_s8]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_softmax_oracle_pin(pin):
    pin(oracle.softmax_rows)


def test_softmax_oracle_rejects_non_2d():
    with pytest.raises(ValueError):
        oracle.softmax_rows(np.zeros(5))


# ----------------------------------------------------------------------------- mutants

def _definition(x, *, no_max=False, col_axis=False, max_only_first=False, drop_last=False, divide_by_max=False):
    x = np.asarray(x, dtype=np.float64)
    ax = 0 if col_axis else 1
    m = x.max(axis=ax, keepdims=True)
    if max_only_first:
        m = x[:, :1] if not col_axis else x[:1, :]
    e = np.exp(x if no_max else x - m)
    s = e.sum(axis=ax, keepdims=True)
    if drop_last:
        s = s - e[:, -1:]
    y = e / s
    if divide_by_max:
        y = e / e.max(axis=ax, keepdims=True)
    return y


MUTANTS = {
    "normalised_over_columns": dict(col_axis=True),
    "last_column_left_out_of_sum": dict(drop_last=True),
    "divided_by_max_not_sum": dict(divide_by_max=True),
    "no_max_subtraction_overflows": dict(no_max=True),
}


def test_definition_copy_passes_all_softmax_pins():
    for pin in PINS:
        pin(_definition)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_softmax_mutants_are_caught(name):
    kw = MUTANTS[name]
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda x: _definition(x, **kw))
        except (AssertionError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every softmax pin"
