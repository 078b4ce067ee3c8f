"""Pins for the GEMM + bias + activation oracle, from facts the definition fixes:

  G1  brute force with scalar loops and math.fsum on small ragged shapes, every
      activation, with and without bias
  G2  B = identity (K = N): C = act(A + bias) exactly
  G3  A of ones: row m of C is act(column sums of B + bias)
  G4  torch.nn.functional.linear and torch's relu / tanh-GELU in CPU float64
      (library special case: linear(x, W, b) = x W^T + b)
  G5  the fused bias + ReLU of "Triton core syntax" 4.4 as the M = K = 1 case:
      y = max(x + bias, 0) on hand-computed values
  G6  GELU (tanh form): GELU(0) = 0, GELU(z) - GELU(-z) = z (tanh is odd),
      GELU(z) -> z and GELU(-z) -> 0 for large z, and torch's tanh-GELU
  G7  K = 0: the empty sum, C = act(bias) in every row
  G8  transposition: act-free C^T equals the product of B^T and A^T

test_gemm_mutants_are_caught plants plausible mistakes in a copy of the
definition and asserts that some pin rejects each.
"""
import math

import numpy as np
import pytest
import torch

from oracle import gemm as og

ACTS = [og.ACT_NONE, og.ACT_RELU, og.ACT_GELU_TANH]


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def gelu_scalar(z):
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def brute(A, B, bias, act):
    M, K = A.shape
    N = B.shape[1]
    out = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            z = math.fsum(A[m, k] * B[k, n] for k in range(K)) + (0.0 if bias is None else bias[n])
            out[m, n] = z if act == 0 else (max(z, 0.0) if act == 1 else gelu_scalar(z))
    return out


def pin_g1(impl):
    for i, (M, N, K) in enumerate([(1, 1, 1), (3, 5, 7), (4, 2, 9), (5, 6, 16)]):
        A, B, bias = rnd((M, K), 10 + i), rnd((K, N), 20 + i), rnd(N, 30 + i)
        for act in ACTS:
            for bv in (None, bias):
                assert np.allclose(impl(A, B, bv, act), brute(A, B, bv, act), rtol=1e-12, atol=1e-13), (M, N, K, act)


def pin_g2(impl):
    A, bias = rnd((6, 5), 40, 2.0), rnd(5, 41)
    for act in ACTS:
        z = A + bias[None, :]
        want = z if act == 0 else (np.maximum(z, 0) if act == 1 else np.vectorize(gelu_scalar)(z))
        assert np.allclose(impl(A, np.eye(5), bias, act), want, rtol=1e-14, atol=1e-15), act


def pin_g3(impl):
    B, bias = rnd((7, 4), 50), rnd(4, 51)
    C = impl(np.ones((3, 7)), B, bias, og.ACT_RELU)
    want = np.maximum(np.array([math.fsum(B[:, n]) for n in range(4)]) + bias, 0.0)
    assert np.allclose(C, np.tile(want, (3, 1)), rtol=1e-14, atol=1e-15)


def pin_g4(impl):
    x, W, b = rnd((9, 33), 60), rnd((17, 33), 61), rnd(17, 62)
    lin = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(W), torch.from_numpy(b))
    for act, f in ((og.ACT_NONE, lambda t: t), (og.ACT_RELU, torch.relu),
                   (og.ACT_GELU_TANH, lambda t: torch.nn.functional.gelu(t, approximate="tanh"))):
        assert np.allclose(impl(x, W.T, b, act), f(lin).numpy(), rtol=1e-12, atol=1e-13), act


def pin_g5(impl):
    x = np.array([-2.0, -0.5, 0.0, 0.5, 2.0, 1e-3])
    bias = np.array([1.0, 1.0, -1.0, 0.25, -3.0, -1e-3 / 2])
    y = impl(np.ones((1, 1)), x[None, :], bias, og.ACT_RELU)
    assert np.array_equal(y, np.array([[0.0, 0.5, 0.0, 0.75, 0.0, 5e-4]]))


def pin_g6(impl):
    z = np.linspace(-6, 6, 97)
    g = impl(np.ones((1, 1)), z[None, :], None, og.ACT_GELU_TANH)[0]
    gn = impl(np.ones((1, 1)), -z[None, :], None, og.ACT_GELU_TANH)[0]
    assert g[48] == 0.0                                            # z = 0
    assert np.allclose(g - gn, z, rtol=0, atol=1e-14)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-13, atol=1e-15)
    big = impl(np.ones((1, 1)), np.array([[30.0, -30.0]]), None, og.ACT_GELU_TANH)[0]
    assert big[0] == 30.0 and big[1] == 0.0


def pin_g7(impl):
    bias = rnd(6, 70)
    for act in ACTS:
        C = impl(np.zeros((4, 0)), np.zeros((0, 6)), bias, act)
        z = np.tile(bias, (4, 1))
        want = z if act == 0 else (np.maximum(z, 0) if act == 1 else np.vectorize(gelu_scalar)(z))
        assert C.shape == (4, 6) and np.allclose(C, want, rtol=1e-15, atol=0)
    assert (impl(np.zeros((2, 0)), np.zeros((0, 3)), None, og.ACT_NONE) == 0).all()


def pin_g8(impl):
    A, B = rnd((5, 11), 80), rnd((11, 7), 81)
    assert np.allclose(impl(B.T, A.T, None, og.ACT_NONE).T, impl(A, B, None, og.ACT_NONE), rtol=1e-13, atol=1e-14)


PINS = [pin_g1, pin_g2, pin_g3, pin_g4, pin_g5, pin_g6, pin_g7, pin_g8]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_gemm_oracle_pin(pin):
    pin(og.gemm_bias_act)


def test_gemm_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        og.gemm_bias_act(np.zeros((2, 3)), np.zeros((4, 2)))
    with pytest.raises(ValueError):
        og.gemm_bias_act(np.zeros((2, 3)), np.zeros((3, 2)), np.zeros(3))
    with pytest.raises(ValueError):
        og.activation(np.zeros(2), 7)


# ----------------------------------------------------------------------------- mutants

def _definition(A, B, bias=None, act=0, *, bias_after_act=False, bias_per_row=False, b_transposed=False,
                relu_abs=False, gelu_const=0.044715, gelu_no_sqrt=False, gelu_erf=False, drop_last_k=False):
    A, B = np.asarray(A, dtype=np.float64), np.asarray(B, dtype=np.float64)
    if b_transposed:
        B = B.T
    if drop_last_k and A.shape[1] > 0:
        A, B = A[:, :-1], B[:-1, :]
    z = A @ B
    bv = None if bias is None else np.asarray(bias, dtype=np.float64)
    if bv is not None and not bias_after_act:
        z = z + (bv[:, None] if bias_per_row else bv[None, :])
    if act == 1:
        z = np.abs(z) if relu_abs else np.maximum(z, 0.0)
    elif act == 2:
        if gelu_erf:
            z = 0.5 * z * (1.0 + np.vectorize(math.erf)(z / math.sqrt(2.0))) if z.size else z
        else:
            c = 1.0 if gelu_no_sqrt else math.sqrt(2.0 / math.pi)
            z = 0.5 * z * (1.0 + np.tanh(c * (z + gelu_const * z ** 3)))
    if bv is not None and bias_after_act:
        z = z + bv[None, :]
    return z


MUTANTS = {
    "bias_added_after_activation": dict(bias_after_act=True),
    "bias_indexed_by_row": dict(bias_per_row=True),
    "b_transposed": dict(b_transposed=True),
    "relu_as_abs": dict(relu_abs=True),
    "gelu_cubic_coefficient_off": dict(gelu_const=0.04715),
    "gelu_without_sqrt_2_over_pi": dict(gelu_no_sqrt=True),
    "gelu_erf_form_instead_of_tanh": dict(gelu_erf=True),
    "last_k_term_dropped": dict(drop_last_k=True),
}


def test_definition_copy_passes_all_gemm_pins():
    for pin in PINS:
        pin(_definition)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gemm_mutants_are_caught(name):
    kw = MUTANTS[name]
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lambda *a: _definition(*a, **kw))
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every GEMM pin"
