"""Matrix product with a fused bias and activation epilogue, in float64 on the
CPU: the oracle for the tiled GEMM kernel.

TEST INFRASTRUCTURE ONLY.  It is imported by the tests, by the smoke check and
by the benchmark's CPU-baseline leg, and by nothing else; the HIP library and
its binding never call it and share no code with it.

What it computes follows the pages:

* "CS336 Lecture 6", Level 3: C = A B for A of shape M x K and B of shape
  K x N, with an element-wise nonlinearity (ReLU, "or GELU") applied to the
  accumulated tile before it is stored, the "linear layer = matmul +
  activation" pattern;
* "Triton core syntax", 4.4: the fused bias + ReLU, y = max(x + bias, 0);
* "Triton: CUDA-level operators in Python", example 3: the product is
  accumulated in fp32 and converted once to the 16-bit output type at the
  store.

Reading of the combination: C[m, n] = act(sum_k A[m, k] B[k, n] + bias[n]),
the bias broadcast over rows (one value per output column, as in a linear
layer) and added before the activation, as in the fused bias + ReLU example.
act is the identity, ReLU max(z, 0), or GELU in its tanh form
0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) (the lecture's GELU example
builds it from tanh).  The exact inputs (16-bit values upcast) are used and
nothing is rounded; the oracle returns float64.

Pinned by tests/test_oracle_gemm_pins.py; no function here is unpinned.
"""
from __future__ import annotations

import numpy as np

ACT_NONE, ACT_RELU, ACT_GELU_TANH = 0, 1, 2

_GELU_C = np.sqrt(2.0 / np.pi)
_GELU_A = 0.044715


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def activation(z: np.ndarray, act: int) -> np.ndarray:
    """The epilogue nonlinearity applied element by element."""
    if act == ACT_NONE:
        return z
    if act == ACT_RELU:
        return np.maximum(z, 0.0)
    if act == ACT_GELU_TANH:
        return 0.5 * z * (1.0 + np.tanh(_GELU_C * (z + _GELU_A * z ** 3)))
    raise ValueError(f"unknown activation {act}")


def gemm_bias_act(a, b, bias=None, act: int = ACT_NONE) -> np.ndarray:
    """a: [M, K]; b: [K, N] (logical, whatever its storage); bias: [N] or None.
    Returns float64 [M, N] = act(a @ b + bias)."""
    A, B = _f64(a), _f64(b)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {A.shape} x {B.shape} do not chain")
    z = A @ B
    if bias is not None:
        bv = _f64(bias)
        if bv.shape != (B.shape[1],):
            raise ValueError(f"bias must have shape ({B.shape[1]},)")
        z = z + bv[None, :]
    return activation(z, act)
