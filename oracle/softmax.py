"""Row softmax in float64 on the CPU: the oracle for the standalone fused row
softmax.

TEST INFRASTRUCTURE ONLY.  It is imported by the tests, by the smoke check and
by the benchmark's CPU-baseline leg, and by nothing else; the HIP library and
its binding never call it and share no code with it.

What it computes is the definition the pages give for the fused softmax
("Triton: CUDA-level operators in Python", example 2; "CS336 Lecture 6",
Level 1): for each row independently, subtract the row's maximum for
numerical stability, exponentiate, and divide by the row's sum of
exponentials:

    y[i, j] = exp(x[i, j] - max_j x[i, j]) / sum_j exp(x[i, j] - max_j x[i, j])

on the exact input values (fp16/bf16/fp32 upcast to float64).

Pinned by tests/test_oracle_softmax_pins.py; no function here is unpinned.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(x) -> np.ndarray:
    """x: [rows, cols] (torch CPU tensor or array, any float dtype) -> float64 [rows, cols]."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be [rows, cols]")
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=1, keepdims=True)
