"""CPU float64 oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg.  The HIP library never imports it.
"""
from .attention import attention, softmax_weights
from .softmax import softmax_rows

__all__ = ["attention", "softmax_weights", "softmax_rows"]
