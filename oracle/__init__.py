"""CPU float64 oracles: exact attention forward and its gradients, the merge of
key-sharded attention results, row softmax, GEMM + bias + activation.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg.  The HIP library never imports it.
"""
from .attention import attention, softmax_weights
from .softmax import softmax_rows
from .gemm import gemm_bias_act
from .backward import attention_bwd, lse_merge

__all__ = ["attention", "softmax_weights", "softmax_rows", "gemm_bias_act", "attention_bwd", "lse_merge"]
