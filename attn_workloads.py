"""Seeded synthetic workloads for the attention forward pass, the row softmax and
the matrix product with its fused epilogue.

This module is shared by the tests, the benchmark and smoke check.  It draws
inputs and sample rows and holds the table of workload shapes; it contains none
of the attention, softmax or matrix-product arithmetic, so neither the CPU
oracle nor the HIP library depends on the other through it.

Recipe (identical for every consumer):
  * numpy ``default_rng(seed)``, seed = 1000 + workload index;
  * Q, K, V drawn in that order as iid N(0, 1) float32 of shape [B, H, N, d];
  * outlier workloads then draw one U[0,1) mask for Q and one for K; entries with
    U < fraction are multiplied by ``factor`` (V is left untouched);
  * the float32 values are cast to fp16/bf16 with round-to-nearest-even by torch
    on the CPU.  Every consumer reads these cast tensors.

The shapes follow the long-sequence attention the pages motivate tiling with
(Triton in depth, section 3.1: sequences of 32K tokens and more) and the
causal rule of the forward kernel (section 3.3).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                     # "fp16" | "bf16"
    causal_modes: tuple            # causal flags to run (1 = causal)
    scale: float
    seed: int
    outlier_fraction: float = 0.0  # fraction of Q and K entries scaled up
    outlier_factor: float = 1.0
    sample_rows: int | None = None  # rows per head the oracle checks (None = all)
    note: str = field(default="", compare=False)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def flops(self, causal: int) -> float:
        """4*B*H*N^2*d, halved when causal (the accounting used for TFLOP/s)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if causal else f

    def algorithmic_bytes(self) -> int:
        """Q, K, V read once, O written once (2-byte elements) and lse written as fp32."""
        elems = self.B * self.H * self.N * self.d
        return 4 * elems * 2 + self.B * self.H * self.N * 4


WORKLOADS = [
    Workload("causal_b1_h1_n128_d64_fp16", 1, 1, 128, 64, "fp16", (1,), 1.0 / math.sqrt(64), 1000,
             note="single tile, latency-bound"),
    Workload("causal_b4_h16_n1024_d64_fp16", 4, 16, 1024, 64, "fp16", (1,), 1.0 / 8.0, 1001),
    Workload("causal_b2_h32_n4096_d128_bf16", 2, 32, 4096, 128, "bf16", (1,), 1.0 / math.sqrt(128), 1002,
             note="headline workload"),
    Workload("long_b1_h16_n32768_d128_bf16", 1, 16, 32768, 128, "bf16", (1, 0), 1.0 / math.sqrt(128), 1003,
             sample_rows=512, note="oracle checks 512 sampled rows per head"),
    Workload("ragged_b3_h8_n3000_d80_fp16", 3, 8, 3000, 80, "fp16", (0,), 1.0 / math.sqrt(80), 1004,
             outlier_fraction=0.01, outlier_factor=20.0, note="N not a tile multiple; 1% x20 outliers in Q, K"),
]

HEADLINE = 2  # index of the workload the benchmark reports


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def draw_fp32(shape, seed: int, outlier_fraction: float = 0.0, outlier_factor: float = 1.0):
    """Q, K, V as float32 numpy arrays following the recipe above."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if outlier_fraction > 0.0:
        mq = rng.random(shape, dtype=np.float32) < outlier_fraction
        mk = rng.random(shape, dtype=np.float32) < outlier_fraction
        q[mq] *= np.float32(outlier_factor)
        k[mk] *= np.float32(outlier_factor)
    return q, k, v


def make_inputs(shape, dtype: str, seed: int, outlier_fraction: float = 0.0, outlier_factor: float = 1.0):
    """Q, K, V as contiguous CPU torch tensors of the given 16-bit dtype (RNE cast)."""
    q, k, v = draw_fp32(shape, seed, outlier_fraction, outlier_factor)
    tdt = DTYPES[dtype]
    return tuple(torch.from_numpy(x).to(tdt).contiguous() for x in (q, k, v))


def workload_inputs(w: Workload):
    return make_inputs(w.shape, w.dtype, w.seed, w.outlier_fraction, w.outlier_factor)


def sample_rows(B: int, H: int, N: int, count: int, seed: int) -> np.ndarray:
    """Per-head sorted query rows [B, H, count]: rows 0 and N-1 forced in, the rest drawn
    without replacement from a seeded generator."""
    count = min(count, N)
    rng = np.random.default_rng(seed)
    out = np.empty((B, H, count), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            forced = np.unique(np.array([0, N - 1], dtype=np.int64))
            rest_pool = np.setdiff1d(np.arange(N, dtype=np.int64), forced)
            rest = rng.choice(rest_pool, size=count - forced.size, replace=False)
            out[b, h] = np.sort(np.concatenate([forced, rest]))
    return out


# --- row softmax ---------------------------------------------------------------
#
# Recipe: numpy default_rng(seed); x drawn as iid N(0, sigma^2) float32 of shape
# [rows, cols] (sigma = 1 is the distribution of the scaled attention scores of
# unit-normal q and k); then cast to the workload's type by torch on the CPU
# (round to nearest even).  The shape of the benchmark workload is the one the
# pages quote the fused softmax's bandwidth at: rows of 32K columns ("Triton:
# CUDA-level operators in Python", example 2).


@dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    rows: int
    cols: int
    dtype: str          # "f32" | "fp16" | "bf16"
    seed: int
    sigma: float = 1.0
    note: str = field(default="", compare=False)

    def algorithmic_bytes(self) -> int:
        """x read once and y written once (the fused kernel's HBM traffic)."""
        es = 4 if self.dtype == "f32" else 2
        return 2 * self.rows * self.cols * es


SOFTMAX_WORKLOADS = [
    SoftmaxWorkload("softmax_rows4096_cols32768_f32", 4096, 32768, "f32", 2000,
                    note="rows of 32K columns, fp32"),
    SoftmaxWorkload("softmax_rows4096_cols32768_bf16", 4096, 32768, "bf16", 2001),
    SoftmaxWorkload("softmax_rows1024_cols262147_f32", 1024, 262147, "f32", 2002,
                    note="rows beyond the in-register limit, ragged"),
]


def softmax_by_name(name: str) -> SoftmaxWorkload:
    for w in SOFTMAX_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def draw_rows(rows: int, cols: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    """x as a float32 numpy array [rows, cols] following the recipe above."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def make_rows(rows: int, cols: int, dtype: str, seed: int, sigma: float = 1.0) -> torch.Tensor:
    """x as a contiguous CPU torch tensor of the given type (RNE cast)."""
    return torch.from_numpy(draw_rows(rows, cols, seed, sigma)).to(DTYPES[dtype]).contiguous()


# --- matrix product with bias and activation -------------------------------------
#
# Recipe: numpy default_rng(seed); A drawn as iid N(0, 1) float32 [M, K], then
# B as iid N(0, 1/K) float32 (stored [K, N], or [N, K] for the weight layout),
# then bias as iid N(0, 1) float32 [N]; each cast to the workload's type by
# torch on the CPU (round to nearest even).  The shapes are the projections on
# either side of the attention workload B=2 H=32 N=4096 d=128: 8192 tokens of
# model width 4096, the fused Q/K/V projection to 3 x 4096 and an MLP
# up-projection to 4 x 4096 with tanh-GELU, plus the pages' K x N layout with
# ReLU ("CS336 Lecture 6", Level 3).


@dataclass(frozen=True)
class GemmWorkload:
    name: str
    M: int
    N: int
    K: int
    dtype: str          # "fp16" | "bf16"
    b_layout: str       # "kn" (B stored K x N) | "nk" (weight W stored N x K, B = W^T)
    act: str            # "none" | "relu" | "gelu_tanh"
    bias: bool
    seed: int
    note: str = field(default="", compare=False)

    def flops(self) -> float:
        """2 M N K for the product (the epilogue is not counted)."""
        return 2.0 * self.M * self.N * self.K

    def algorithmic_bytes(self) -> int:
        """A, B (and bias) read once, C written once."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N + (self.N if self.bias else 0))


GEMM_WORKLOADS = [
    GemmWorkload("gemm_qkv_m8192_n12288_k4096_bf16", 8192, 12288, 4096, "bf16", "nk", "none", True, 3000,
                 note="fused Q/K/V projection of 8192 tokens, width 4096"),
    GemmWorkload("gemm_mlp_m8192_n16384_k4096_bf16_gelu", 8192, 16384, 4096, "bf16", "nk", "gelu_tanh", True, 3001,
                 note="MLP up-projection with tanh-GELU"),
    GemmWorkload("gemm_kn_m4096_n4096_k4096_fp16_relu", 4096, 4096, 4096, "fp16", "kn", "relu", True, 3002,
                 note="the pages' K x N layout with the fused ReLU"),
]


def gemm_by_name(name: str) -> GemmWorkload:
    for w in GEMM_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def draw_gemm(M: int, N: int, K: int, b_layout: str, seed: int):
    """(A, B, bias) as float32 numpy arrays following the recipe above; B is returned
    in its storage layout ([K, N] for "kn", [N, K] for "nk")."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    shape = (K, N) if b_layout == "kn" else (N, K)
    b = rng.standard_normal(shape, dtype=np.float32) * np.float32(1.0 / math.sqrt(max(K, 1)))
    bias = rng.standard_normal(N, dtype=np.float32)
    return a, b, bias


def make_gemm(M: int, N: int, K: int, dtype: str, b_layout: str, seed: int):
    """(A, B, bias) as contiguous CPU torch tensors of the given 16-bit type (RNE cast)."""
    tdt = DTYPES[dtype]
    return tuple(torch.from_numpy(x).to(tdt).contiguous() for x in draw_gemm(M, N, K, b_layout, seed))


def gemm_workload_inputs(w: GemmWorkload):
    return make_gemm(w.M, w.N, w.K, w.dtype, w.b_layout, w.seed)
