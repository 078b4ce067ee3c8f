"""GPU parity of the matrix product with fused bias + activation (gemm_bias_act,
include/gemm.h) against the float64 oracle (oracle/gemm.py, pinned in
test_oracle_gemm_pins.py).

Exact cases.  With small-integer A, B and bias (|values| <= 4) every product and
every partial sum is an integer below 2^24, so the fp32 accumulation is exact
whatever its order; the kernel's only rounding is then the final one to the
16-bit type, and its output must equal the oracle's value rounded to nearest
even, bit for bit (identity and ReLU epilogues).

Bar for general inputs.  Let u = 2^-24 and u_out the unit roundoff of the
output type (2^-8 bf16, 2^-11 fp16), S = |A| |B| + |bias| (the oracle on
absolute values) and z the oracle's pre-activation value.  Summing K products
in fp32 in any order errs by at most (K + 2) u S (K - 1 additions, the bias
addition, one spare), call it d.  ReLU is 1-Lipschitz; tanh-GELU has slope at
most 1.13, and its fp32 evaluation (a cubic, exp2, a division) adds at most
e_g = 3e-6 (1 + |z|).  The final rounding adds u_out of the result.  So every
element must satisfy
    |C - C_oracle| <= L d + e_g + u_out (|C_oracle| + L d + e_g),
with L = 1 (none, ReLU) or 1.13 (GELU) and e_g = 0 except for GELU.
"""
import numpy as np
import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
from oracle import gemm as og

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
U_OUT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}
ACT = {"none": og.ACT_NONE, "relu": og.ACT_RELU, "gelu_tanh": og.ACT_GELU_TANH}


def logical_b(b, b_layout):
    """The K x N matrix B from its storage."""
    return b if b_layout == "kn" else b.t()


def oracle_c(a, b, bias, act, b_layout, rows=None):
    A = a if rows is None else a[rows]
    return og.gemm_bias_act(A, logical_b(b, b_layout), bias, ACT[act])


def check(c_gpu, a, b, bias, act, b_layout, dtype, label, rows=None):
    A = a if rows is None else a[rows]
    ref = oracle_c(a, b, bias, act, b_layout, rows)
    z = og.gemm_bias_act(A, logical_b(b, b_layout), bias, og.ACT_NONE)
    S = og.gemm_bias_act(A.abs(), logical_b(b, b_layout).abs(), None if bias is None else bias.abs(), og.ACT_NONE)
    K = a.shape[1]
    d = (K + 2) * U32 * S
    L, eg = (1.13, 3e-6 * (1 + np.abs(z))) if act == "gelu_tanh" else (1.0, 0.0)
    bound = L * d + eg + U_OUT[dtype] * (np.abs(ref) + L * d + eg)
    got = (c_gpu if rows is None else c_gpu[rows]).double().cpu().numpy()
    err = np.abs(got - ref)
    if not (err <= bound).all():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{label}: |C - ref| = {err[i]:.3e} > bound {bound[i]:.3e} at {i} (C={got[i]}, ref={ref[i]})")


def int_inputs(M, N, K, b_layout, dtype, seed):
    g = np.random.default_rng(seed)
    tdt = TORCH[dtype]
    a = torch.from_numpy(g.integers(-4, 5, (M, K)).astype(np.float32)).to(tdt)
    b = torch.from_numpy(g.integers(-4, 5, (K, N) if b_layout == "kn" else (N, K)).astype(np.float32)).to(tdt)
    bias = torch.from_numpy(g.integers(-4, 5, N).astype(np.float32)).to(tdt)
    return a, b, bias


def run(a, b, bias, act, b_layout):
    c = eta.gemm_bias_act(a.cuda(), b.cuda(), None if bias is None else bias.cuda(), act, b_layout)
    torch.cuda.synchronize()
    return c.cpu()


# M, N around the 256-row tiles and the 32-row MFMA blocks; K around the 64-wide
# steps and the 8-element chunks
SHAPES = [(1, 1, 8), (5, 7, 8), (33, 65, 16), (256, 256, 64), (257, 255, 72), (300, 520, 1000), (512, 40, 136),
          (70, 600, 256), (1000, 300, 512)]


@pytest.mark.parametrize("b_layout", ["kn", "nk"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_gemm_exact_on_integers(lib, b_layout, dtype):
    for i, (M, N, K) in enumerate(SHAPES):
        a, b, bias = int_inputs(M, N, K, b_layout, dtype, 4000 + i)
        for act in ("none", "relu"):
            for bv in (bias, None):
                print(f"\n[case] gemm exact {dtype} {b_layout} M={M} N={N} K={K} act={act} bias={bv is not None}",
                      flush=True)
                c = run(a, b, bv, act, b_layout)
                want = torch.from_numpy(oracle_c(a, b, bv, act, b_layout)).to(TORCH[dtype])
                bad = (c.view(torch.int16) != want.view(torch.int16))
                assert not bad.any(), (f"{dtype} {b_layout} {M}x{N}x{K} {act}: {int(bad.sum())} elements differ, "
                                       f"first at {tuple(bad.nonzero()[0].tolist())}")


@pytest.mark.parametrize("b_layout", ["kn", "nk"])
@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh"])
def test_gemm_parity_random(lib, b_layout, act):
    for i, (M, N, K) in enumerate(SHAPES):
        dtype = "bf16" if i % 2 == 0 else "fp16"
        a, b, bias = aw.make_gemm(M, N, K, dtype, b_layout, 4100 + i)
        print(f"\n[case] gemm random {dtype} {b_layout} M={M} N={N} K={K} act={act}", flush=True)
        check(run(a, b, bias, act, b_layout), a, b, bias, act, b_layout, dtype, f"{dtype} {b_layout} {M}x{N}x{K} {act}")


def test_gemm_k_zero_is_the_activated_bias(lib):
    for act in ("none", "relu", "gelu_tanh"):
        bias = aw.make_gemm(3, 70, 8, "bf16", "nk", 4200)[2]
        a = torch.empty((37, 0), dtype=torch.bfloat16, device="cuda")
        b = torch.empty((70, 0), dtype=torch.bfloat16, device="cuda")
        c = eta.gemm_bias_act(a, b, bias.cuda(), act, "nk")
        torch.cuda.synchronize()
        check(c, a.cpu(), b.cpu(), bias, act, "nk", "bf16", f"K=0 {act}")
    c = eta.gemm_bias_act(a, b, None, "none", "nk")
    torch.cuda.synchronize()
    assert (c == 0).all()


@pytest.mark.parametrize("b_layout", ["kn", "nk"])
def test_gemm_strided_operands_and_output(lib, b_layout):
    """Row strides beyond the logical widths (views of wider buffers), a 2-byte-aligned
    C (element stores), and padding between rows left untouched."""
    M, N, K = 150, 200, 96
    a_big, b_big, bias = aw.make_gemm(M, N + 24, K + 40, "bf16", b_layout, 4300)
    a = a_big[:, 8:8 + K]                                      # lda = K + 40, offset 16 bytes
    b = b_big[:K, 16:16 + N] if b_layout == "kn" else b_big[:N, 8:8 + K]
    bias = bias[:N].contiguous()
    for c_off in (0, 1):                                       # 1: C rows start 2 bytes past 8-byte alignment
        c_big = torch.full((M, N + 11), 7.0, dtype=torch.bfloat16, device="cuda")
        c = c_big[:, c_off:c_off + N]
        print(f"\n[case] gemm strided {b_layout} c_off={c_off}", flush=True)
        eta.gemm_bias_act(a.cuda(), b.cuda(), bias.cuda(), "relu", b_layout, c=c)
        torch.cuda.synchronize()
        check(c, a, b, bias, "relu", b_layout, "bf16", f"strided {b_layout} c_off={c_off}")
        cb = c_big.cpu()
        assert (cb[:, :c_off] == 7.0).all() and (cb[:, c_off + N:] == 7.0).all(), "C padding was written"


def test_gemm_many_tiles_in_m(lib):
    """More than 256 tile rows and a ragged last tile (grid of 274 x 1 work-groups)."""
    M, N, K = 70001, 96, 64
    a, b, bias = aw.make_gemm(M, N, K, "bf16", "nk", 4400)
    c = run(a, b, bias, "none", "nk")
    rows = torch.from_numpy(np.unique(np.concatenate([np.arange(4), np.arange(M - 300, M),
                                                      np.random.default_rng(1).choice(M, 200, False)])))
    check(c, a, b, bias, "none", "nk", "bf16", "M=70001", rows=rows)


@pytest.mark.parametrize("name", [w.name for w in aw.GEMM_WORKLOADS])
def test_gemm_full_size_workloads(lib, name):
    """The benchmark's shapes at full size, launched as bench.py launches them: 48
    sampled rows (first and last included) match the oracle element by element."""
    w = aw.gemm_by_name(name)
    print(f"\n[case] gemm workload {name}", flush=True)
    a, b, bias = aw.gemm_workload_inputs(w)
    c = eta.gemm_bias_act(a.cuda(), b.cuda(), bias.cuda() if w.bias else None, w.act, w.b_layout)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.unique(np.concatenate([[0, w.M - 1], np.random.default_rng(w.seed).choice(w.M, 46, False)])))
    check(c, a, b, bias if w.bias else None, w.act, w.b_layout, w.dtype, name, rows=rows)


@pytest.mark.parametrize("b_layout", ["kn", "nk"])
def test_gemm_binding_pads_unaligned_operands(lib, b_layout):
    """K not a multiple of 8 and rows not 16-byte aligned: the binding copies A and B
    into zero-padded buffers before the call; the result is the same product."""
    for M, N, K in ((9, 13, 13), (40, 70, 21), (3, 5, 1)):
        a, b, bias = int_inputs(M, N, K, b_layout, "bf16", 4500 + K)
        print(f"\n[case] gemm padded by the binding {b_layout} M={M} N={N} K={K}", flush=True)
        c = run(a, b, bias, "relu", b_layout)
        want = torch.from_numpy(oracle_c(a, b, bias, "relu", b_layout)).to(torch.bfloat16)
        assert torch.equal(c.view(torch.int16), want.view(torch.int16))
    # an A whose rows start 2 bytes past a 16-byte boundary
    a_big, b, bias = int_inputs(64, 48, 33, b_layout, "bf16", 4600)
    a = a_big.cuda()[:, 1:33]
    c = eta.gemm_bias_act(a, b[:32].cuda() if b_layout == "kn" else b[:, :32].cuda(), bias.cuda(), "none", b_layout)
    torch.cuda.synchronize()
    bl = b[:32] if b_layout == "kn" else b[:, :32]
    want = torch.from_numpy(oracle_c(a.cpu(), bl, bias, "none", b_layout)).to(torch.bfloat16)
    assert torch.equal(c.cpu().view(torch.int16), want.view(torch.int16))
