"""Run-to-run determinism of the kernels that the parity tests meet only through
tolerances: the 8-wave two-group forward on the headline shape, the backward's dQ and
dK/dV kernels, and the two-group GEMM.  None of them uses atomics or a data-dependent
reduction order, so two calls on the same inputs must agree bit for bit."""
import math

import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def test_forward_wide_schedule_is_deterministic(lib):
    B, H, N, d = 2, 32, 4096, 128
    assert eta.attn_fwd_schedule(B, H, N, d, True) == eta.ATTN_SCHEDULE_WIDE
    q, k, v = (t.cuda() for t in aw.make_inputs((B, H, N, d), "bf16", 31))
    print("\n[case] forward 8-wave headline shape, twice", flush=True)
    o1, l1 = eta.attention(q, k, v, True, 1 / math.sqrt(d))
    o2, l2 = eta.attention(q, k, v, True, 1 / math.sqrt(d))
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o2)) and torch.equal(l1, l2)


def test_backward_is_deterministic(lib):
    shape, scale = (2, 8, 1024, 128), 1 / math.sqrt(128)
    q, k, v = (t.cuda() for t in aw.make_inputs(shape, "bf16", 32))
    do = aw.make_inputs(shape, "bf16", 33)[0].cuda()
    out, lse = eta.attention(q, k, v, True, scale)
    print("\n[case] backward causal (2, 8, 1024, 128) bf16, twice", flush=True)
    r1 = eta.attn_bwd(q, k, v, out, lse, do, causal=True, scale=scale)
    r2 = eta.attn_bwd(q, k, v, out, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(bits(a), bits(b))


def test_gemm_two_group_kernel_is_deterministic(lib):
    a, b, bias = (t.cuda() for t in aw.make_gemm(2048, 1536, 1000, "bf16", "nk", 34))
    print("\n[case] gemm 2048 x 1536 x 1000 bf16, twice", flush=True)
    c1 = eta.gemm_bias_act(a, b, bias, act="gelu_tanh", b_layout="nk")
    c2 = eta.gemm_bias_act(a, b, bias, act="gelu_tanh", b_layout="nk")
    torch.cuda.synchronize()
    assert torch.equal(bits(c1), bits(c2))
