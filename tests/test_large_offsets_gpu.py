"""Tensors past 4 GiB: the attention forward and backward address every head from
a 64-bit offset, the GEMM every row of C, the shard merge every row of its parts
and result; the rows and heads checked here include those holding and following
byte 2^32 of their tensors.

Shape B=2 H=52500 N=256 d=80 fp16: 4.30e9 bytes per tensor.  Head bh (= b*H + h)
starts at byte bh * N * d * 2 = 40960 bh, so bh 104857 straddles 2^32 and bh
104858 .. 104999 lie wholly past it (d = 80: a head size that does not divide
2^32, and the padded head dimension).  Inputs are drawn on the GPU (a seeded
torch generator, iid N(0,1) rounded to fp16: a host-side draw of this size would
take minutes) and the checked heads are copied back for the float64 oracle.  The bars are the ones
the other parity tests use: the forward's derived per-element bound, and the
backward's derived gradient bound with the checked heads' O and lse taken from
the oracle."""
import numpy as np
import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
import oracle
from oracle import backward as ob
from parity_util import assert_within_derived_bound
from test_bwd_gpu import U_OUT, check_bwd
from test_gemm_gpu import check as check_gemm

pytestmark = pytest.mark.gpu

B, H, N, D = 2, 52500, 256, 80
SCALE = 0.11
_STRADDLE = 2 ** 32 // (N * D * 2)          # the head holding byte 2^32
# (b, h): the first head, the one straddling byte 2^32, the first past it, the last
HEADS = [(0, 0), (1, _STRADDLE - H), (1, _STRADDLE + 1 - H), (1, H - 1)]


def gpu_normal(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((B, H, N, D), generator=g, device="cuda", dtype=torch.float16)


def head(t, b, h):
    return t[b:b + 1, h:h + 1].cpu()


def test_shape_crosses_4gib():
    bh = [b * H + h for b, h in HEADS]
    per_head = N * D * 2
    assert B * H * per_head > 2 ** 32
    assert bh[1] * per_head < 2 ** 32 < (bh[1] + 1) * per_head
    assert bh[2] * per_head >= 2 ** 32


@pytest.mark.parametrize("causal", [0, 1])
def test_forward_heads_past_4gib(lib, causal):
    print(f"\n[case] forward B={B} H={H} N={N} d={D} fp16 causal={causal}", flush=True)
    q, k, v = (gpu_normal(9900 + i) for i in range(3))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    eta.attn_fwd(q, k, v, out, lse, bool(causal), SCALE)
    torch.cuda.synchronize()
    for b, h in HEADS:
        assert_within_derived_bound(head(out, b, h), head(lse, b, h), head(q, b, h), head(k, b, h), head(v, b, h),
                                    causal, SCALE, label=f"head ({b},{h}) causal={causal}")
    del q, k, v, out, lse
    torch.cuda.empty_cache()


def test_backward_heads_past_4gib(lib):
    print(f"\n[case] backward B={B} H={H} N={N} d={D} fp16 causal", flush=True)
    q, k, v, do = (gpu_normal(9910 + i) for i in range(4))
    out, lse = eta.attention(q, k, v, True, SCALE)
    # the checked heads' O and lse from the oracle, so the bar's inputs are exact
    # (heads are independent: the others' values do not reach them)
    for b, h in HEADS:
        O, L = oracle.attention(head(q, b, h), head(k, b, h), head(v, b, h), 1, SCALE)
        out[b, h] = torch.from_numpy(O[0, 0]).to(torch.float16).cuda()
        lse[b, h] = torch.from_numpy(L[0, 0]).to(torch.float32).cuda()
    dq, dk, dv, delta = eta.attn_bwd(q, k, v, out, lse, do, causal=True, scale=SCALE)
    torch.cuda.synchronize()
    for b, h in HEADS:
        got = (head(dq, b, h), head(dk, b, h), head(dv, b, h))
        check_bwd(got, head(q, b, h), head(k, b, h), head(v, b, h), head(do, b, h), 1, SCALE, "fp16",
                  f"head ({b},{h})")
    del q, k, v, do, out, lse, dq, dk, dv, delta
    torch.cuda.empty_cache()


def test_gemm_output_past_4gib(lib):
    """C of 70000 x 32760 bf16 (4.59e9 bytes): rows from 65552 on (the row holding
    byte 2^32 and those after it) against the oracle, with the GEMM tests' bar."""
    M, N, K = 70000, 32760, 64
    print(f"\n[case] gemm M={M} N={N} K={K} bf16 nk relu", flush=True)
    a, b, bias = aw.make_gemm(M, N, K, "bf16", "nk", 9950)
    c = eta.gemm_bias_act(a.cuda(), b.cuda(), bias.cuda(), "relu", "nk")
    torch.cuda.synchronize()
    assert c.numel() * c.element_size() > 2 ** 32
    straddle = 2 ** 32 // (N * 2)
    rows = torch.tensor([0, straddle - 1, straddle, straddle + 1, M - 1])
    check_gemm(c, a, b, bias, "relu", "nk", "bf16", "C past 4 GiB", rows=rows)
    del c
    torch.cuda.empty_cache()


def test_merge_past_4gib(lib):
    """Two shards of R = 2^32 / 160 + 1000 rows at d = 80 fp16: the parts take 8.6e9
    bytes and the merged O 4.3e9; rows around and past byte 2^32 of O (and the
    matching rows of the parts, past 2^33) against the oracle merge, with the merge
    test's bar; some of them with an empty shard."""
    G, d = 2, 80
    straddle = 2 ** 32 // (d * 2)
    R = straddle + 1000
    print(f"\n[case] merge G={G} R={R} d={d} fp16", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(9960)
    o_parts = torch.randn((G, R, d), generator=g, device="cuda", dtype=torch.float16)
    l_parts = torch.randn((G, R), generator=g, device="cuda", dtype=torch.float32) * 2.0 + 5.0
    rows = torch.tensor([0, 1, straddle - 1, straddle, straddle + 1, R - 2, R - 1])
    l_parts[1, rows[-2:].cuda()] = -float("inf")            # the last two rows: second shard empty
    o, lse = eta.attn_lse_merge(o_parts, l_parts)
    torch.cuda.synchronize()
    assert o.numel() * o.element_size() > 2 ** 32
    op, lp = o_parts[:, rows.cuda()].cpu().double().numpy(), l_parts[:, rows.cuda()].cpu().double().numpy()
    ro, rl = ob.lse_merge(op, lp)
    got_o, got_l = o[rows.cuda()].cpu().double().numpy(), lse[rows.cuda()].cpu().double().numpy()
    big = np.abs(op).max(axis=0)
    assert (np.abs(got_o - ro) <= U_OUT["fp16"] * np.abs(ro) + 1e-5 * (1 + big)).all()
    assert (np.abs(got_l - rl) <= 1e-5 * (1 + np.abs(rl))).all()
    del o_parts, l_parts, o, lse
    torch.cuda.empty_cache()
