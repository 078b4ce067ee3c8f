"""GPU parity of the attention backward (attn_bwd) and of the merge of key-sharded
results (attn_lse_merge), include/attn_bwd.h, against the float64 oracles of
oracle/backward.py (pinned in test_oracle_bwd_pins.py).

Backward inputs: q, k, v, dO seeded; O and lse from the float64 forward oracle,
O rounded to the input type and lse to fp32 (what a forward hands over).

Bar (u_out = unit roundoff of the 16-bit type, 2^-8 bf16, 2^-11 fp16).  The
kernels round two things besides the outputs: P and dS become 16-bit MFMA
operands (as the forward rounds P), and D is formed from the 16-bit O, which
moves D_i by at most u_out E_i with E_i = sum_c |dO_ic O_ic|, i.e. dS_ij by
P_ij u_out E_i.  Propagating these through the three products, with P, dS from
the oracle:
    |dV - ref| <= u_out (P^T |dO|)                                + u_out |ref|
    |dK - ref| <= u_out |scale| (|dS|^T |Q| + (P E)^T |Q|)        + u_out |ref|
    |dQ - ref| <= u_out |scale| (|dS| |K| + (P E) |K|)            + u_out |ref|
plus 2e-5 (1 + the propagated term) for the fp32 evaluation of exp, the
products and their sums.

Merge: against the oracle merge of the same 16-bit parts, within
u_out |ref| + 1e-5 (1 + max_g |O_g|) (fp32 weights and sums, one rounding).
"""
import math

import numpy as np
import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta
import oracle
from oracle import backward as ob

pytestmark = pytest.mark.gpu

U_OUT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def bwd_inputs(shape, dtype, seed, causal, scale):
    q, k, v = aw.make_inputs(shape, dtype, seed)
    do = aw.make_inputs(shape, dtype, seed + 500)[0]
    O, L = oracle.attention(q, k, v, causal, scale)
    out = torch.from_numpy(O).to(TORCH[dtype])
    lse = torch.from_numpy(L).to(torch.float32)
    return q, k, v, do, out, lse


def run_bwd(q, k, v, do, out, lse, causal, scale):
    dq, dk, dv, delta = eta.attn_bwd(*(t.cuda() for t in (q, k, v, out, lse, do)), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu(), delta.cpu()


def check_bwd(got, q, k, v, do, causal, scale, dtype, label, heads=None, fwd_err=None):
    """got = (dq, dk, dv) CPU tensors; heads = optional list of (b, h) to compare.

    fwd_err = (|O_fwd - O|, |lse_fwd - lse|) when the backward was fed a forward's
    outputs rather than the oracle's: those measured errors are carried through
    the backward's products to first order and added to the bar.  With
    eta_i = exp(|dlse_i|) - 1 the rebuilt P_ij moves by at most P_ij eta_i, D_i
    by at most dD_i = sum_c |dO_ic| |dO_fwd_ic|, so dS_ij by at most
    P_ij eta_i |dP_ij - D_i| + P_ij dD_i, and dV, dK, dQ by P eta and that dS
    bound propagated through their products (|.| of the other operand)."""
    u = U_OUT[dtype]
    sel = (lambda t: t) if heads is None else (lambda t: np.stack([np.asarray(t)[b, h] for b, h in heads])[None])
    Q, K, V, dO = (sel(t.double().numpy()) for t in (q, k, v, do))
    dq_r, dk_r, dv_r = ob.attention_bwd(Q, K, V, dO, causal, scale)
    P = oracle.softmax_weights(Q, K, causal, scale)
    O = P @ V
    dP = dO @ np.swapaxes(V, -1, -2)
    D = (dO * O).sum(-1, keepdims=True)
    dS = P * (dP - D)
    E = (np.abs(dO) * np.abs(O)).sum(-1, keepdims=True)
    PE = P * E
    s = abs(float(np.float32(scale)))
    t_dv = np.swapaxes(P, -1, -2) @ np.abs(dO)
    t_dk = s * (np.swapaxes(np.abs(dS), -1, -2) @ np.abs(Q) + np.swapaxes(PE, -1, -2) @ np.abs(Q))
    t_dq = s * (np.abs(dS) @ np.abs(K) + PE @ np.abs(K))
    extra = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    if fwd_err is not None:
        o_err, l_err = (sel(np.asarray(e, dtype=np.float64)) for e in fwd_err)
        eta = np.expm1(l_err)[..., None]
        dD = (np.abs(dO) * o_err).sum(-1, keepdims=True)
        Peta = P * eta
        dS_err = Peta * np.abs(dP - D) + P * dD
        extra["dv"] = np.swapaxes(Peta, -1, -2) @ np.abs(dO)
        extra["dk"] = s * (np.swapaxes(dS_err, -1, -2) @ np.abs(Q))
        extra["dq"] = s * (dS_err @ np.abs(K))
    for name, g, ref, t in (("dq", got[0], dq_r, t_dq), ("dk", got[1], dk_r, t_dk), ("dv", got[2], dv_r, t_dv)):
        gv = sel(g.double().numpy())
        bound = u * t + u * np.abs(ref) + 2e-5 * (1.0 + t) + 1.01 * extra[name]
        err = np.abs(gv - ref)
        if not (err <= bound).all():
            i = np.unravel_index(np.argmax(err - bound), err.shape)
            raise AssertionError(f"{label} {name}: err {err[i]:.3e} > bound {bound[i]:.3e} at {i} "
                                 f"(got {gv[i]:.5f}, ref {ref[i]:.5f})")


CASES = [((1, 2, 64, 64), "fp16"), ((2, 2, 128, 64), "bf16"), ((1, 3, 300, 80), "fp16"), ((2, 2, 257, 128), "bf16"),
         ((1, 1, 1, 64), "bf16"), ((1, 2, 33, 128), "fp16"), ((1, 2, 700, 128), "bf16")]


@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_parity_small(lib, causal):
    for i, (shape, dtype) in enumerate(CASES):
        scale = 1.0 / math.sqrt(shape[3])
        print(f"\n[case] bwd {shape} {dtype} causal={causal}", flush=True)
        q, k, v, do, out, lse = bwd_inputs(shape, dtype, 5000 + i, causal, scale)
        got = run_bwd(q, k, v, do, out, lse, causal, scale)
        check_bwd(got, q, k, v, do, causal, scale, dtype, f"{shape} {dtype} causal={causal}")
        # delta is D_i of the 16-bit O
        D = (do.double() * out.double()).sum(-1).numpy()
        E = (do.double().abs() * out.double().abs()).sum(-1).numpy()
        assert (np.abs(got[3].double().numpy() - D) <= 1e-6 * (1 + E)).all()


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9])
def test_bwd_odd_scales(lib, scale):
    shape, dtype = (1, 2, 190, 64), "bf16"
    for causal in (0, 1):
        print(f"\n[case] bwd scale={scale} causal={causal}", flush=True)
        q, k, v, do, out, lse = bwd_inputs(shape, dtype, 5100, causal, scale)
        got = run_bwd(q, k, v, do, out, lse, causal, scale)
        check_bwd(got, q, k, v, do, causal, scale, dtype, f"scale={scale} causal={causal}")


def test_bwd_after_gpu_forward(lib):
    """The library's own forward output and lse fed to the backward (the training step's
    order): the gradients stay within the backward's bar plus the forward's measured
    output and lse errors carried through the backward's products."""
    shape, dtype, causal = (2, 4, 512, 128), "bf16", 1
    scale = 1.0 / math.sqrt(128)
    q, k, v = aw.make_inputs(shape, dtype, 5200)
    do = aw.make_inputs(shape, dtype, 5700)[0]
    out, lse = eta.attention(q.cuda(), k.cuda(), v.cuda(), True, scale)
    dq, dk, dv, _ = eta.attn_bwd(q.cuda(), k.cuda(), v.cuda(), out, lse, do.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    O, L = oracle.attention(q, k, v, causal, scale)
    fwd_err = (np.abs(out.cpu().double().numpy() - O), np.abs(lse.cpu().double().numpy() - L))
    check_bwd((dq.cpu(), dk.cpu(), dv.cpu()), q, k, v, do, causal, scale, dtype, "after the GPU forward",
              fwd_err=fwd_err)


def test_bwd_full_size_headline_heads(lib):
    """Causal B=2 H=32 N=4096 d=128 bf16 (the forward's headline shape) at full size:
    every row of two heads against the oracle."""
    shape, dtype, causal = (2, 32, 4096, 128), "bf16", 1
    scale = 1.0 / math.sqrt(128)
    q, k, v = aw.make_inputs(shape, dtype, 5300)
    do = aw.make_inputs(shape, dtype, 5800)[0]
    heads = [(0, 0), (1, 31)]
    # O and lse of all heads from the GPU forward (the oracle would take minutes for 64 heads)
    out, lse = eta.attention(q.cuda(), k.cuda(), v.cuda(), True, scale)
    # replace the two checked heads' O, lse by the oracle's, so the bar's inputs are exact
    for b, h in heads:
        O, L = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], causal, scale)
        out[b, h] = torch.from_numpy(O[0, 0]).to(torch.bfloat16).cuda()
        lse[b, h] = torch.from_numpy(L[0, 0]).to(torch.float32).cuda()
    print("\n[case] bwd headline shape, two heads checked", flush=True)
    dq, dk, dv, _ = eta.attn_bwd(q.cuda(), k.cuda(), v.cuda(), out, lse, do.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    check_bwd((dq.cpu(), dk.cpu(), dv.cpu()), q, k, v, do, causal, scale, dtype, "headline", heads=heads)


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (80, "fp16"), (128, "bf16")])
def test_lse_merge_parity(lib, d, dtype):
    B, H, N = 2, 3, 157
    q, k, v = aw.make_inputs((B, H, N, d), dtype, 5400 + d)
    scale = 1.0 / math.sqrt(d)
    for cuts in ([0, N], [0, 50, N], [0, 1, 2, 90, 130, N]):
        parts = [oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0, scale) for a, b in zip(cuts, cuts[1:])]
        o_parts = torch.stack([torch.from_numpy(p[0]).to(TORCH[dtype]) for p in parts])
        l_parts = torch.stack([torch.from_numpy(p[1]).to(torch.float32) for p in parts])
        # an empty shard for some rows and a row with every shard empty
        if len(parts) > 2:
            l_parts[1, 0, 0, :10] = -float("inf")
            l_parts[:, 1, 2, 5] = -float("inf")
        print(f"\n[case] merge d={d} {dtype} shards={len(parts)}", flush=True)
        o, lse = eta.attn_lse_merge(o_parts.cuda(), l_parts.cuda())
        torch.cuda.synchronize()
        ro, rl = ob.lse_merge(o_parts.double().numpy(), l_parts.double().numpy())
        got_o, got_l = o.cpu().double().numpy(), lse.cpu().double().numpy()
        empty = ~np.isfinite(rl)
        assert (np.isneginf(got_l) == empty).all()
        assert (got_o[empty] == 0).all()
        ok = ~empty
        big = np.abs(o_parts.double().numpy()).max(axis=0)
        assert (np.abs(got_o - ro)[ok] <= (U_OUT[dtype] * np.abs(ro) + 1e-5 * (1 + big))[ok]).all()
        assert (np.abs(got_l[ok] - rl[ok]) <= 1e-5 * (1 + np.abs(rl[ok]))).all()
        if len(parts) == 2 or cuts == [0, N]:
            full_o, full_l = oracle.attention(q, k, v, 0, scale)
            assert np.abs(got_o - full_o).max() <= 3 * U_OUT[dtype] * np.abs(full_o).max() + 1e-5
