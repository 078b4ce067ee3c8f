"""The entry points under HIP graph capture (torch.cuda.CUDAGraph): each call
enqueues kernels only (no allocation, memset or synchronisation), so a captured
sequence replays the same computation.  Each graph is replayed several times
with new inputs copied in place between replays, eager work and synchronisation
in between, and every replay's outputs must equal, bit for bit, an eager call of
the same entry points on the same inputs (the kernels are deterministic).  Each
entry point is called once eagerly before capture, so its per-device lookups
(architecture check, the no-alloc entry's array address) are already cached."""
import math

import pytest
import torch

import attn_workloads as aw
import exact_tiled_attention_03_amd as eta

pytestmark = pytest.mark.gpu

REPLAYS = 4


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def same(a, b):
    return torch.equal(bits(a), bits(b))


def inputs(shape, dtype, seed):
    """REPLAYS + 1 seeded input sets on the GPU (the first one is used for the capture)."""
    return [[t.cuda() for t in aw.make_inputs(shape, dtype, seed + 10 * i)] for i in range(REPLAYS + 1)]


def test_forward_and_backward_graph(lib):
    B, H, N, d = 2, 4, 1000, 128
    scale = 1.0 / math.sqrt(d)
    sets = inputs((B, H, N, d), "bf16", 7100)
    dos = [aw.make_inputs((B, H, N, d), "bf16", 7600 + i)[0].cuda() for i in range(REPLAYS + 1)]
    q, k, v = (t.clone() for t in sets[0])
    do = dos[0].clone()
    out, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dq2, dk2, dv2 = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def step():
        eta.attn_fwd(q, k, v, out, lse, True, scale)
        eta.attn_bwd(q, k, v, out, lse, do, dq, dk, dv, delta, causal=True, scale=scale)
        eta.attn_bwd_noalloc(q, k, v, out, lse, do, dq2, dk2, dv2, causal=True, scale=scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # eager warm-up: per-device lookups cached
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(1, REPLAYS + 1):
        print(f"\n[case] forward/backward graph replay {i}", flush=True)
        for dst, src in zip((q, k, v, do), (*sets[i], dos[i])):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, lse, dq, dk, dv, dq2, dk2, dv2)]
        step()                                  # eager, on the same inputs
        torch.cuda.synchronize()
        want = (out, lse, dq, dk, dv, dq2, dk2, dv2)
        names = ("out", "lse", "dq", "dk", "dv", "dq (noalloc)", "dk (noalloc)", "dv (noalloc)")
        for name, a, b in zip(names, got, want):
            assert same(a, b), f"replay {i}: {name} differs from the eager call"
        # the two backward entry points agree with each other too
        assert same(dq, dq2) and same(dk, dk2) and same(dv, dv2)


def test_forward_with_workspace_graph(lib):
    """attn_fwd_ws on a shape it splits: two kernels (the key-range parts, then the
    merge) in the graph."""
    B, H, N, d = 1, 20, 3500, 64
    scale = 0.125
    need = eta.attn_fwd_workspace_bytes(B, H, N, d, False)
    if need == 0:
        pytest.skip("this device does not split the shape (fewer than 256 compute units)")
    sets = inputs((B, H, N, d), "fp16", 7200)
    q, k, v = (t.clone() for t in sets[0])
    out, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step():
        eta.attn_fwd_ws(q, k, v, out, lse, False, scale, ws)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(1, REPLAYS + 1):
        print(f"\n[case] attn_fwd_ws graph replay {i}", flush=True)
        for dst, src in zip((q, k, v), sets[i]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        step()
        torch.cuda.synchronize()
        assert same(got[0], out) and same(got[1], lse), f"replay {i}"


def test_softmax_and_gemm_graph(lib):
    rows, cols = 300, 5000
    xs = [aw.make_rows(rows, cols, "bf16", 7300 + i).cuda() for i in range(REPLAYS + 1)]
    M, N, K = 700, 512, 256
    gs = [[t.cuda() for t in aw.make_gemm(M, N, K, "bf16", "nk", 7400 + i)] for i in range(REPLAYS + 1)]
    x = xs[0].clone()
    y = torch.empty_like(x)
    a, b, bias = (t.clone() for t in gs[0])
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        eta.softmax_rows(x, y)
        eta.gemm_bias_act(a, b, bias, "gelu_tanh", "nk", c=c)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(1, REPLAYS + 1):
        print(f"\n[case] softmax/gemm graph replay {i}", flush=True)
        x.copy_(xs[i])
        for dst, src in zip((a, b, bias), gs[i]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = (y.clone(), c.clone())
        step()
        torch.cuda.synchronize()
        assert same(got[0], y) and same(got[1], c), f"replay {i}"
