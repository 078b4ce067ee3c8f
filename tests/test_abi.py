"""The C ABI without a GPU: the library loads, exports every function include/attn.h
declares, maps status codes to text, and rejects bad arguments on the host before
any device work (no compute call is made here)."""
import ctypes
import math
import os
import re

import pytest

import exact_tiled_attention_03_amd as eta
from conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "attn.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(eta.LIB_PATH):
        from exact_tiled_attention_03_amd.build import build
        build()
    return eta.load_library()


def declared_functions(headers=None):
    """Function names declared (outside comments) in the given headers, default all of include/*.h."""
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_]\w*)\s*\(", text, flags=re.M))
    return sorted(names)


def declared_enum(name_prefix, header=HEADER):
    text = open(header).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(rf"\b({name_prefix}\w+)\s*=\s*(\d+)", text)}


def test_header_declares_entry_points():
    assert declared_functions([HEADER]) == ["attn_fwd", "attn_fwd_schedule", "attn_fwd_window", "attn_fwd_workspace_bytes",
                                            "attn_fwd_ws", "attn_status_string"]
    assert declared_functions() == ["attn_bwd", "attn_bwd_noalloc", "attn_fwd", "attn_fwd_schedule",
                                    "attn_fwd_window", "attn_fwd_workspace_bytes", "attn_fwd_ws", "attn_lse_merge",
                                    "attn_status_string", "gemm_bias_act", "softmax_rows"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libattn.so does not export {name}"


def test_python_constants_match_header():
    enum = declared_enum("ATTN_")
    assert enum["ATTN_F16"] == eta.ATTN_F16 and enum["ATTN_BF16"] == eta.ATTN_BF16
    assert enum["ATTN_F32"] == eta.ATTN_F32
    assert enum["ATTN_OK"] == eta.ATTN_OK


def test_status_strings(lib):
    codes = {k: v for k, v in declared_enum("ATTN_").items() if k.startswith("ATTN_ERR") or k == "ATTN_OK"}
    seen = set()
    for name, code in codes.items():
        s = eta.attn_status_string(code)
        assert s and s != "unknown status", name
        seen.add(s)
    assert len(seen) == len(codes)
    assert eta.attn_status_string(999) == "unknown status"


A = 0x10000          # fake, 16-byte aligned, never dereferenced: validation fails before any use
SZ = 1 << 24         # spacing that keeps the fake buffers disjoint


def call(lib, q=A, k=A + SZ, v=A + 2 * SZ, out=A + 3 * SZ, lse=A + 4 * SZ, B=1, H=1, N=16, d=64, causal=1,
         scale=0.125, dtype=0):
    return lib.attn_fwd(q, k, v, out, lse, B, H, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=0), 2), (dict(B=1 << 20, H=1 << 12, N=1 << 10), 2),
    (dict(d=96), 3), (dict(d=32), 3), (dict(d=0), 3),
    (dict(dtype=2), 4), (dict(dtype=-1), 4),
    (dict(scale=math.inf), 5), (dict(scale=math.nan), 5), (dict(scale=-math.inf), 5),
    (dict(q=A + 8), 6), (dict(out=A + 3 * SZ + 2), 6), (dict(lse=A + 4 * SZ + 2), 6),
    (dict(causal=2), 9), (dict(causal=-1), 9),
    (dict(out=A + 64), 10), (dict(lse=A + 3 * SZ + 16), 10), (dict(lse=A + 2 * SZ), 10),
])
def test_argument_validation(lib, kw, code):
    assert call(lib, **kw) == code, eta.attn_status_string(code)


def call_window(lib, window, **kw):
    a = dict(q=A, k=A + SZ, v=A + 2 * SZ, out=A + 3 * SZ, lse=A + 4 * SZ, B=1, H=1, N=16, d=64, causal=1,
             scale=0.125, dtype=0)
    a.update(kw)
    return lib.attn_fwd_window(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                               a["causal"], window, a["scale"], a["dtype"], None)


@pytest.mark.parametrize("window,kw,code", [
    (-1, {}, 11), (-100, dict(causal=0), 11),
    (4, dict(q=None), 1), (4, dict(d=96), 3), (4, dict(causal=2), 9), (4, dict(scale=math.nan), 5),
    (4, dict(out=A + 64), 10), (4, dict(B=0), 2),
])
def test_window_argument_validation(lib, window, kw, code):
    assert call_window(lib, window, **kw) == code, eta.attn_status_string(code)


def test_window_valid_arguments_reach_the_device_check(lib):
    if gpu_available():
        pytest.skip("device check refuses only where no gfx950 is current")
    for w in (0, 1, 7, 16, 10**9):
        assert call_window(lib, w) == 7


WS = A + 8 * SZ      # fake workspace, 256-byte aligned, disjoint from the other fake buffers


def call_ws(lib, ws=WS, ws_bytes=1 << 30, **kw):
    a = dict(q=A, k=A + SZ, v=A + 2 * SZ, out=A + 3 * SZ, lse=A + 4 * SZ, B=1, H=1, N=16, d=64, causal=0,
             scale=0.125, dtype=0)
    a.update(kw)
    return lib.attn_fwd_ws(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["causal"],
                           a["scale"], a["dtype"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(B=0), 2), (dict(N=0), 2), (dict(d=96), 3),
    (dict(dtype=2), 4), (dict(scale=math.nan), 5), (dict(q=A + 8), 6), (dict(causal=2), 9),
    (dict(out=A + 64), 10), (dict(lse=A + 2 * SZ), 10),
])
def test_ws_argument_validation(lib, kw, code):
    """attn_fwd_ws checks the arguments attn_fwd checks before any device query."""
    assert call_ws(lib, **kw) == code, eta.attn_status_string(code)
    assert call_ws(lib, ws=None, ws_bytes=0, **kw) == code


def test_ws_valid_arguments_reach_the_device_check(lib):
    if gpu_available():
        pytest.skip("device check refuses only where no gfx950 is current")
    for kw in (dict(), dict(causal=1), dict(lse=None), dict(ws=None, ws_bytes=0), dict(ws_bytes=0)):
        assert call_ws(lib, **kw) == 7
    assert lib.attn_fwd_workspace_bytes(1, 24, 3000, 80, 0) == -7


@pytest.mark.parametrize("args,code", [
    ((0, 1, 16, 64, 0), 2), ((1, 1, 0, 64, 0), 2), ((1, 1, 16, 96, 0), 3), ((1, 1, 16, 64, 2), 9),
])
def test_workspace_bytes_rejects_bad_shapes(lib, args, code):
    assert lib.attn_fwd_workspace_bytes(*args) == -code


def test_lse_may_be_null_then_device_is_checked(lib):
    """Valid arguments get past validation; without a gfx950 the device check refuses."""
    if gpu_available():
        pytest.skip("device check refuses only where no gfx950 is current")
    assert call(lib, lse=None) == 7
    assert call(lib) == 7


def test_schedule_choice(lib):
    import attn_workloads as aw
    want = {"causal_b1_h1_n128_d64_fp16": 0, "causal_b4_h16_n1024_d64_fp16": 0,
            "causal_b2_h32_n4096_d128_bf16": 1, "long_b1_h16_n32768_d128_bf16": 1, "ragged_b3_h8_n3000_d80_fp16": 0}
    for w in aw.WORKLOADS:
        for c in w.causal_modes:
            assert eta.attn_fwd_schedule(w.B, w.H, w.N, w.d, c) == want[w.name], (w.name, c)
    assert eta.attn_fwd_schedule(8, 64, 200, 80, 1) == 1      # 512 heads of one 256-query tile
    assert eta.attn_fwd_schedule(8, 63, 200, 80, 1) == 0
    assert eta.ATTN_SCHEDULE_SPLIT == 2
    # d = 64, N >= 2048, fewer than 512 work-groups of 128 queries: the key split
    assert eta.attn_fwd_schedule(1, 16, 4096, 64, 1) == 2     # 16 pairs x 16 heads = 256
    assert eta.attn_fwd_schedule(1, 32, 4096, 64, 1) == 0     # 512
    assert eta.attn_fwd_schedule(1, 31, 4096, 64, 1) == 2
    assert eta.attn_fwd_schedule(1, 15, 2048, 64, 0) == 2     # 16 tiles x 15 heads = 240
    assert eta.attn_fwd_schedule(1, 15, 2047, 64, 0) == 0     # N below 2048
    assert eta.attn_fwd_schedule(1, 4, 4096, 80, 1) == 0      # d = 80 never splits
    assert eta.attn_fwd_schedule(8, 64, 2048, 64, 1) == 1     # wide wins first
    assert eta.attn_fwd_schedule(1, 16, 2048, 64, 1) == 0     # causal below 4096 keys: 256 unpaired tiles
    assert eta.attn_fwd_schedule(1, 32, 2048, 64, 1) == 0     # 512 unpaired tiles
    assert eta.attn_fwd_schedule(1, 33, 2048, 64, 1) == 2     # 528: pairs, and the key split
    assert eta.attn_fwd_schedule(1, 16, 2048, 64, 0) == 2     # non-causal keeps the split from 2048
    assert eta.attn_fwd_schedule(1, 1, 8, 96, 0) == -3
    assert eta.attn_fwd_schedule(0, 1, 8, 64, 0) == -2
    assert lib.attn_fwd_schedule(1, 1, 8, 64, 3) == -9   # the binding itself coerces causal to 0/1


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        eta.attn_fwd(q, q, q, torch.empty_like(q), None, True, 0.125)


# --- softmax_rows (include/softmax.h) -----------------------------------------

def call_softmax(lib, x=A, xs=64, y=A + SZ, ys=64, rows=4, cols=50, dtype=2):
    return lib.softmax_rows(x, xs, y, ys, rows, cols, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(y=None), 1),
    (dict(rows=0), 2), (dict(rows=-3), 2), (dict(cols=0), 2), (dict(xs=49), 2), (dict(ys=10), 2),
    (dict(xs=1 << 62), 2), (dict(rows=1 << 30, xs=1 << 20), 2),
    (dict(dtype=3), 4), (dict(dtype=-1), 4),
    (dict(x=A + 2), 6), (dict(y=A + SZ + 1), 6), (dict(dtype=0, x=A + 1), 6), (dict(dtype=1, y=A + SZ + 3), 6),
    (dict(y=A + 16), 10), (dict(y=A, ys=128), 10), (dict(y=A + 3 * 64 * 4 + 48), 10),
])
def test_softmax_argument_validation(lib, kw, code):
    assert code != 0   # every case here must fail validation: the fake pointers are never dereferenced
    assert call_softmax(lib, **kw) == code, eta.attn_status_string(code)


def test_softmax_valid_arguments_reach_the_device_check(lib):
    # valid arguments would launch on the fake pointers where a gfx950 is current
    if gpu_available():
        pytest.skip("device check refuses only where no gfx950 is current")
    for kw in (dict(), dict(y=A), dict(x=A + SZ, y=A), dict(rows=1, cols=1, xs=1 << 20, ys=4), dict(dtype=0, cols=64),
               dict(dtype=1, cols=1 << 20, xs=1 << 20, ys=1 << 20, y=A + (1 << 23)),
               dict(y=A + 4 * 64 * 4),   # y starts just past x's last row
               dict(x=A + 4, xs=63), dict(dtype=0, x=A + 2, xs=51, y=A + SZ + 6)):   # element-aligned rows
        assert call_softmax(lib, **kw) == 7, kw


def test_softmax_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        eta.softmax_rows(x)                       # on the CPU
    with pytest.raises(ValueError):
        eta.softmax_rows(torch.zeros(2, 3, 4))    # not 2-D


# --- gemm_bias_act (include/gemm.h) ---------------------------------------------

def call_gemm(lib, a=A, lda=64, b=A + SZ, ldb=64, b_layout=1, bias=A + 2 * SZ, c=A + 3 * SZ, ldc=64, M=4, N=5,
              K=16, act=0, dtype=1):
    return lib.gemm_bias_act(a, lda, b, ldb, b_layout, bias, c, ldc, M, N, K, act, dtype, None)


def test_gemm_enums_match_binding():
    enum = declared_enum("GEMM_", os.path.join(ROOT, "include", "gemm.h"))
    assert enum["GEMM_ACT_NONE"] == eta.GEMM_ACT["none"] and enum["GEMM_ACT_RELU"] == eta.GEMM_ACT["relu"]
    assert enum["GEMM_ACT_GELU_TANH"] == eta.GEMM_ACT["gelu_tanh"]
    assert enum["GEMM_B_KN"] == eta.GEMM_B_KN and enum["GEMM_B_NK"] == eta.GEMM_B_NK
    assert declared_enum("ATTN_ERR_")["ATTN_ERR_LAYOUT"] == 12


@pytest.mark.parametrize("kw,code", [
    (dict(a=None), 1), (dict(b=None), 1), (dict(c=None), 1), (dict(c=None, K=0), 1),
    (dict(M=0), 2), (dict(N=-1), 2), (dict(K=-8), 2), (dict(K=12), 2), (dict(K=3), 2), (dict(lda=8), 2),
    (dict(ldb=8), 2), (dict(b_layout=0, ldb=4), 2), (dict(ldc=4), 2), (dict(lda=1 << 23), 2),
    (dict(b_layout=0, ldb=(1 << 24) + 8), 2), (dict(ldb=1 << 23), 2),
    (dict(dtype=2), 4), (dict(dtype=-1), 4),
    (dict(b_layout=2), 12), (dict(b_layout=-1), 12), (dict(act=3), 12), (dict(act=-1), 12),
    (dict(a=A + 8), 6), (dict(b=A + SZ + 2), 6), (dict(lda=60), 6), (dict(ldb=20), 6),
    (dict(c=A + 3 * SZ + 1), 6), (dict(bias=A + 2 * SZ + 1), 6),
    (dict(c=A), 10), (dict(c=A + SZ + 64), 10), (dict(c=A + 2 * SZ - 8), 10), (dict(bias=A + 3 * SZ + 4), 10),
])
def test_gemm_argument_validation(lib, kw, code):
    assert code != 0   # every case here must fail validation: the fake pointers are never dereferenced
    assert call_gemm(lib, **kw) == code, eta.attn_status_string(code)


def test_gemm_valid_arguments_reach_the_device_check(lib):
    # valid arguments would launch on the fake pointers where a gfx950 is current
    if gpu_available():
        pytest.skip("device check refuses only where no gfx950 is current")
    for kw in (dict(), dict(bias=None), dict(b_layout=0), dict(act=2, dtype=0), dict(a=None, b=None, K=0),
               dict(M=1 << 20, N=1 << 10, lda=16, ldb=16, ldc=1 << 10, c=A + (1 << 40))):
        assert call_gemm(lib, **kw) == 7, kw


def test_gemm_binding_rejects_bad_tensors():
    import torch
    a = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        eta.gemm_bias_act(a, torch.zeros(16, 8, dtype=torch.bfloat16))          # on the CPU
    with pytest.raises(ValueError):
        eta.gemm_bias_act(a, torch.zeros(15, 8, dtype=torch.bfloat16))          # inner dims differ
    with pytest.raises(TypeError):
        eta.gemm_bias_act(a, torch.zeros(16, 8, dtype=torch.float16))           # dtypes differ
    with pytest.raises(ValueError):
        eta.gemm_bias_act(a, torch.zeros(16, 8, dtype=torch.bfloat16), act="tanh")


# --- attn_bwd, attn_lse_merge (include/attn_bwd.h) ---------------------------------

def call_bwd(lib, **kw):
    a = dict(q=A, k=A + SZ, v=A + 2 * SZ, out=A + 3 * SZ, lse=A + 4 * SZ, dout=A + 5 * SZ, dq=A + 6 * SZ,
             dk=A + 7 * SZ, dv=A + 8 * SZ, delta=A + 9 * SZ, B=1, H=2, N=16, d=64, causal=1, scale=0.125, dtype=1)
    a.update(kw)
    return lib.attn_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"], a["delta"],
                        a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(lse=None), 1), (dict(dout=None), 1), (dict(dv=None), 1), (dict(delta=None), 1),
    (dict(B=0), 2), (dict(N=0), 2), (dict(d=96), 3), (dict(dtype=2), 4), (dict(scale=math.nan), 5),
    (dict(q=A + 8), 6), (dict(dk=A + 7 * SZ + 2), 6), (dict(delta=A + 9 * SZ + 2), 6), (dict(causal=3), 9),
    (dict(dq=A + 64), 10), (dict(dv=A + 6 * SZ + 16), 10), (dict(delta=A + 8 * SZ), 10), (dict(dk=A + 5 * SZ), 10),
])
def test_bwd_argument_validation(lib, kw, code):
    assert code != 0   # every case must fail validation: the fake pointers are never dereferenced
    assert call_bwd(lib, **kw) == code, eta.attn_status_string(code)


def call_merge(lib, op=A, lp=A + SZ, G=3, o=A + 2 * SZ, lse=A + 3 * SZ, R=100, d=128, dtype=1):
    return lib.attn_lse_merge(op, lp, G, o, lse, R, d, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), 1), (dict(lse=None), 1), (dict(G=0), 2), (dict(R=0), 2), (dict(d=96), 3), (dict(dtype=2), 4),
    (dict(op=A + 8), 6), (dict(lse=A + 3 * SZ + 2), 6), (dict(o=A + 64), 10), (dict(lse=A + SZ + 4), 10),
    (dict(o=A + 3 * SZ - 16), 10),
])
def test_merge_argument_validation(lib, kw, code):
    assert code != 0
    assert call_merge(lib, **kw) == code, eta.attn_status_string(code)


def test_bwd_and_merge_valid_arguments_reach_the_device_check(lib):
    # valid arguments would launch on the fake pointers where a gfx950 is current
    if gpu_available():
        pytest.skip("device check refuses only where no gfx950 is current")
    assert call_bwd(lib) == 7 and call_bwd(lib, causal=0, d=80, scale=-0.3) == 7
    assert call_merge(lib) == 7 and call_merge(lib, G=1, R=1, d=64) == 7


def call_bwd_noalloc(lib, **kw):
    a = dict(q=A, k=A + SZ, v=A + 2 * SZ, out=A + 3 * SZ, lse=A + 4 * SZ, dout=A + 5 * SZ, dq=A + 6 * SZ,
             dk=A + 7 * SZ, dv=A + 8 * SZ, B=1, H=2, N=16, d=64, causal=1, scale=0.125, dtype=1)
    a.update(kw)
    return lib.attn_bwd_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                                a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"], None)


def noalloc_max_rows():
    text = open(os.path.join(ROOT, "include", "attn_bwd.h")).read()
    return int(re.search(r"#define\s+ATTN_BWD_NOALLOC_MAX_ROWS\s+(\d+)", text).group(1))


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(dv=None), 1), (dict(B=0), 2), (dict(d=96), 3), (dict(dtype=2), 4),
    (dict(scale=math.nan), 5), (dict(q=A + 8), 6), (dict(causal=3), 9), (dict(dq=A + 64), 10),
    (dict(B=1, H=1, N=4194305), 2), (dict(B=2, H=4, N=524289), 2),
])
def test_bwd_noalloc_argument_validation(lib, kw, code):
    assert noalloc_max_rows() == 4194304   # the row limit the cases above straddle
    assert call_bwd_noalloc(lib, **kw) == code, eta.attn_status_string(code)


def test_bwd_noalloc_valid_arguments_reach_the_device_check(lib):
    if gpu_available():
        pytest.skip("device check refuses only where no gfx950 is current")
    assert call_bwd_noalloc(lib) == 7
    big = 1 << 30   # buffers of 512 MiB, kept disjoint
    ptrs = {n: A + i * big for i, n in enumerate(("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv"))}
    assert call_bwd_noalloc(lib, B=1, H=1, N=4194304, d=64, **ptrs) == 7   # exactly at the limit
