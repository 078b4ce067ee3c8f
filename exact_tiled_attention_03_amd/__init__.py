"""Python binding of the fused exact-attention forward library (libattn.so, gfx950).

Argument marshalling only: every step of the forward and backward passes, the
merge of key-sharded results, the row softmax and the matrix product with its
epilogue runs in the HIP kernels behind the C ABI declared in include/attn.h,
include/attn_bwd.h, include/softmax.h and include/gemm.h.  torch is used for
device memory and the current stream.  If the compiled library is missing the
binding raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_F16 = 0
ATTN_BF16 = 1
ATTN_F32 = 2
ATTN_OK = 0

GEMM_ACT = {"none": 0, "relu": 1, "gelu_tanh": 2}
GEMM_B_KN = 0
GEMM_B_NK = 1

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"call failed with status {status}: {msg}")
        self.status = status


def load_library():
    """Load libattn.so (built by __graft_entry__.build()); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                             ctypes.c_int, ctypes.c_void_p]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_fwd_window.restype = ctypes.c_int
    lib.attn_fwd_window.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_schedule.restype = ctypes.c_int
    lib.attn_fwd_schedule.argtypes = [ctypes.c_int] * 5
    lib.attn_fwd_ws.restype = ctypes.c_int
    lib.attn_fwd_ws.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_fwd_workspace_bytes.restype = ctypes.c_longlong
    lib.attn_fwd_workspace_bytes.argtypes = [ctypes.c_int] * 5
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                           ctypes.c_void_p]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                                 ctypes.c_void_p]
    lib.attn_lse_merge.restype = ctypes.c_int
    lib.attn_lse_merge.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.gemm_bias_act.restype = ctypes.c_int
    lib.gemm_bias_act.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.softmax_rows.restype = ctypes.c_int
    lib.softmax_rows.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


ATTN_SCHEDULE_SMALL = 0
ATTN_SCHEDULE_WIDE = 1
ATTN_SCHEDULE_SPLIT = 2


def attn_fwd_schedule(B: int, H: int, N: int, d: int, causal: bool) -> int:
    """Kernel schedule attn_fwd uses for this shape (negative status if rejected)."""
    return load_library().attn_fwd_schedule(int(B), int(H), int(N), int(d), int(bool(causal)))


def _dtype_code(t, allow_f32=False):
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if allow_f32 and t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16" + (" or float32" if allow_f32 else ""))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check_attn_tensors(q, k, v, out, lse):
    """Shapes, dtypes and placement of attn_fwd's tensors; returns (B, H, N, d)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("out", out)):
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(B, H, N, d)}")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    tensors = [q, k, v, out] + ([lse] if lse is not None else [])
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if lse is not None:
        import torch
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be float32 [B, H, N]")
    return B, H, N, d


def attn_fwd(q, k, v, out, lse, causal: bool, scale: float, stream=None, window: int = 0) -> None:
    """Enqueue the forward pass on `stream` (default: torch's current stream).

    q, k, v, out: contiguous [B, H, N, d] float16/bfloat16 tensors on the GPU.
    lse: contiguous [B, H, N] float32 tensor on the GPU, or None.
    window: 0 for full attention (attn_fwd), W >= 1 for the sliding window of
    attn_fwd_window (key j kept only if i - W < j, and j < i + W when not causal).
    Raises AttnError with the library's status on rejected arguments."""
    lib = load_library()
    B, H, N, d = _check_attn_tensors(q, k, v, out, lse)
    lse_ptr = lse.data_ptr() if lse is not None else None
    if window:
        st = lib.attn_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                                 B, H, N, d, int(bool(causal)), int(window), float(scale), _dtype_code(q),
                                 _stream_handle(stream))
    else:
        st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse_ptr,
                          B, H, N, d, int(bool(causal)), float(scale), _dtype_code(q), _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, attn_status_string(st))


def attn_fwd_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool) -> int:
    """Workspace bytes attn_fwd_ws uses for this shape on the current device (0: no split)."""
    r = load_library().attn_fwd_workspace_bytes(int(B), int(H), int(N), int(d), int(bool(causal)))
    if r < 0:
        raise AttnError(-r, attn_status_string(-r))
    return r


def attn_fwd_ws(q, k, v, out, lse, causal: bool, scale: float, workspace, stream=None) -> None:
    """attn_fwd_ws: attn_fwd that may cut the last query tiles into key ranges run
    on otherwise idle CUs, with partial results in `workspace` (a contiguous GPU
    tensor of at least attn_fwd_workspace_bytes bytes, or None for attn_fwd)."""
    lib = load_library()
    B, H, N, d = _check_attn_tensors(q, k, v, out, lse)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = lib.attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr() if lse is not None else None, B, H, N, d, int(bool(causal)), float(scale),
                         _dtype_code(q), ws_ptr, ws_bytes, _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, attn_status_string(st))


def attention(q, k, v, causal: bool, scale: float, stream=None, window: int = 0):
    """Allocate out [B,H,N,d] and lse [B,H,N] with torch, then call attn_fwd (or
    attn_fwd_window when window > 0)."""
    import torch
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd(q, k, v, out, lse, causal, scale, stream, window)
    return out, lse


def softmax_rows(x, y=None, stream=None):
    """Row softmax of a 2-D GPU tensor x (float32, float16 or bfloat16) into y.

    y defaults to a new tensor with x's row stride; y may be x itself (in place).
    Rows may be strided (stride(1) must be 1); 16-byte aligned row starts take
    the vectorised kernels.  Enqueued on
    `stream` (default: torch's current stream); returns y.  An empty x has nothing
    to compute and returns y at once.  Raises AttnError with the library's status
    on rejected arguments."""
    import torch
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    if y is None:
        row = x.stride(0) if x.dim() == 2 and x.shape[0] > 1 and x.stride(1) == 1 else x.shape[-1]
        y = torch.empty_strided(tuple(x.shape), (max(row, x.shape[-1]), 1), dtype=x.dtype, device=x.device)
    if tuple(y.shape) != tuple(x.shape) or y.dtype != x.dtype:
        raise ValueError(f"y must match x: {tuple(x.shape)} {x.dtype}")
    for name, t in (("x", x), ("y", y)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} rows must be contiguous (stride(1) == 1)")
    rows, cols = x.shape
    if rows == 0 or cols == 0:
        return y
    st = lib.softmax_rows(x.data_ptr(), x.stride(0) if rows > 1 else cols, y.data_ptr(),
                          y.stride(0) if rows > 1 else cols, rows, cols, _dtype_code(x, allow_f32=True),
                          _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, attn_status_string(st))
    return y


def attn_bwd(q, k, v, out, lse, dout, dq=None, dk=None, dv=None, delta=None, causal=True, scale=None,
             stream=None):
    """Gradients (dq, dk, dv) of attn_fwd for the upstream gradient dout.

    q, k, v, out, dout: contiguous [B, H, N, d] float16/bfloat16 GPU tensors (out
    and lse as attn_fwd returned them); lse: contiguous [B, H, N] float32.
    dq, dk, dv: outputs like q (allocated when None); delta: [B, H, N] float32
    workspace that receives D_i = sum_c dout * out (allocated when None).
    scale defaults to 1/sqrt(d).  Returns (dq, dk, dv, delta)."""
    import math
    import torch
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, H, N, d] of {q.dtype}")
    for name, t in (("lse", lse), ("delta", delta)):
        if tuple(t.shape) != (B, H, N) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [B, H, N]")
    for t in (q, k, v, out, lse, dout, dq, dk, dv, delta):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous GPU tensors")
    st = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, int(bool(causal)),
                      float(scale), _dtype_code(q), _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, attn_status_string(st))
    return dq, dk, dv, delta


def attn_bwd_noalloc(q, k, v, out, lse, dout, dq, dk, dv, causal=True, scale=None, stream=None):
    """attn_bwd_noalloc: the gradients of attn_bwd into the given dq, dk, dv, with D_i
    kept in the library's own per-GPU device array (nothing is allocated, here or in
    the library; B*H*N must not exceed ATTN_BWD_NOALLOC_MAX_ROWS).  Tensors as for
    attn_bwd.  Returns (dq, dk, dv)."""
    import math
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, H, N, d] of {q.dtype}")
    if tuple(lse.shape) != (B, H, N) or str(lse.dtype) != "torch.float32":
        raise ValueError("lse must be float32 [B, H, N]")
    for t in (q, k, v, out, lse, dout, dq, dk, dv):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous GPU tensors")
    st = lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                              int(bool(causal)), float(scale), _dtype_code(q), _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, attn_status_string(st))
    return dq, dk, dv


def attn_lse_merge(o_parts, lse_parts, o=None, lse=None, stream=None):
    """Merge G partial attention results over disjoint key shards.

    o_parts: contiguous [G, ..., d] float16/bfloat16; lse_parts: contiguous
    [G, ...] float32 (natural log, -inf for a shard with no key for a row).
    Returns (o [..., d], lse [...])."""
    import torch
    lib = load_library()
    G = o_parts.shape[0]
    d = o_parts.shape[-1]
    rows_shape = tuple(o_parts.shape[1:-1])
    if tuple(lse_parts.shape) != (G,) + rows_shape or lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be float32 [G, ...] matching o_parts")
    o = torch.empty(rows_shape + (d,), dtype=o_parts.dtype, device=o_parts.device) if o is None else o
    lse = torch.empty(rows_shape, dtype=torch.float32, device=o_parts.device) if lse is None else lse
    for t in (o_parts, lse_parts, o, lse):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous GPU tensors")
    R = 1
    for x in rows_shape:
        R *= x
    st = lib.attn_lse_merge(o_parts.data_ptr(), lse_parts.data_ptr(), G, o.data_ptr(), lse.data_ptr(), R, d,
                            _dtype_code(o_parts), _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, attn_status_string(st))
    return o, lse


def _row_stride(t, rows):
    """Elements between rows of a 2-D tensor whose rows are contiguous."""
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    return t.stride(0) if rows > 1 else t.shape[1]


def _aligned(t, rows):
    """Every row of t starts on a 16-byte boundary."""
    return t.data_ptr() % 16 == 0 and (rows == 1 or t.stride(0) % 8 == 0)


def _padded(t, rows_to, cols_to):
    """t copied into the top-left corner of a zeroed [rows_to, cols_to] buffer on its device."""
    import torch
    out = torch.zeros((rows_to, cols_to), dtype=t.dtype, device=t.device)
    out[:t.shape[0], :t.shape[1]].copy_(t)
    return out


def gemm_bias_act(a, b, bias=None, act="none", b_layout="kn", c=None, stream=None):
    """C = act(A B + bias) on the GPU, fp32 accumulation, one rounding to the input type.

    a: [M, K] float16/bfloat16 with contiguous rows.
    b: [K, N] when b_layout == "kn"; when b_layout == "nk", the [N, K] matrix W
       whose transpose is B (a linear layer's weight: C = a W^T).
    bias: [N] of the same dtype, or None.  act: "none", "relu" or "gelu_tanh".
    c: [M, N] output (allocated when None).  Enqueued on `stream` (default:
    torch's current stream); returns c.  Raises AttnError with the library's
    status on rejected arguments.

    The library reads A and B in 16-byte chunks: it needs 16-byte aligned rows
    and K a multiple of 8.  Operands that do not meet this are first copied on
    the GPU into zero-padded buffers (padding K with zeros adds nothing to the
    sum); every arithmetic step still runs in the library's kernel."""
    import torch
    lib = load_library()
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    if b_layout not in ("kn", "nk"):
        raise ValueError("b_layout must be 'kn' or 'nk'")
    M, K = a.shape
    N = b.shape[1] if b_layout == "kn" else b.shape[0]
    if (b.shape[0] if b_layout == "kn" else b.shape[1]) != K:
        raise ValueError(f"inner dimensions differ: a {tuple(a.shape)}, b {tuple(b.shape)} ({b_layout})")
    if b.dtype != a.dtype or (bias is not None and bias.dtype != a.dtype):
        raise TypeError("a, b and bias must share a dtype")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or (N > 1 and bias.stride(0) != 1)):
        raise ValueError(f"bias must be a contiguous [{N}] vector")
    if act not in GEMM_ACT:
        raise ValueError(f"act must be one of {sorted(GEMM_ACT)}")
    if c is None:
        c = torch.empty((M, N), dtype=a.dtype, device=a.device)
    if tuple(c.shape) != (M, N) or c.dtype != a.dtype:
        raise ValueError(f"c must be [{M}, {N}] of {a.dtype}")
    for name, t in (("a", a), ("b", b), ("c", c)) + ((("bias", bias),) if bias is not None else ()):
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
    if M == 0 or N == 0:
        return c
    if K > 0:
        _row_stride(a, M)
        _row_stride(b, K if b_layout == "kn" else N)
        K8 = -(-K // 8) * 8
        if K8 != K or not _aligned(a, M):
            a = _padded(a, M, K8)
        if b_layout == "kn":
            if K8 != K or not _aligned(b, K):
                b = _padded(b, K8, -(-N // 8) * 8)[:, :N]
        elif K8 != K or not _aligned(b, N):
            b = _padded(b, N, K8)
        K = K8
    lda = _row_stride(a, M) if K > 0 else K
    brows = K if b_layout == "kn" else N
    ldb = _row_stride(b, brows) if K > 0 else (N if b_layout == "kn" else K)
    ldc = _row_stride(c, M)
    st = lib.gemm_bias_act(a.data_ptr() if K > 0 else None, lda, b.data_ptr() if K > 0 else None, ldb,
                           GEMM_B_KN if b_layout == "kn" else GEMM_B_NK,
                           bias.data_ptr() if bias is not None else None, c.data_ptr(), ldc, M, N, K, GEMM_ACT[act],
                           _dtype_code(a), _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, attn_status_string(st))
    return c


def linear(x, weight, bias=None, act="none", stream=None):
    """act(x W^T + bias) for x [M, K] and a weight W [N, K] (gemm_bias_act with b_layout 'nk')."""
    return gemm_bias_act(x, weight, bias, act, "nk", None, stream)


__all__ = ["attn_bwd", "attn_lse_merge", "gemm_bias_act", "linear", "GEMM_ACT", "attn_fwd", "attn_fwd_schedule", "attn_status_string", "attention", "softmax_rows", "load_library",
           "AttnError", "ATTN_F16", "ATTN_BF16", "ATTN_F32", "ATTN_SCHEDULE_SMALL", "ATTN_SCHEDULE_WIDE",
           "ATTN_SCHEDULE_SPLIT"]
