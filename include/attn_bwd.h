/*
 * attn_bwd.h -- C ABI of the exact-attention backward pass and of the merge of
 * attention results computed over disjoint key shards (MI355X, gfx950).
 *
 * Backward.  The pages name fused backward operators only in passing ("Triton:
 * CUDA-level operators in Python", f.mffb.com.cn, section on why Triton) and
 * give no algorithm; what is computed is the derivative of the forward of
 * attn.h ("Triton in depth", ybb.press, 3.1-3.3): with S = scale Q K^T (causal
 * entries j > i removed), P = softmax_rows(S), O = P V and the upstream
 * gradient dO,
 *
 *     D_i = sum_c dO_ic O_ic,   dS = P * (dO V^T - D),
 *     dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 *
 * with P rebuilt tile by tile from the forward's lse (P_ij = exp(S_ij - lse_i)),
 * so the N x N matrices never reach HBM, in the manner of the forward's tiling.
 *
 * Merge.  From the definition of lse (natural log of the row's softmax
 * denominator): results (O_g, lse_g) over key shards g combine as
 * lse = ln sum_g exp(lse_g) and O = sum_g exp(lse_g - lse) O_g; a shard whose
 * lse_g is -inf contributes nothing.  This is the one exchange a key-sharded
 * (context-parallel) forward needs.
 *
 * Status codes and element types are those of attn.h.
 */
#ifndef ETA_ATTN_BWD_H
#define ETA_ATTN_BWD_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_bwd -- dQ, dK, dV of attn_fwd on the current HIP device.
 *
 *   q, k, v, out, dout : device pointers, contiguous [B, H, N, d] of dtype: the
 *              forward's inputs, its output O and the gradient dO of a loss
 *              with respect to O.
 *   lse      : device pointer, contiguous [B, H, N] fp32, the forward's lse
 *              (natural log).
 *   dq, dk, dv : device pointers, contiguous [B, H, N, d] of dtype: written with
 *              the gradients (fp32 accumulation, rounded to nearest even).
 *   delta    : device pointer, contiguous [B, H, N] fp32: written with D_i; the
 *              caller provides it (the library allocates nothing).
 *   B, H, N, d, causal, scale, dtype, stream : as for attn_fwd (d in {64, 80,
 *              128}; scale finite, any sign).
 *
 * Layout and alignment as for attn_fwd (16-byte aligned 16-bit tensors, 4-byte
 * aligned fp32 tensors).  Ownership: caller-owned buffers valid until the work
 * on `stream` completes; dq, dk, dv, delta must not overlap each other or the
 * inputs.
 *
 * Returns ATTN_OK or an attn_status code, checked on the host before any device
 * work: ATTN_ERR_NULL (a pointer is NULL), ATTN_ERR_SHAPE, ATTN_ERR_HEAD_DIM,
 * ATTN_ERR_DTYPE, ATTN_ERR_SCALE, ATTN_ERR_ALIGN, ATTN_ERR_CAUSAL,
 * ATTN_ERR_ALIAS, ATTN_ERR_DEVICE, ATTN_ERR_LAUNCH.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* lse, const void* dout,
             void* dq, void* dk, void* dv, void* delta, int B, int H, int N, int d, int causal, float scale, int dtype,
             void* stream);

/* Rows (B*H*N) of D_i that attn_bwd_noalloc can hold: 4 Mi rows, 16 MiB per GPU. */
#define ATTN_BWD_NOALLOC_MAX_ROWS 4194304

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and gradients, without the delta workspace.  D_i
 * goes to a device array the library owns, one per GPU, of
 * ATTN_BWD_NOALLOC_MAX_ROWS floats (16 MiB), reserved when the library's code is
 * loaded on that GPU and held until the process ends.  The call itself
 * allocates nothing; its first call on a device looks up that device's array
 * address once.
 *
 * Arguments, layout, ownership and status codes as for attn_bwd (without
 * delta), plus ATTN_ERR_SHAPE when B*H*N exceeds ATTN_BWD_NOALLOC_MAX_ROWS and
 * ATTN_ERR_DEVICE when the array's address cannot be obtained.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from threads without ordering) race; order them on one stream.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                     float scale, int dtype, void* stream);

/*
 * attn_lse_merge -- combine G partial results over disjoint key shards.
 *
 *   o_parts   : device pointer, contiguous [G, R, d] of dtype (R = B*H*N rows).
 *   lse_parts : device pointer, contiguous [G, R] fp32; -inf marks a shard with
 *               no key for that row.
 *   o, lse    : device pointers, contiguous [R, d] of dtype and [R] fp32: the
 *               merged result (fp32 arithmetic, o rounded to nearest even).  A
 *               row whose every lse_g is -inf gets lse = -inf and o = 0.
 *   G >= 1, R >= 1, d in {64, 80, 128}.
 *
 * Alignment: o_parts and o 16-byte aligned, lse_parts and lse 4-byte aligned.
 * o and lse must not overlap the parts or each other.  Returns ATTN_OK or
 * ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_HEAD_DIM, ATTN_ERR_DTYPE,
 * ATTN_ERR_ALIGN, ATTN_ERR_ALIAS, ATTN_ERR_DEVICE, ATTN_ERR_LAUNCH.
 */
int attn_lse_merge(const void* o_parts, const void* lse_parts, int G, void* o, void* lse, long long R, int d,
                   int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ETA_ATTN_BWD_H */
