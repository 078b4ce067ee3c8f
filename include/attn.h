/*
 * attn.h -- C ABI of the fused exact-attention forward library (MI355X, gfx950).
 *
 * The operation is the exact attention forward pass
 *
 *     O = softmax(scale * Q K^T  [+ causal mask]) V,   lse = ln sum_j exp(scale * q_i . k_j)
 *
 * as defined by "Triton in depth: from matmul to Flash Attention" (ybb.press),
 * section 3.1 (the standard attention it replaces), computed the way its
 * section 3.2 describes (Q, K and V split into tiles, running row statistics
 * m and l, O(N) extra memory, exact result) and its section 3.3 kernel shows
 * (one work unit per query tile and head, a loop over key/value tiles, the
 * causal rule "key index <= query index", rescaling of the accumulator when
 * the running max grows, one division by l after the loop).  The logsumexp
 * output is an addition of this library; it is what a later merge of
 * key-sharded partial results needs.
 *
 * Every function is plain C: pointers, integers and a float.  No allocation,
 * no synchronisation and no global state beyond a per-device architecture
 * cache happen inside the library.
 */
#ifndef ETA_ATTN_H
#define ETA_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out (and of softmax_rows' x and y). */
typedef enum {
    ATTN_F16 = 0,  /* IEEE binary16 */
    ATTN_BF16 = 1, /* bfloat16 */
    ATTN_F32 = 2   /* IEEE binary32: softmax_rows only; attn_fwd rejects it */
} attn_dtype;

/* Return codes.  On any code other than ATTN_OK nothing has been written and
 * nothing has been launched, except ATTN_ERR_LAUNCH (the launch itself failed).
 * The notes give attn_fwd's causes; softmax.h and gemm.h state those of
 * softmax_rows and gemm_bias_act. */
typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,      /* q, k, v or out is NULL */
    ATTN_ERR_SHAPE = 2,     /* B, H or N < 1, the grid would exceed 2^31-1 work-groups, or N*d*2 > 2^31-1 bytes */
    ATTN_ERR_HEAD_DIM = 3,  /* d is not one of 64, 80, 128 */
    ATTN_ERR_DTYPE = 4,     /* dtype is not an attn_dtype value */
    ATTN_ERR_SCALE = 5,     /* scale is NaN or infinite */
    ATTN_ERR_ALIGN = 6,     /* q, k, v or out not 16-byte aligned, or lse not 4-byte aligned */
    ATTN_ERR_DEVICE = 7,    /* no current HIP device, or it is not a gfx950 */
    ATTN_ERR_LAUNCH = 8,    /* the kernel launch returned an error */
    ATTN_ERR_CAUSAL = 9,    /* causal is neither 0 nor 1 */
    ATTN_ERR_ALIAS = 10,    /* out or lse overlaps q, k, v, or each other */
    ATTN_ERR_WINDOW = 11,   /* window is negative */
    ATTN_ERR_LAYOUT = 12,   /* gemm_bias_act: b_layout or act is not a listed value */
    ATTN_ERR_WORKSPACE = 13 /* attn_fwd_ws: workspace smaller than attn_fwd_workspace_bytes */
} attn_status;

/*
 * attn_fwd -- fused exact-attention forward on the current HIP device.
 *
 *   q, k, v : device pointers, contiguous row-major [B, H, N, d] of `dtype`
 *             (element (b,h,i,c) at offset ((b*H + h)*N + i)*d + c).  Read only.
 *             Elements are finite numbers; a row whose scores meet a NaN or an
 *             infinite element gets unspecified out and lse values (the kernels
 *             assume no NaN arises when they form the running row max).
 *   out     : device pointer, contiguous [B, H, N, d] of `dtype`.  Every element
 *             is written: out[b,h,i,:] = sum_j softmax_j(scale * q_i . k_j) v_j,
 *             rounded to nearest even from an fp32 accumulator.
 *   lse     : device pointer to contiguous [B, H, N] float32, or NULL to skip it.
 *             lse[b,h,i] = ln sum_{j allowed} exp(scale * q_i . k_j), natural log.
 *   B, H, N : batch, heads, sequence length (queries = keys = N), each >= 1.
 *   d       : head dimension, one of 64, 80, 128.
 *   causal  : 1 keeps key j for query i iff j <= i (top-left aligned, diagonal
 *             kept); 0 keeps every key.
 *   scale   : score scale, any finite float (usually 1/sqrt(d)); applied in fp32
 *             to the fp32 dot products (inputs are never pre-scaled in 16 bit).
 *   dtype   : attn_dtype of q, k, v and out.
 *   stream  : a hipStream_t cast to void*, or NULL for the null stream.  The call
 *             only enqueues work on it and returns without waiting; the caller
 *             synchronises before reading out or lse.  Faults during execution
 *             surface at that synchronisation, not here.
 *
 * Ownership: the caller owns every buffer; all must live on the current device
 * and stay valid until the work on `stream` completes.  out and lse must not
 * overlap the inputs or each other.  The library allocates nothing and keeps
 * no reference after the call returns.
 *
 * Arithmetic: fp16/bf16 products with fp32 accumulation for both Q K^T and P V;
 * probabilities are rounded to `dtype` before P V.  Results are deterministic
 * run to run (no atomics).
 *
 * Returns ATTN_OK or an attn_status error code; argument checks run on the
 * host before any device work, so an error leaves out and lse untouched.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int N, int d, int causal, float scale, int dtype,
             void* stream);

/*
 * attn_fwd_window -- attn_fwd restricted to a sliding window (local band).
 *
 * "Triton: CUDA-level operators in Python" (f.mffb.com.cn), section "when to
 * use Triton", names sliding-window attention as one of the attention variants
 * a tiled kernel serves, without defining it; the reading implemented is the
 * usual local band.  With window = W >= 1, key j is kept for query i only if
 *
 *     i - W < j                  (the W most recent keys, the diagonal included)
 *     j < i + W                  (causal = 0 only: the symmetric band |i - j| < W)
 *
 * on top of the causal rule when causal = 1.  window = 0 (or W >= N, which keeps
 * every key) gives exactly attn_fwd.  lse is over the kept keys.  Tiles wholly
 * outside every row's band are never loaded or computed: the work is
 * proportional to N * min(N, W) instead of N^2.
 *
 * Arguments, layout, ownership, arithmetic and errors as attn_fwd; in addition
 * ATTN_ERR_WINDOW when window < 0.
 */
int attn_fwd_window(const void* q, const void* k, const void* v, void* out, float* lse,
                    int B, int H, int N, int d, int causal, int window, float scale, int dtype,
                    void* stream);

/*
 * attn_fwd_ws -- attn_fwd with a caller workspace, used to fill the GPU when
 * the query tiles leave an incomplete last round.
 *
 * Query tile i and head h are one unit of work in the method of "Triton in
 * depth" section 3.3; on a GPU that runs S work-groups at a time, a last round
 * of r < S units keeps the other S - r compute units idle for a whole unit's
 * time.  For causal = 0, when 0 < r <= S/2 for the 256-query tiles, the last r
 * tiles are instead each cut into P = min(S / r, key tiles / 2) key ranges
 * (64 keys per key tile) that run in one short round, and every row of those
 * tiles is combined from its P partial results exactly as attn_lse_merge
 * (attn_bwd.h) documents: each partial is computed like attn_fwd over its key
 * range, its O rounded to `dtype`.  Rows of the cut tiles therefore differ
 * from attn_fwd's by that extra rounding of the partial O (the merge weights
 * sum to 1, so at most one rounding of the row's weighted |V|).  The other
 * rows run the 8-wave schedule: bitwise equal to attn_fwd where it uses that
 * schedule too (attn_fwd_schedule returns ATTN_SCHEDULE_WIDE), else equal up
 * to floating-point summation order.
 *
 *   workspace       : device pointer, 256-byte aligned, or NULL.  NULL, or a
 *                     shape that needs no split (attn_fwd_workspace_bytes returns
 *                     0), gives exactly attn_fwd.  Its contents on entry do not
 *                     matter; on return they are unspecified.
 *   workspace_bytes : its size; at least attn_fwd_workspace_bytes(B, H, N, d,
 *                     causal) when workspace is not NULL.
 *
 * Other arguments, layout, arithmetic and the remaining errors as attn_fwd (no
 * window).  Two kernels are enqueued on `stream` (the forward, then the merge).
 * Errors: ATTN_ERR_WORKSPACE when workspace is not NULL, a split is used and
 * workspace_bytes is too small; ATTN_ERR_ALIGN when workspace is not 256-byte
 * aligned; ATTN_ERR_ALIAS when it overlaps q, k, v, out or lse.  The caller owns
 * the workspace; calls that may run at the same time need workspaces of their own.
 */
int attn_fwd_ws(const void* q, const void* k, const void* v, void* out, float* lse,
                int B, int H, int N, int d, int causal, float scale, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_fwd_workspace_bytes -- workspace attn_fwd_ws uses for a shape on the
 * current device (its compute-unit count sets S): 0 when it would not split,
 * else P x rows x (2 d + 4) + rows x 4 bytes (rows = those of the cut tiles),
 * each area rounded up to 256 bytes.  A negative attn_status for arguments
 * attn_fwd would reject by shape, or -ATTN_ERR_DEVICE.
 */
long long attn_fwd_workspace_bytes(int B, int H, int N, int d, int causal);

/*
 * attn_fwd_schedule -- which kernel schedule attn_fwd uses for a shape
 * (attn_fwd_window makes the same choice, except that it never uses
 * ATTN_SCHEDULE_SPLIT).
 *
 * Returns ATTN_SCHEDULE_SMALL (4 waves, 128 queries per work-group, two
 * work-groups per CU; causal query tiles in pairs (i, T-1-i) per work-group,
 * or one per work-group, longest first, when all of them fit one round of two
 * per CU; with a window one tile per work-group), ATTN_SCHEDULE_WIDE (8 waves, 256 queries per work-group, one per
 * CU), ATTN_SCHEDULE_SPLIT (d = 64 and N >= 2048 where the small schedule
 * would give fewer than 512 work-groups, except causal problems below 4096
 * keys whose tiles fit the unpaired round: 8 waves, 128 queries per
 * work-group, one per CU; the two waves that hold the same 32 rows each take
 * one half of the query tile's key tiles and their partial results are merged
 * at the end), or a negative
 * attn_status for arguments attn_fwd would reject by shape (ATTN_ERR_SHAPE,
 * ATTN_ERR_HEAD_DIM, ATTN_ERR_CAUSAL).  Pure host function: no device is
 * touched.  The choice depends on B*H, N, d and causal only; results do not
 * depend on it beyond floating-point rounding order.
 */
typedef enum { ATTN_SCHEDULE_SMALL = 0, ATTN_SCHEDULE_WIDE = 1, ATTN_SCHEDULE_SPLIT = 2 } attn_schedule;
int attn_fwd_schedule(int B, int H, int N, int d, int causal);

/* Static, NUL-terminated English description of a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ETA_ATTN_H */
