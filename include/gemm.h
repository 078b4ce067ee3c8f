/*
 * gemm.h -- C ABI of the tiled matrix product with a fused bias + activation
 * epilogue (MI355X, gfx950).
 *
 * The operation is the blocked matrix product of "Triton: CUDA-level
 * operators in Python" (f.mffb.com.cn), example 3, and "CS336 Lecture 6"
 * (xwysyy.cn), section "Level 3": each work-group computes one tile of C,
 * accumulating in fp32 along K, and applies the element-wise epilogue to the
 * finished tile before its single store (the lecture's "linear layer = matmul
 * + activation"); the bias is the fused bias + ReLU of "Triton core syntax"
 * (5688vip.com), section 4.4:
 *
 *     C[m, n] = act( sum_k A[m, k] * B[k, n] + bias[n] )
 *
 * with the sum in fp32, bias added in fp32, act in fp32, and one rounding to
 * the 16-bit output type (nearest even) at the store.
 *
 * Status codes and element types are those of attn.h.
 */
#ifndef ETA_GEMM_H
#define ETA_GEMM_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Epilogue nonlinearity. */
typedef enum {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1,      /* max(z, 0) */
    GEMM_ACT_GELU_TANH = 2  /* 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) */
} gemm_act;

/* Storage of the K x N operand B. */
typedef enum {
    GEMM_B_KN = 0,  /* B[k, n] at b[k * ldb + n]: rows of N contiguous (the pages' matmul) */
    GEMM_B_NK = 1   /* B[k, n] at b[n * ldb + k]: a linear layer's weight W[n, k], y = x W^T */
} gemm_b_layout;

/*
 * gemm_bias_act -- C = act(A B + bias) on the current HIP device.
 *
 *   a        : device pointer, A[m, k] at a[m * lda + k] (row-major, K contiguous).
 *   lda      : elements between rows of A, >= K.
 *   b        : device pointer, B as b_layout says; ldb >= N (GEMM_B_KN) or >= K (GEMM_B_NK).
 *   bias     : device pointer to N elements of dtype, or NULL for none.
 *   c        : device pointer, C[m, n] at c[m * ldc + n]; only those M x N elements are written.
 *   ldc      : elements between rows of C, >= N.
 *   M, N, K  : M, N >= 1; K >= 0 and a multiple of 8 (K = 0 gives C = act(bias)).
 *   act      : a gemm_act value.
 *   dtype    : ATTN_F16 or ATTN_BF16, shared by a, b, bias and c.
 *   stream   : a hipStream_t cast to void*, or NULL; the call only enqueues work.
 *
 * Layout: a and b 16-byte aligned and lda, ldb multiples of 8 (16-byte rows);
 * bias and c 2-byte aligned (C is stored 8 bytes at a time where c and ldc
 * allow, else element by element).  Limits: 256 rows of A (or of B in
 * GEMM_B_NK) must span less than 2^31 bytes; in GEMM_B_KN, 64 rows of B must.
 *
 * Ownership: the caller owns every buffer; all must live on the current device
 * and stay valid until the work on `stream` completes.  c must not overlap a,
 * b or bias.  The library allocates nothing and keeps no reference after the
 * call returns.
 *
 * Returns ATTN_OK or an attn_status code, checked on the host before any device
 * work: ATTN_ERR_NULL (a, b or c NULL; a or b may be NULL only when K == 0),
 * ATTN_ERR_SHAPE (M or N < 1, K < 0 or not a multiple of 8, a leading dimension
 * too small or past the limits above), ATTN_ERR_DTYPE, ATTN_ERR_ALIGN,
 * ATTN_ERR_ALIAS (c overlaps an input), ATTN_ERR_LAYOUT (b_layout or act not a
 * listed value), ATTN_ERR_DEVICE (the current device is not a gfx950),
 * ATTN_ERR_LAUNCH.  An error leaves c untouched.
 */
int gemm_bias_act(const void* a, long long lda, const void* b, long long ldb, int b_layout, const void* bias, void* c,
                  long long ldc, int M, int N, int K, int act, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ETA_GEMM_H */
