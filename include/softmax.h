/*
 * softmax.h -- C ABI of the standalone fused row softmax (MI355X, gfx950).
 *
 * The operation is the fused softmax of "Triton: CUDA-level operators in
 * Python" (f.mffb.com.cn), example 2, and "CS336 Lecture 6: GPU kernels &
 * Triton" (xwysyy.cn), section "Level 1: Softmax": every row independently,
 *
 *     y[i, j] = exp(x[i, j] - max_j x[i, j]) / sum_j exp(x[i, j] - max_j x[i, j])
 *
 * with the row read from HBM once and written once (the pages contrast this
 * with the five reads and three writes of the unfused sequence).  Rows longer
 * than one work-group holds in registers (65536 elements) are processed in
 * tiles (the lecture's "Level 2" tiled row reduction) with a running max and
 * sum, which costs one extra read of the row.
 *
 * Status codes and element types are those of attn.h.
 */
#ifndef ETA_SOFTMAX_H
#define ETA_SOFTMAX_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * softmax_rows -- row softmax on the current HIP device.
 *
 *   x        : device pointer, rows of `cols` elements of `dtype`; row i starts
 *              at element i * x_stride.  Read only (but see in-place below).
 *   x_stride : elements between row starts of x, >= cols.
 *   y        : device pointer, the same shape with row stride y_stride; every
 *              element of each row's first `cols` is written, nothing else.
 *   rows, cols : >= 1 each.
 *   dtype    : ATTN_F16, ATTN_BF16 or ATTN_F32; x and y share it.  Arithmetic is
 *              fp32; a 16-bit y is rounded to nearest even.
 *   stream   : a hipStream_t cast to void*, or NULL; the call only enqueues work.
 *
 * Layout: row-major rows, elements of a row contiguous.  x and y must be
 * aligned to the element size.  When every row start of both is 16-byte
 * aligned (pointers, and stride * element size unless rows == 1, multiples of
 * 16) the kernels move 16-byte vectors; otherwise one element per lane
 * (correct, slower).
 *
 * Ownership: the caller owns both buffers; they must live on the current device
 * and stay valid until the work on `stream` completes.  y may be x itself (with
 * y_stride == x_stride: in place); otherwise the byte spans of x and y (first
 * row start to last row end) must not overlap.  The library allocates nothing
 * and keeps no reference after the call returns.
 *
 * Special values follow IEEE arithmetic on the definition: -inf entries give 0;
 * a row whose entries are all -inf, or that holds +inf or NaN, gives NaN
 * throughout.
 *
 * Returns ATTN_OK or an attn_status code, checked on the host before any device
 * work: ATTN_ERR_NULL (x or y NULL), ATTN_ERR_SHAPE (rows or cols < 1, a stride
 * below cols, or a buffer spanning more than 2^48 bytes), ATTN_ERR_DTYPE,
 * ATTN_ERR_ALIGN (x or y not aligned to the element size), ATTN_ERR_ALIAS
 * (x and y overlap other than exactly in place),
 * ATTN_ERR_DEVICE (the current device is not a gfx950), ATTN_ERR_LAUNCH.  An
 * error leaves y untouched.  Faults during the kernel surface at the caller's
 * next synchronisation of `stream`, as for any HIP work.
 */
int softmax_rows(const void* x, long long x_stride, void* y, long long y_stride, int rows, int cols, int dtype,
                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ETA_SOFTMAX_H */
