// status.cpp -- text of the status codes shared by every entry point of the
// library (attn.h, softmax.h, gemm.h).
#include "attn.h"

extern "C" const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL:
            return "a required pointer is NULL (attn_fwd: q, k, v, out; softmax_rows: x, y; gemm_bias_act: a, b, c)";
        case ATTN_ERR_SHAPE:
            return "a size is out of range (attn_fwd: B, H, N >= 1, grid within 2^31-1 work-groups, one head within "
                   "2 GB; softmax_rows: rows, cols >= 1, strides >= cols; gemm_bias_act: M, N >= 1, K >= 0 and a "
                   "multiple of 8, leading dimensions large enough and within the stated spans)";
        case ATTN_ERR_HEAD_DIM: return "head dim must be 64, 80 or 128";
        case ATTN_ERR_DTYPE: return "dtype is not accepted by this entry point (attn_fwd and gemm_bias_act: ATTN_F16 "
                                    "or ATTN_BF16; softmax_rows: also ATTN_F32)";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_ALIGN:
            return "a buffer or leading dimension is misaligned (attn_fwd: 16-byte q, k, v, out and 4-byte lse; "
                   "softmax_rows: element-aligned x, y; gemm_bias_act: 16-byte a, b and lda, ldb multiples of 8, "
                   "2-byte bias, c)";
        case ATTN_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        case ATTN_ERR_CAUSAL: return "causal must be 0 or 1";
        case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
        case ATTN_ERR_WINDOW: return "window must be >= 0";
        case ATTN_ERR_LAYOUT: return "b_layout or act is not a listed value";
        case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_fwd_workspace_bytes for this shape";
        default: return "unknown status";
    }
}
