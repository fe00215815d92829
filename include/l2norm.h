/*
 * l2norm.h -- C ABI of the row-wise L2 norm in libattn_mi355x.so, the second
 * workload of the repair algebra the attention kernels use.
 *
 * For each row x of H elements:
 *     norm = sqrt(sum_j x_j^2),     y_j = x_j / norm      (y = 0 for a zero row).
 *
 * The "Neptune论文浅读" notes (gentlecold.top), section 4, list the numerically
 * stable L2 norm among the reductions that their repair algebra fuses, and
 * section 9 reports it among the non-attention operators that gain from it.
 * The stable form carries, instead of the attention's running max m and sum
 * l, a reference exponent e and the sum s of squares scaled by 2^-e:
 *     s = sum_j (x_j * 2^-e)^2,     norm = 2^e * sqrt(s),
 * and when the reference moves from e to e' the partial sum is repaired by
 *     h(s, e, e') = s * 4^(e - e')
 * (the analogue of the softmax's t * exp(r - r') in section 4 of those notes).
 * Scaling by powers of two is exact, so no square overflows or underflows in
 * fp32 whatever the magnitude of the (finite) inputs, and the result is as
 * accurate as the plain sum.  Two forms, as for the attention:
 *   - one pass (the rolling update, section 5 of the notes): a row that fits in
 *     one wave's registers is read once, reduced, and written scaled;
 *   - split-K (section 6): the row is cut into num_splits chunks, each chunk
 *     yields a partial (e_c, s_c) in the workspace, and a second kernel merges
 *     a row's partials with the repair and scales its chunk (the row is read
 *     twice).
 *
 * Conventions: x is [rows, H] with rows x_stride elements apart, element type
 * ATTN_BF16 or ATTN_F32; y (same shape, y_stride, element type y_dtype) may be
 * NULL when only the norms are wanted; norm is a [rows] fp32 array or NULL.
 * All pointers are device pointers owned by the caller.  x is read in 16-byte
 * vectors (16-byte aligned base, H and x_stride multiples of 16 bytes' worth of
 * elements); each vector's output is stored in one piece of up to 16 bytes (8
 * bytes for fp32 -> bf16), whose size y and y_stride must keep aligned.
 * Otherwise ATTN_ERR_UNSUPPORTED.  Inputs
 * must be finite.  Errors are reported as for the attention entry points
 * (validation before any launch; ATTN_ERR_HIP for a launch failure).
 */
#ifndef L2NORM_MI355X_H
#define L2NORM_MI355X_H

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct l2norm_args {
    int64_t rows, H;                 /* number of rows, elements per row */
    int32_t x_dtype;                 /* ATTN_F32 or ATTN_BF16 */
    int32_t y_dtype;                 /* ATTN_F32 or ATTN_BF16 (ignored when y == NULL) */
    const void *x;                   /* device, row r at x + r * x_stride elements */
    int64_t x_stride;
    void *y;                         /* device or NULL */
    int64_t y_stride;
    float *norm;                     /* device [rows] fp32, or NULL */
} l2norm_args;

/*
 * l2norm_rows -- norms and scaled rows.  num_splits = 1 runs the one-pass
 * kernel (rows of up to l2norm_max_onepass(x_dtype) elements, no workspace);
 * num_splits >= 2 runs the split-K path with 8 * rows * num_splits bytes of
 * device workspace (l2norm_workspace_bytes; 16-byte aligned, contents on entry
 * irrelevant).  A too small workspace returns ATTN_ERR_WORKSPACE.
 */
attn_status l2norm_rows(const l2norm_args *a, int32_t num_splits, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * l2norm_choose_splits -- 1 (one pass) when a row fits the one-pass kernel,
 * else the smallest split count that gives cu_count compute units four
 * workgroups each, with at least 4096 bytes of the row per chunk (pure host
 * function).
 */
int32_t l2norm_choose_splits(int64_t rows, int64_t H, int32_t x_dtype, int32_t cu_count);

/* l2norm_max_onepass -- the longest row the one-pass kernel takes. */
int64_t l2norm_max_onepass(int32_t x_dtype);

/* l2norm_workspace_bytes -- workspace of the split-K path (0 for num_splits <= 1). */
size_t l2norm_workspace_bytes(int64_t rows, int32_t num_splits);

/* l2norm_validate -- the host-side check l2norm_rows runs (pure host function). */
attn_status l2norm_validate(const l2norm_args *a, int32_t num_splits);

/* l2norm_args_size -- sizeof(l2norm_args). */
size_t l2norm_args_size(void);

#ifdef __cplusplus
}
#endif

#endif /* L2NORM_MI355X_H */
