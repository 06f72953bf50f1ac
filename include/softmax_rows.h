/*
 * softmax_rows.h -- row softmax on MI355X (gfx950): the fused kernel and the
 * unfused four-pass baseline, as a C ABI.
 *
 * y[r][j] = exp(x[r][j] - m_r) / sum_k exp(x[r][k] - m_r),  m_r = max_k x[r][k]
 *
 * the numerically stable softmax of every row (page "Kernel Fusion and the Memory
 * Wall", section "Softmax needs a global row statistic"; the denominator covers the
 * whole row).  Entries equal to -inf are masked: their output is 0.  A row whose
 * entries are all -inf has no valid entry and its output is all zeros (the same
 * convention attn_fwd uses for a query without a valid key).
 *
 * x and y: float32, rows x cols, row-major and contiguous (row r starts at
 * r * cols), device pointers, 4-byte aligned; y may equal x (in place).  Every call
 * is stream-ordered and returns before the work completes; status codes are those
 * of attn.h.  Arguments are checked on the host before anything is launched: an
 * error status means nothing ran and nothing was written.
 */
#ifndef SOFTMAX_ROWS_H
#define SOFTMAX_ROWS_H

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * softmax_rows_f32 -- the fused kernel: one launch.  A row of up to 16384 entries
 * is read once and written once (it stays in registers between its maximum, its
 * exponentials, its sum and the division); a longer row is read twice (an online
 * pass for the maximum and the sum, then the pass that writes y) and written once
 * (page "Kernel Fusion and the Memory Wall", same section: rows too large for the
 * chip need tiling or additional passes).
 *
 * rows, cols >= 1 (ATTN_ERR_SHAPE otherwise; rows * cols * 4 must fit in 64 bits,
 * cols * 4 in 31 bits: ATTN_ERR_TOO_LARGE).  ATTN_ERR_NULL for a NULL pointer,
 * ATTN_ERR_ALIGN for a pointer that is not 4-byte aligned.
 */
int softmax_rows_f32(const float* x, float* y, int rows, int cols, void* stream);

/*
 * softmax_rows_unfused_workspace_bytes -- device workspace softmax_rows_unfused_f32
 * needs: the row maxima and the row sums, 2 * rows float32 (plus padding).  0 when
 * rows < 1.
 */
size_t softmax_rows_unfused_workspace_bytes(int rows);

/*
 * softmax_rows_unfused_f32 -- the unfused baseline, four launches in the order the
 * page lists them: (1) read x for the row maxima; (2) read x again and write the
 * exponentials exp(x - m) to y; (3) read y for the row sums; (4) read y again and
 * write y / sum.  Four reads and two writes of every row.  `workspace` is a
 * caller-owned device buffer of at least softmax_rows_unfused_workspace_bytes(rows)
 * bytes, 256-byte aligned (ATTN_ERR_WORKSPACE otherwise); its contents on return are
 * unspecified.  Same results as softmax_rows_f32 up to rounding.
 */
int softmax_rows_unfused_f32(const float* x, float* y, int rows, int cols, void* workspace,
                             size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SOFTMAX_ROWS_H */
