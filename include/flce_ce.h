/*
 * flce_ce.h -- cross-entropy over materialised logits, forward and backward, for AMD
 * Instinct MI355X (gfx950).  C ABI of libflce.so (with flce.h).
 *
 * The operation, for logits Z[N][V] (row pitch ld elements) and labels y[N]:
 *
 *   lse[n]   = log sum_v exp(Z[n, v])
 *   loss     = (1 / N_valid) * sum_{n valid} (lse[n] - Z[n, y[n]])
 *   dZ[n, v] = (exp(Z[n, v] - lse[n]) - [v == y[n]]) * g / N_valid   (valid rows; else 0)
 *
 * "Unsloth Kernel Architecture: Custom Triton Backpropagation and QLoRA Memory Scaling",
 * section 1 "Fused Cross-Entropy Loss with Logit Streaming": one program per row streams
 * the vocabulary in blocks, keeping a running maximum and a running sum of exponentials,
 * and the row loss is the log-sum-exp minus the label's logit.  This is that kernel for
 * logits that already exist in HBM (the unfused case the fused path avoids): it reads
 * every logit once in the forward and reads and writes every logit once in the backward,
 * so its bound is HBM bandwidth.  Rows, N_valid and ignore_index as in flce.h.
 *
 * Conventions: device pointers on the current HIP device; Z and dZ row-major with row
 * pitches ld and ld_out elements (>= V); dtype FLCE_F32, FLCE_BF16 or FLCE_F16 for Z and
 * dZ (loss, lse fp32).  Z and dZ must be 16-byte aligned with ld, ld_out multiples of
 * 16 bytes' worth of elements (4 fp32 or 8 16-bit); a row of Z may be read up to the next
 * 4-byte boundary past column V - 1 (inside its pitch), never past it, and the bytes past
 * column V - 1 do not affect any result.  Calls are asynchronous on `stream`;
 * results are deterministic (fixed reduction orders).  Size limits: 1 <= N <= 2^31 - 1,
 * 1 <= V and ld * element size < 2^31 bytes per row.
 */
#ifndef FLCE_CE_H
#define FLCE_CE_H

#include <stddef.h>
#include <stdint.h>

#include "flce.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes flce_ce_forward needs: 16 * N for per-row loss terms and flags plus
 * 16 per 256 rows for block sums, each region rounded up to 256 bytes.  0 for N < 1. */
size_t flce_ce_workspace_bytes(int64_t N);

/*
 * Forward: loss, lse[N], n_valid and dev_status (1 when a label is neither ignore_index
 * nor in [0, V); such rows count as ignored), as flce_forward.
 * Errors (synchronous, nothing launched): FLCE_ERR_INVALID_ARG (null pointer, size,
 * dtype, ld < V), FLCE_ERR_ALIGN, FLCE_ERR_WORKSPACE; FLCE_ERR_HIP if a launch failed.
 */
flce_status flce_ce_forward(const void* Z, int64_t ld, const int64_t* y, int64_t N, int64_t V, int dtype,
                            int64_t ignore_index, float* loss, float* lse, int32_t* n_valid,
                            int32_t* dev_status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward: dZ from Z, y and the forward's lse and n_valid; grad_loss is a device pointer
 * to g (NULL means 1).  dZ may be Z itself (ld_out == ld): each element is read before it
 * is overwritten by the same thread.  Columns v >= V of dZ are not touched.
 * Errors as for flce_ce_forward (no workspace).
 */
flce_status flce_ce_backward(const void* Z, int64_t ld, const int64_t* y, const float* lse,
                             const int32_t* n_valid, const float* grad_loss, int64_t N, int64_t V, int dtype,
                             int64_t ignore_index, void* dZ, int64_t ld_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_CE_H */
