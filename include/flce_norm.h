/*
 * flce_norm.h -- RMSNorm forward and fused backward for the hidden states fed to the
 * lm_head, on AMD Instinct MI355X (gfx950).  C ABI of libflce.so (with flce.h).
 *
 * For X[N][D] and a per-channel weight gamma[D]:
 *
 *   rstd[n]   = 1 / sqrt(mean_d X[n, d]^2 + eps)
 *   H[n, d]   = X[n, d] * rstd[n] * gamma[d]
 *   dX[n, d]  = rstd[n] * gamma[d] * dH[n, d] - X[n, d] * rstd[n]^3 * s[n] / D,
 *               s[n] = sum_i gamma[i] * X[n, i] * dH[n, i]
 *   dgamma[d] = sum_n dH[n, d] * X[n, d] * rstd[n]
 *
 * "Unsloth Kernel Architecture: Custom Triton Backpropagation and QLoRA Memory Scaling",
 * section 3 "Fused RMSNorm & SwiGLU Kernels": RMSNorm of a row, and its closed-form
 * gradient computed in one pass per row.  The page writes that gradient with gamma outside
 * the bracket, which is exact only when gamma is uniform; dX above is the chain-rule form
 * for a per-channel gamma and reduces to it in that case.  The backward's dH is the
 * hidden-state gradient of flce_backward (it feeds the norm that produced H).
 *
 * Conventions: device pointers on the current HIP device; X, gamma, H, dH, dX row-major
 * contiguous in dtype FLCE_F32, FLCE_BF16 or FLCE_F16 (all the same); rstd and dgamma fp32.
 * Pointers 16-byte aligned (rstd, dgamma 4-byte) and D a multiple of 16 bytes' worth of
 * elements (8 16-bit or 4 fp32); D <= 16384.
 * All math in fp32, outputs rounded to nearest even.  Calls are asynchronous on `stream`
 * and deterministic (fixed reduction orders; no atomics).  A row of zeros with eps = 0
 * gives rstd = inf and NaN outputs, as the formula does.
 */
#ifndef FLCE_NORM_H
#define FLCE_NORM_H

#include <stddef.h>
#include <stdint.h>

#include "flce.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes flce_rmsnorm_backward needs for the dgamma partials: an fp32 row of D per
 * backward workgroup (min(N, 512) of them) plus one per 32 of those, each region rounded
 * up to 256 bytes.  0 for N < 1 or D outside [1, 16384]. */
size_t flce_rmsnorm_workspace_bytes(int64_t N, int64_t D);

/*
 * Forward: H and rstd (saved for the backward).  eps >= 0.
 * Errors (synchronous, nothing launched): FLCE_ERR_INVALID_ARG (null pointer, N or D out of
 * range, dtype, eps < 0 or NaN), FLCE_ERR_ALIGN; FLCE_ERR_HIP if a launch failed.
 */
flce_status flce_rmsnorm_forward(const void* X, const void* gamma, int64_t N, int64_t D, int dtype, float eps,
                                 void* H, float* rstd, void* stream);

/*
 * Backward: dX (dtype) and dgamma (fp32, overwritten) from X, gamma, the forward's rstd and
 * the output gradient dH.  dX must not alias X or dH.
 * Errors as for the forward, plus FLCE_ERR_WORKSPACE.
 */
flce_status flce_rmsnorm_backward(const void* X, const void* gamma, const float* rstd, const void* dH, int64_t N,
                                  int64_t D, int dtype, void* dX, float* dgamma, void* workspace,
                                  size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_NORM_H */
