/*
 * flce.h -- fused lm_head projection + cross-entropy loss, forward and backward,
 * for AMD Instinct MI355X (gfx950).  C ABI of libflce.so.
 *
 * The operation (for N token rows, hidden size D, vocabulary V):
 *
 *   z[n, v]   = sum_d H[n, d] * W[v, d]                 logits, never stored
 *   lse[n]    = log sum_v exp(z[n, v])                  per-row log-sum-exp
 *   loss      = (1 / N_valid) * sum_{n valid} (lse[n] - z[n, y[n]])
 *   dz[n, v]  = (exp(z[n, v] - lse[n]) - [v == y[n]]) * g / N_valid   (valid rows; else 0)
 *   dH        = dz W,    dW = dz^T H
 *
 * The lm_head projection and the loss follow "Arquitectura interna de Unsloth y
 * optimización en Triton", section 3 (Fused Cross Entropy: the projection Z = X W_vocab^T,
 * the max-subtracted log-sum-exp, the analytic gradient softmax - onehot, and
 * backpropagation into both X and W_vocab without writing the logit matrix), and
 * "Unsloth Architecture: 5x Faster LLM Training via Triton", pillar 1 "Fused Chunked
 * Cross-Entropy Loss" (the per-row loss -z_y + log sum exp z, its gradient p - onehot,
 * and the online log-sum-exp over chunks) with its numpy walk-through (mean over
 * tokens).  A row is valid when its label is not ignore_index; N_valid counts valid rows.
 * g is the upstream gradient of the loss (1 when grad_loss is NULL).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers on the current HIP device, row-major and
 *    contiguous: H[N][D], W[V][D] (the nn.Linear weight layout), y[N] int64, lse[N]
 *    fp32, dH[N][D] in the input element type, dW[V][D] fp32.
 *  - dtype FLCE_BF16: H, W, dH are bf16 (raw 16-bit patterns); products accumulate in
 *    fp32; loss, lse and dW are fp32.  dtype FLCE_F16: the same with IEEE fp16 for H, W
 *    and dH (the pages name fp16 next to bf16 as a 16-bit training format).  dtype
 *    FLCE_F32: everything is fp32.  The logit gradient dz is rounded to the input type
 *    before the two backward contractions; for fp16, whose range cannot hold dz itself
 *    (about g / N_valid / V), it is held as dz * 2^14 * N_valid / |g| and the factor is
 *    divided out in fp32 after each contraction.  The fp16 dH output itself is about
 *    |g| |W| / N_valid per entry: with g = 1 and thousands of valid rows it falls below
 *    fp16's smallest normal (6.1e-5), where the spacing of subnormals (6e-8) is a visible
 *    fraction of the value, so fp16 callers scale the loss (g of 2^10 or more at N_valid
 *    ~ 10^4), as fp16 training does, and divide the gradients by it.
 *  - The caller owns and allocates every buffer, including the workspace (device
 *    scratch).  The library allocates nothing, frees nothing and keeps no state between
 *    calls, so its peak scratch memory is exactly workspace_bytes.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 *    The return value reports only argument and launch errors.  Two calls may run
 *    concurrently only with distinct workspaces and outputs.
 *  - A call issues kernel launches only (no allocation, memset, copy or synchronisation),
 *    so it may be captured into a HIP graph and replayed; flce_forward_backward_static
 *    looks up its array's device address on its first call on a device, so make one call
 *    outside the capture first.
 *  - Results are deterministic: fixed tile shapes and fixed reduction orders, no
 *    floating-point atomics; a repeated call with the same inputs and the same
 *    workspace_bytes produces bitwise-identical outputs.
 *  - Size limits: 1 <= N, V <= 2^31 - 512, 1 <= D <= 65536; D must be a multiple of
 *    8 (bf16, fp16) or 4 (fp32); H, W, dH, dW and workspace must be 16-byte aligned.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flce_status {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = 1, /* null pointer, size < 1 or too large, unknown dtype */
  FLCE_ERR_ALIGN = 2,       /* misaligned pointer, or D (flce_*) or a row pitch (flce_ce_*) not a
                               multiple of 8 elements (bf16, fp16) / 4 (fp32) */
  FLCE_ERR_WORKSPACE = 3,   /* workspace smaller than the call needs */
  FLCE_ERR_HIP = 4          /* a kernel launch failed (hipGetLastError after launching) */
} flce_status;

typedef enum flce_dtype {
  FLCE_F32 = 0,
  FLCE_BF16 = 1,
  FLCE_F16 = 2
} flce_dtype;

/*
 * Workspace bytes that let both flce_forward and flce_backward run with their default
 * chunking (the maximum of the two).  Returns 0 for invalid sizes or dtype.
 *
 * Forward needs S * N * 8 bytes of (max, sum-exp) partials plus ~4 * N bytes, where
 * S = min(max(256 / ceil(N / 256), 1), ceil(V / 256)) (integer division) is the number
 * of workgroups that share one 256-row token tile.  Backward needs 12 * N bytes of per-row
 * state plus one 256-byte scalar region, a dz slab of tc_pad * vc_pad elements of the
 * input type, and (16-bit types only) an fp32 dH accumulator of tc_pad * D floats,
 * where tc_pad and vc_pad are the token and vocabulary chunk sizes: by default
 * min(N, 4096) and min(V, 8192) rounded up to 256, with the vocabulary chunk trimmed in
 * steps of 256 (not below 4096) while the backward workspace exceeds 5% of N * V * 2
 * bytes.  Every region is rounded up to 256 bytes.
 */
size_t flce_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype);

/*
 * The chunking flce_backward uses for a workspace of `workspace_bytes`: the largest
 * (token_chunk, vocab_chunk), multiples of 256, that fit, shrinking the larger of the two
 * by halves from the default.  Writes them to *token_chunk and *vocab_chunk (either may
 * be NULL).  Returns FLCE_ERR_WORKSPACE when even 256 x 256 chunks do not fit, and
 * FLCE_ERR_INVALID_ARG for invalid sizes or dtype.  Host-only; touches no device.
 * Different chunkings give results that differ only in fp32 summation order.
 */
flce_status flce_backward_chunks(int64_t N, int64_t D, int64_t V, int dtype, size_t workspace_bytes,
                                 int64_t* token_chunk, int64_t* vocab_chunk);

/*
 * Forward: loss and per-row log-sum-exp without materialising the [N, V] logits.
 *
 *   H, W, y        inputs (device), layouts above; y[n] in [0, V) or == ignore_index.
 *   loss           [1] fp32 out: mean loss over valid rows (0 when N_valid == 0).
 *   lse            [N] fp32 out: log-sum-exp of every row, ignored rows included
 *                  (the only per-row state the backward needs besides y).
 *   n_valid        [1] int32 out: N_valid.
 *   dev_status     [1] int32 out: 0, or 1 when some label is neither ignore_index nor in
 *                  [0, V); such rows are then treated as ignored (a precondition
 *                  violation reported asynchronously; read it after synchronising).
 *   workspace      device scratch of workspace_bytes bytes (>= the forward's need).
 *
 * Errors (synchronous, nothing launched): FLCE_ERR_INVALID_ARG, FLCE_ERR_ALIGN,
 * FLCE_ERR_WORKSPACE.  FLCE_ERR_HIP if a launch failed.
 */
flce_status flce_forward(const void* H, const void* W, const int64_t* y, int64_t N, int64_t D,
                         int64_t V, int dtype, int64_t ignore_index, float* loss, float* lse,
                         int32_t* n_valid, int32_t* dev_status, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Backward: dH and dW from the saved per-row lse, recomputing logit tiles on the fly.
 *
 *   H, W, y        the forward's inputs (device).
 *   lse, n_valid   the forward's outputs (device).
 *   grad_loss      [1] fp32 device pointer to g = dL_total/dloss, or NULL for g = 1.
 *   dH             [N][D] out, input element type: overwritten; ignored rows get zeros.
 *   dW             [V][D] fp32 out: overwritten.
 *   workspace      device scratch; its size picks the chunking (flce_backward_chunks).
 *
 * Labels outside [0, V) that are not ignore_index are treated as ignored (the forward
 * reports them through dev_status).  Errors as for flce_forward.
 */
flce_status flce_backward(const void* H, const void* W, const int64_t* y, const float* lse,
                          const int32_t* n_valid, const float* grad_loss, int64_t N, int64_t D,
                          int64_t V, int dtype, int64_t ignore_index, void* dH, float* dW,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-pass workspace: the least bytes with which flce_forward_backward runs without
 * recomputing the logits.  Token chunks of T = min(N, 4096) rows (rounded up to 256) keep,
 * for the whole vocabulary, p~ = exp(z - m) in the input type (T x V' elements, V' = V
 * rounded up to 256) and the maxima m of each 128-row half tile in fp32 (T x V'/128), plus
 * a few MB of per-row and per-block terms: about T V' es + 4 T V'/128 bytes.  That is far
 * above the recomputing schedule's workspace: 1.07 GB, 25% of the 16-bit N x V logit
 * bytes, at N = 16384, V = 128256, bf16, and 102% of them at N = 4096, V = 32000.
 *
 * The kernels address operands through 32-bit buffer offsets, which must stay below
 * 2^31: a token chunk whose kept slab (T x V' x es bytes, read transposed by the dW
 * contraction) or hidden rows (T x D x es) would pass that is capped to the largest
 * multiple of 256 rows that fits (at V' es = 304128 bytes, 6912 rows; in fp32 at
 * V = 152064, 3328 rows).  Where no chunk fits -- the dH contraction reads all of W at
 * once, so V D es must stay below about 2^31 (e.g. not fp32 with V = 152064, D = 4096,
 * nor bf16 with V = 152064, D = 8192) -- the single pass is unavailable: this function returns
 * flce_workspace_bytes(...), and flce_forward_backward takes the recomputing schedule.
 * 0 for invalid sizes.
 */
size_t flce_forward_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, int dtype);

/*
 * The schedule flce_forward_backward takes for a workspace of `workspace_bytes`: writes the
 * single pass's token chunk to *token_chunk (a multiple of 256; min(N, 4096) rows rounded
 * up at the least, then multiples of 4096 up to N as the workspace allows, within the cap
 * above), or 0 when the call runs flce_forward then flce_backward.  Returns
 * FLCE_ERR_WORKSPACE when neither schedule fits and FLCE_ERR_INVALID_ARG for invalid
 * sizes or dtype.  Host-only; touches no device.
 */
flce_status flce_forward_backward_chunk(int64_t N, int64_t D, int64_t V, int dtype, size_t workspace_bytes,
                                        int64_t* token_chunk);

/*
 * Forward and backward in one call: loss, lse[N], n_valid, dev_status as flce_forward and
 * dH, dW (for the upstream gradient *grad_loss, NULL meaning 1) as flce_backward.
 *
 * "Unsloth Architecture: 5x Faster LLM Training via Triton", pillar 1 and its numpy walk
 * through, computes the loss and the hidden-state gradient of a token chunk in one pass
 * over its logits; "Arquitectura interna de Unsloth y optimización en Triton", section 3,
 * backpropagates into H and W directly.  When flce_forward_backward_chunk reports a token
 * chunk for the workspace, each chunk's logits are computed once (6 N V D flops in all):
 * the logit GEMM keeps p~ and m, the chunk's lse is combined, p~ becomes dz in place, and
 * dH (over the whole vocabulary at once) and dW are contracted from it.  Otherwise (a
 * workspace of at least flce_workspace_bytes but below the single pass's, or sizes where
 * the single pass cannot run) the call runs flce_forward then flce_backward (8 N V D
 * flops, the logits recomputed).
 *
 * Conventions, alignment, errors and determinism as flce_forward / flce_backward; results
 * of the two schedules agree within rounding (the single pass rounds p~ to the input type
 * before scaling it to dz).
 */
flce_status flce_forward_backward(const void* H, const void* W, const int64_t* y, int64_t N, int64_t D,
                                  int64_t V, int dtype, int64_t ignore_index, const float* grad_loss,
                                  float* loss, float* lse, int32_t* n_valid, int32_t* dev_status,
                                  void* dH, float* dW, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Bytes of the device array flce_forward_backward_static works in (one array per GPU). */
#define FLCE_STATIC_SCRATCH_BYTES ((size_t)144 << 20)

/*
 * flce_forward_backward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation, arguments (minus the workspace) and outputs as flce_forward_backward, with
 * the workspace taken from a fixed device array of FLCE_STATIC_SCRATCH_BYTES (144 MiB)
 * inside the library: the schedule and results are those of flce_forward_backward with a
 * caller workspace of that size (the recomputing schedule at the workload shapes here:
 * 134.4 MB at N = 16384, D = 4096, V = 128256, bf16; the single pass where it fits).
 *
 * The call allocates and frees nothing.  Each GPU holds its own copy of the array until
 * the process ends; its address is looked up once per device, on that device's first
 * call (the first call may therefore make the runtime load the library's code object).
 * Every call on one GPU shares that GPU's array, so calls that overlap on one GPU -- on
 * different streams, or from different host threads without ordering -- race and give
 * wrong results; calls ordered on one stream are safe.  Nothing in the array needs to
 * start at zero: every call writes each byte it reads first.
 *
 * Errors: FLCE_ERR_WORKSPACE when the problem needs more scratch than the array holds
 * (neither schedule fits FLCE_STATIC_SCRATCH_BYTES: the recomputing schedule needs 12
 * bytes per row of N besides its chunks, so e.g. 16M rows at a vocabulary too wide for the
 * single pass), reported before anything touches the device; FLCE_ERR_HIP when the array's
 * address cannot be obtained or a launch fails; otherwise as flce_forward_backward.
 */
flce_status flce_forward_backward_static(const void* H, const void* W, const int64_t* y, int64_t N, int64_t D,
                                         int64_t V, int dtype, int64_t ignore_index, const float* grad_loss,
                                         float* loss, float* lse, int32_t* n_valid, int32_t* dev_status, void* dH,
                                         float* dW, void* stream);

/*
 * Launch timing, a measurement aid for benchmarks and profilers (the computation needs none
 * of it).  Every kernel launch of flce_forward, flce_backward, flce_forward_backward and
 * flce_forward_backward_static has one of these ids:
 */
enum flce_kernel_id {
  FLCE_KERNEL_FWD = 0,           /* forward logit tiles with the online log-sum-exp */
  FLCE_KERNEL_FWD_KEEP = 1,      /* the same, keeping p~ = exp(z - m) (single pass) */
  FLCE_KERNEL_FWD_COMBINE = 2,   /* merge of the vocabulary splits: lse, row losses */
  FLCE_KERNEL_FWD_FINALIZE = 3,  /* loss, N_valid, status */
  FLCE_KERNEL_BWD_PREP = 4,      /* per-row terms of dz */
  FLCE_KERNEL_DZ = 5,            /* recomputed logit tiles -> dz slab */
  FLCE_KERNEL_DHDW = 6,          /* dH and dW of one chunk, contracted from its dz slab */
  FLCE_KERNEL_LABELS = 7,        /* N_valid before any chunk (single pass) */
  FLCE_KERNEL_KEEP_TO_DZ = 8     /* kept exponentials -> dz slab (single pass) */
};

/*
 * flce_timing_begin(events, kernel_ids, capacity): until flce_timing_end, the i-th launch
 * (i < capacity) carries events[2 i] and events[2 i + 1] -- hipEvent_t handles the caller
 * created with timing enabled -- as the start and stop events of its own dispatch
 * (hipExtLaunchKernel: stamped from the launch itself, no marker queued between kernels),
 * and its flce_kernel_id is written to kernel_ids[i].  Launches past `capacity` run
 * without events.  Host-global state: one caller at a time, and no calls on other threads
 * meanwhile.  Returns FLCE_OK, or FLCE_ERR_INVALID_ARG for null arrays or capacity < 1.
 * flce_timing_end() stops and returns the number of launches recorded; read the events
 * after synchronising.
 */
int32_t flce_timing_begin(void** events, int32_t* kernel_ids, int32_t capacity);
int32_t flce_timing_end(void);

/* Static, human-readable name of a status code. */
const char* flce_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
