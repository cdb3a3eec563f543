"""fp64 CPU oracle for the fused lm_head projection + cross-entropy loss and its gradients.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
``cpu_baseline`` leg may import this module.  The product path never calls it, and it
shares no code with the HIP library: it is a plain, slow, obviously correct statement
of what the fused kernels must produce.

What it computes (all in fp64, inputs widened exactly from their fp32 / bf16 values):

* logits       z[n, v] = sum_d H[n, d] * W[v, d]              -- the lm_head projection
  Z = X W_vocab^T of "Arquitectura interna de Unsloth y optimización en Triton",
  section 3 (Fused Cross Entropy), and Z = H W^T of "Unsloth Architecture: 5x Faster
  LLM Training via Triton", section "The Un-Fused Cross-Entropy Logit Disaster".
* per-row log-sum-exp lse[n] = m + log(sum_v exp(z[n, v] - m)), m = max_v z[n, v]:
  the max-subtracted normaliser of the same two sections (two passes over a fully
  materialised row; the streaming form the kernels use is deliberately not used here).
* per-row loss l[n] = lse[n] - z[n, y[n]] (the cross-entropy equation of the "Fused
  Chunked Cross-Entropy Loss" pillar of the second page above); rows whose label equals
  ``ignore_index`` contribute nothing.
* loss = sum_n l[n] / N_valid, N_valid = number of non-ignored rows.  The page's numpy
  reference divides by the token count; with ignored rows the divisor is the number of
  rows that carry a label (PyTorch's ignore_index + mean convention).  N_valid = 0
  gives loss 0 and zero gradients.
* logit gradient dz[n, v] = (softmax(z[n])[v] - [v == y[n]]) * g / N_valid for valid
  rows and 0 for ignored rows (the analytic gradient p - onehot of section 3 of the
  first page and of the second page's pillar; g is the upstream gradient of the loss).
* dH = dz W and dW = dz^T H: the gradient flows into the hidden states and into the
  vocabulary weight (section 3 of the first page names both).
* ce_from_logits: the same loss, lse and logit gradient for logits given directly (the
  row-streaming kernel of "Unsloth Kernel Architecture: Custom Triton Backpropagation and
  QLoRA Memory Scaling", section 1, takes logits and labels).

Rows are processed in blocks of ``row_block`` rows only so that a block's logits fit in
memory; every row is computed independently from its own full logit vector.

Pins: the test suite checks this module against closed forms (W = 0, H = 0),
invariants (gradient rows summing to zero, shift invariance, the <dW, W> = <dH, H>
coupling), central finite differences, PyTorch's fp64 cross_entropy + autograd on
small shapes, and a statistical band for the loss on the paper-shaped workloads;
ce_from_logits against PyTorch's fp64 cross_entropy on logits and the constant-logit
closed form.
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


def count_valid(y: np.ndarray, V: int, ignore_index: int = IGNORE_INDEX) -> int:
    """N_valid.  A label outside [0, V) that is not ``ignore_index`` is a caller error."""
    y = np.asarray(y, dtype=np.int64)
    ignored = y == ignore_index
    bad = (~ignored) & ((y < 0) | (y >= V))
    if bad.any():
        raise ValueError(f"labels outside [0, {V}) at rows {np.nonzero(bad)[0][:8].tolist()}")
    return int((~ignored).sum())


def logits(H: np.ndarray, W: np.ndarray, rows) -> np.ndarray:
    """Full logit rows z[rows, :] = H[rows] W^T (fp64 matrix product)."""
    return np.asarray(H[rows], dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    """Two-pass log-sum-exp of each row: subtract the row maximum, sum, take the log."""
    m = Z.max(axis=1)
    return m + np.log(np.exp(Z - m[:, None]).sum(axis=1))


def _scale(n_valid: int, g: float) -> float:
    return float(g) / n_valid if n_valid > 0 else 0.0


def logit_grad(Z: np.ndarray, lse: np.ndarray, y_rows: np.ndarray, s: float,
               ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """dz for a block of rows: (exp(z - lse) - onehot(y)) * s, zero for ignored rows."""
    P = np.exp(Z - lse[:, None])
    valid = y_rows != ignore_index
    idx = np.nonzero(valid)[0]
    P[idx, y_rows[idx]] -= 1.0
    P[~valid] = 0.0
    return P * s


def forward_backward(H: np.ndarray, W: np.ndarray, y: np.ndarray,
                     ignore_index: int = IGNORE_INDEX, g: float = 1.0,
                     row_block: int = 64, grads: bool = True) -> dict:
    """Loss, per-row lse and per-row loss, and (optionally) dH and dW, all fp64."""
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    N, D = H.shape
    V = W.shape[0]
    n_valid = count_valid(y, V, ignore_index)
    s = _scale(n_valid, g)
    lse = np.empty(N)
    row_loss = np.zeros(N)
    dH = np.zeros((N, D)) if grads else None
    dW = np.zeros((V, D)) if grads else None
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        Z = logits(H, W, slice(r0, r1))
        l = logsumexp_rows(Z)
        lse[r0:r1] = l
        yy = y[r0:r1]
        idx = np.nonzero(yy != ignore_index)[0]
        row_loss[r0 + idx] = l[idx] - Z[idx, yy[idx]]
        if grads:
            dZ = logit_grad(Z, l, yy, s, ignore_index)
            dH[r0:r1] = dZ @ W
            dW += dZ.T @ H[r0:r1]
    loss = row_loss.sum() / n_valid if n_valid > 0 else 0.0
    return dict(loss=float(loss), lse=lse, row_loss=row_loss, dH=dH, dW=dW,
                n_valid=n_valid, scale=s)


def forward_stats(H: np.ndarray, W: np.ndarray, y: np.ndarray,
                  ignore_index: int = IGNORE_INDEX, row_block: int = 256) -> dict:
    """Forward only: loss, lse and per-row loss for every row (no gradients)."""
    out = forward_backward(H, W, y, ignore_index, 1.0, row_block, grads=False)
    return dict(loss=out["loss"], lse=out["lse"], row_loss=out["row_loss"],
                n_valid=out["n_valid"])


def dH_rows(H: np.ndarray, W: np.ndarray, y: np.ndarray, rows, n_valid: int,
            g: float = 1.0, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """dH for selected rows.  Each row needs only its own logits and N_valid."""
    rows = np.asarray(rows, dtype=np.int64)
    W = np.asarray(W, dtype=np.float64)
    Z = logits(H, W, rows)
    lse = logsumexp_rows(Z)
    dZ = logit_grad(Z, lse, np.asarray(y, dtype=np.int64)[rows], _scale(n_valid, g),
                    ignore_index)
    return dZ @ W


def dW_rows(H: np.ndarray, W: np.ndarray, y: np.ndarray, vrows, lse: np.ndarray,
            n_valid: int, g: float = 1.0, ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """dW for selected vocabulary rows: dW[v] = sum_n dz[n, v] H[n].  ``lse`` must be this
    module's per-row log-sum-exp for every row (from ``forward_stats``)."""
    vrows = np.asarray(vrows, dtype=np.int64)
    H = np.asarray(H, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    Zc = H @ np.asarray(W, dtype=np.float64)[vrows].T  # z[:, vrows], [N, len(vrows)]
    P = np.exp(Zc - lse[:, None])
    P -= (y[:, None] == vrows[None, :]).astype(np.float64)
    P[y == ignore_index] = 0.0
    return (P * _scale(n_valid, g)).T @ H


def ce_from_logits(Z: np.ndarray, y: np.ndarray, ignore_index: int = IGNORE_INDEX, g: float = 1.0,
                   row_block: int = 256, grads: bool = True) -> dict:
    """Cross-entropy of logits that are already materialised, Z [N, V] (fp64): per-row
    log-sum-exp minus the label's logit, mean over valid rows, and the gradient
    (softmax - onehot) g / N_valid ("Unsloth Kernel Architecture: Custom Triton
    Backpropagation and QLoRA Memory Scaling", section 1 "Fused Cross-Entropy Loss with
    Logit Streaming", whose kernel takes the logits and labels of one row at a time).
    Rows are processed in blocks only for memory; each row uses its own full logit row.
    Returns loss, lse, row_loss, n_valid and (grads) dZ."""
    Z = np.asarray(Z, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    N, V = Z.shape
    n_valid = count_valid(y, V, ignore_index)
    s = _scale(n_valid, g)
    lse = np.empty(N)
    row_loss = np.zeros(N)
    dZ = np.empty((N, V)) if grads else None
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        Zb = Z[r0:r1]
        yb = y[r0:r1]
        Lb = logsumexp_rows(Zb)
        lse[r0:r1] = Lb
        valid = yb != ignore_index
        idx = np.nonzero(valid)[0]
        row_loss[r0 + idx] = Lb[idx] - Zb[idx, yb[idx]]
        if grads:
            dZ[r0:r1] = logit_grad(Zb, Lb, yb, s, ignore_index)
    loss = float(row_loss.sum() / n_valid) if n_valid else 0.0
    out = dict(loss=loss, lse=lse, row_loss=row_loss, n_valid=n_valid)
    if grads:
        out["dZ"] = dZ
    return out
