"""fp64 CPU oracle for RMSNorm, the normalisation that produces the hidden states H fed to
the lm_head, forward and backward.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
``cpu_baseline`` leg may import this module.  The product path never calls it, and it
shares no code with the HIP library.

"Unsloth Kernel Architecture: Custom Triton Backpropagation and QLoRA Memory Scaling",
section 3 "Fused RMSNorm & SwiGLU Kernels", defines, per row x of width d,

    RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma        (gamma per channel)

and prints a closed-form gradient with gamma / RMS(x) outside the bracket.  That form is
the exact derivative when gamma is the same for every channel; for a per-channel gamma
the chain rule gives, with r = sqrt(mean(x^2) + eps) and dy the gradient of the output,

    dx_j     = (gamma_j dy_j) / r - x_j * (sum_i gamma_i x_i dy_i) / (d r^3)
    dgamma_j = sum over rows of dy_j x_j / r

which is what this module computes (it reduces to the page's form for uniform gamma).

Pins: PyTorch's fp64 ``rms_norm`` + autograd, the page's printed gradient at uniform
gamma, scale invariance (eps = 0: H(a x) = H(x) and <dx, x> = 0 per row; eps > 0: the
closed form of <dx, x>), the coupling sum_j gamma_j dgamma_j = sum_n <dy_n, y_n>, and
central finite differences.
"""
from __future__ import annotations

import numpy as np


def rmsnorm_forward(X: np.ndarray, gamma: np.ndarray, eps: float = 0.0) -> dict:
    """H = X / r * gamma per row, r = sqrt(mean(X^2) + eps); returns H and rstd = 1 / r."""
    X = np.asarray(X, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    r = np.sqrt(np.mean(X * X, axis=1) + eps)
    return dict(H=X / r[:, None] * gamma[None, :], rstd=1.0 / r)


def rmsnorm_backward(X: np.ndarray, gamma: np.ndarray, dH: np.ndarray, eps: float = 0.0) -> dict:
    """dX and dgamma of H = RMSNorm(X) * gamma for the output gradient dH (chain rule)."""
    X = np.asarray(X, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    dH = np.asarray(dH, dtype=np.float64)
    d = X.shape[1]
    r = np.sqrt(np.mean(X * X, axis=1) + eps)
    s = np.sum(gamma[None, :] * X * dH, axis=1)              # sum_i gamma_i x_i dy_i per row
    dX = (gamma[None, :] * dH) / r[:, None] - X * (s / (d * r ** 3))[:, None]
    dgamma = np.sum(dH * X / r[:, None], axis=0)
    return dict(dX=dX, dgamma=dgamma)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """x rounded to the storage type ("f32", "bf16" or "f16") with round to nearest even,
    through fp32 as a kernel computing in fp32 stores it; returned as fp64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype == "f16":
        return f.astype(np.float16).astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)

