"""ctypes binding of libflce.so (include/flce.h, include/flce_ce.h, include/flce_norm.h).  Argument marshalling only: every step
of the computation runs in the library's HIP kernels; torch provides device memory and
the current stream.

Importing this module loads the library and raises ImportError if it was not built
(``python -m linear_cross_entropy_lm_amd.build``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce.so")

FLCE_OK, FLCE_ERR_INVALID_ARG, FLCE_ERR_ALIGN, FLCE_ERR_WORKSPACE, FLCE_ERR_HIP = range(5)
FLCE_F32, FLCE_BF16, FLCE_F16 = 0, 1, 2
FLCE_STATIC_SCRATCH_BYTES = 144 << 20  # include/flce.h
# enum flce_kernel_id of include/flce.h
KERNEL_NAMES = ["fwd", "fwd_keep", "fwd_combine", "fwd_finalize", "bwd_prep", "dz", "dhdw", "labels", "keep_to_dz"]
IGNORE_INDEX = -100

# symbol -> (restype, argtypes), in the order of include/flce.h, flce_ce.h, flce_norm.h
_P, _I64, _I32, _SZ, _F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "flce_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I32]),
    "flce_backward_chunks": (_I32, [_I64, _I64, _I64, _I32, _SZ, _P, _P]),
    "flce_forward": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I32, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "flce_backward": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I64, _P, _P, _P, _SZ, _P]),
    "flce_forward_backward_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I32]),
    "flce_forward_backward_chunk": (_I32, [_I64, _I64, _I64, _I32, _SZ, _P]),
    "flce_forward_backward": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                     _P]),
    "flce_forward_backward_static": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I32, _I64, _P, _P, _P, _P, _P, _P, _P,
                                            _P]),
    "flce_timing_begin": (_I32, [_P, _P, _I32]),
    "flce_timing_end": (_I32, []),
    "flce_status_string": (ctypes.c_char_p, [_I32]),
    "flce_ce_workspace_bytes": (_SZ, [_I64]),
    "flce_ce_forward": (_I32, [_P, _I64, _P, _I64, _I64, _I32, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "flce_ce_backward": (_I32, [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I32, _I64, _P, _I64, _P]),
    "flce_rmsnorm_workspace_bytes": (_SZ, [_I64, _I64]),
    "flce_rmsnorm_forward": (_I32, [_P, _P, _I64, _I64, _I32, _F32, _P, _P, _P]),
    "flce_rmsnorm_backward": (_I32, [_P, _P, _P, _P, _I64, _I64, _I32, _P, _P, _P, _SZ, _P]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m linear_cross_entropy_lm_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


class FlceError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {flce_status_string(code)}")
        self.code = code


def flce_status_string(code: int) -> str:
    return lib.flce_status_string(int(code)).decode()


def dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return FLCE_BF16
    if dtype == torch.float16:
        return FLCE_F16
    if dtype == torch.float32:
        return FLCE_F32
    raise TypeError(f"unsupported element type {dtype} (bf16, fp16 or fp32)")


def flce_workspace_bytes(N: int, D: int, V: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(lib.flce_workspace_bytes(N, D, V, code))


def flce_backward_chunks(N: int, D: int, V: int, dtype, workspace_bytes: int) -> tuple[int, int]:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    tc, vc = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib.flce_backward_chunks(N, D, V, code, workspace_bytes, ctypes.byref(tc), ctypes.byref(vc))
    if st != FLCE_OK:
        raise FlceError(st, "flce_backward_chunks")
    return tc.value, vc.value


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(t: torch.Tensor, name: str, dtype: torch.dtype | None = None, shape=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def flce_forward(H, W, y, loss, lse, n_valid, dev_status, workspace, ignore_index=IGNORE_INDEX,
                 stream=None) -> None:
    """Launch the forward on ``stream`` (default: torch's current stream)."""
    N, D = H.shape
    V = W.shape[0]
    _check(H, "H")
    _check(W, "W", H.dtype, (V, D))
    _check(y, "y", torch.int64, (N,))
    _check(loss, "loss", torch.float32, (1,))
    _check(lse, "lse", torch.float32, (N,))
    _check(n_valid, "n_valid", torch.int32, (1,))
    _check(dev_status, "dev_status", torch.int32, (1,))
    _check(workspace, "workspace", torch.uint8)
    st = lib.flce_forward(_ptr(H), _ptr(W), _ptr(y), N, D, V, dtype_code(H.dtype), ignore_index,
                          _ptr(loss), _ptr(lse), _ptr(n_valid), _ptr(dev_status), _ptr(workspace),
                          workspace.numel(), _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_forward")


def flce_backward(H, W, y, lse, n_valid, grad_loss, dH, dW, workspace, ignore_index=IGNORE_INDEX,
                  stream=None) -> None:
    """Launch the backward on ``stream``; ``grad_loss`` may be None (g = 1)."""
    N, D = H.shape
    V = W.shape[0]
    _check(H, "H")
    _check(W, "W", H.dtype, (V, D))
    _check(y, "y", torch.int64, (N,))
    _check(lse, "lse", torch.float32, (N,))
    _check(n_valid, "n_valid", torch.int32, (1,))
    if grad_loss is not None:
        _check(grad_loss, "grad_loss", torch.float32, (1,))
    _check(dH, "dH", H.dtype, (N, D))
    _check(dW, "dW", torch.float32, (V, D))
    _check(workspace, "workspace", torch.uint8)
    st = lib.flce_backward(_ptr(H), _ptr(W), _ptr(y), _ptr(lse), _ptr(n_valid), _ptr(grad_loss),
                           N, D, V, dtype_code(H.dtype), ignore_index, _ptr(dH), _ptr(dW),
                           _ptr(workspace), workspace.numel(), _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_backward")


def flce_forward_backward_workspace_bytes(N: int, D: int, V: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(lib.flce_forward_backward_workspace_bytes(N, D, V, code))


def flce_forward_backward_chunk(N: int, D: int, V: int, dtype, workspace_bytes: int) -> int:
    """The single pass's token chunk for this workspace, or 0 when flce_forward_backward
    takes the two-call schedule."""
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    tc = ctypes.c_int64(-1)
    st = lib.flce_forward_backward_chunk(N, D, V, code, workspace_bytes, ctypes.byref(tc))
    if st != FLCE_OK:
        raise FlceError(st, "flce_forward_backward_chunk")
    return tc.value


def flce_forward_backward(H, W, y, grad_loss, loss, lse, n_valid, dev_status, dH, dW, workspace,
                          ignore_index=IGNORE_INDEX, stream=None) -> None:
    """Forward and backward in one call; the single-pass schedule when ``workspace`` holds
    flce_forward_backward_workspace_bytes, else forward then the recomputing backward."""
    N, D = H.shape
    V = W.shape[0]
    _check(H, "H")
    _check(W, "W", H.dtype, (V, D))
    _check(y, "y", torch.int64, (N,))
    if grad_loss is not None:
        _check(grad_loss, "grad_loss", torch.float32, (1,))
    _check(loss, "loss", torch.float32, (1,))
    _check(lse, "lse", torch.float32, (N,))
    _check(n_valid, "n_valid", torch.int32, (1,))
    _check(dev_status, "dev_status", torch.int32, (1,))
    _check(dH, "dH", H.dtype, (N, D))
    _check(dW, "dW", torch.float32, (V, D))
    _check(workspace, "workspace", torch.uint8)
    st = lib.flce_forward_backward(_ptr(H), _ptr(W), _ptr(y), N, D, V, dtype_code(H.dtype), ignore_index,
                                   _ptr(grad_loss), _ptr(loss), _ptr(lse), _ptr(n_valid), _ptr(dev_status),
                                   _ptr(dH), _ptr(dW), _ptr(workspace), workspace.numel(), _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_forward_backward")


def flce_forward_backward_static(H, W, y, grad_loss, loss, lse, n_valid, dev_status, dH, dW,
                                 ignore_index=IGNORE_INDEX, stream=None) -> None:
    """flce_forward_backward in the library's own fixed device array of
    FLCE_STATIC_SCRATCH_BYTES (no workspace argument, nothing allocated).  Calls that
    overlap on one GPU share that array and race."""
    N, D = H.shape
    V = W.shape[0]
    _check(H, "H")
    _check(W, "W", H.dtype, (V, D))
    _check(y, "y", torch.int64, (N,))
    if grad_loss is not None:
        _check(grad_loss, "grad_loss", torch.float32, (1,))
    _check(loss, "loss", torch.float32, (1,))
    _check(lse, "lse", torch.float32, (N,))
    _check(n_valid, "n_valid", torch.int32, (1,))
    _check(dev_status, "dev_status", torch.int32, (1,))
    _check(dH, "dH", H.dtype, (N, D))
    _check(dW, "dW", torch.float32, (V, D))
    st = lib.flce_forward_backward_static(_ptr(H), _ptr(W), _ptr(y), N, D, V, dtype_code(H.dtype), ignore_index,
                                          _ptr(grad_loss), _ptr(loss), _ptr(lse), _ptr(n_valid), _ptr(dev_status),
                                          _ptr(dH), _ptr(dW), _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_forward_backward_static")


# --- cross-entropy over materialised logits (include/flce_ce.h) ----------------------


def _check_rows(t: torch.Tensor, name: str) -> int:
    """A 2-D device tensor whose rows are contiguous (row pitch t.stride(0) >= t.shape[1]);
    returns the pitch."""
    if not t.is_cuda or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D device tensor")
    if t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} must have contiguous rows")
    return t.stride(0)


def flce_ce_workspace_bytes(N: int) -> int:
    return int(lib.flce_ce_workspace_bytes(int(N)))


def flce_ce_forward(Z, y, loss, lse, n_valid, dev_status, workspace, ignore_index=IGNORE_INDEX,
                    stream=None) -> None:
    """Mean cross-entropy of logits Z [N, V] (row pitch Z.stride(0)) against y."""
    ld = _check_rows(Z, "Z")
    N, V = Z.shape
    _check(y, "y", torch.int64, (N,))
    _check(loss, "loss", torch.float32, (1,))
    _check(lse, "lse", torch.float32, (N,))
    _check(n_valid, "n_valid", torch.int32, (1,))
    _check(dev_status, "dev_status", torch.int32, (1,))
    _check(workspace, "workspace", torch.uint8)
    st = lib.flce_ce_forward(_ptr(Z), ld, _ptr(y), N, V, dtype_code(Z.dtype), ignore_index, _ptr(loss),
                             _ptr(lse), _ptr(n_valid), _ptr(dev_status), _ptr(workspace), workspace.numel(),
                             _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_ce_forward")


def flce_ce_backward(Z, y, lse, n_valid, grad_loss, dZ, ignore_index=IGNORE_INDEX, stream=None) -> None:
    """dZ = (softmax(Z) - onehot(y)) * g / N_valid; dZ may be Z itself."""
    ld = _check_rows(Z, "Z")
    ldo = _check_rows(dZ, "dZ")
    N, V = Z.shape
    if tuple(dZ.shape) != (N, V) or dZ.dtype != Z.dtype:
        raise ValueError("dZ must match Z's shape and dtype")
    _check(y, "y", torch.int64, (N,))
    _check(lse, "lse", torch.float32, (N,))
    _check(n_valid, "n_valid", torch.int32, (1,))
    if grad_loss is not None:
        _check(grad_loss, "grad_loss", torch.float32, (1,))
    st = lib.flce_ce_backward(_ptr(Z), ld, _ptr(y), _ptr(lse), _ptr(n_valid), _ptr(grad_loss), N, V,
                              dtype_code(Z.dtype), ignore_index, _ptr(dZ), ldo, _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_ce_backward")


# --- RMSNorm of the hidden states (include/flce_norm.h) -------------------------------


def flce_rmsnorm_workspace_bytes(N: int, D: int) -> int:
    return int(lib.flce_rmsnorm_workspace_bytes(int(N), int(D)))


def flce_rmsnorm_forward(X, gamma, H, rstd, eps=0.0, stream=None) -> None:
    """H = X / sqrt(mean(X^2) + eps) * gamma per row; rstd[n] saved for the backward."""
    N, D = X.shape
    _check(X, "X")
    _check(gamma, "gamma", X.dtype, (D,))
    _check(H, "H", X.dtype, (N, D))
    _check(rstd, "rstd", torch.float32, (N,))
    st = lib.flce_rmsnorm_forward(_ptr(X), _ptr(gamma), N, D, dtype_code(X.dtype), float(eps), _ptr(H),
                                  _ptr(rstd), _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_rmsnorm_forward")


def flce_rmsnorm_backward(X, gamma, rstd, dH, dX, dgamma, workspace, stream=None) -> None:
    """dX (X's dtype) and dgamma (fp32) of the RMSNorm that produced H, from dH."""
    N, D = X.shape
    _check(X, "X")
    _check(gamma, "gamma", X.dtype, (D,))
    _check(rstd, "rstd", torch.float32, (N,))
    _check(dH, "dH", X.dtype, (N, D))
    _check(dX, "dX", X.dtype, (N, D))
    _check(dgamma, "dgamma", torch.float32, (D,))
    _check(workspace, "workspace", torch.uint8)
    st = lib.flce_rmsnorm_backward(_ptr(X), _ptr(gamma), _ptr(rstd), _ptr(dH), N, D, dtype_code(X.dtype),
                                   _ptr(dX), _ptr(dgamma), _ptr(workspace), workspace.numel(), _stream(stream))
    if st != FLCE_OK:
        raise FlceError(st, "flce_rmsnorm_backward")


def _check_labels(status: torch.Tensor) -> None:
    """Raise if the forward flagged a label outside [0, V) that is not ignore_index (reads the
    device status: one synchronisation)."""
    if int(status.item()) != 0:
        raise ValueError("labels outside [0, V) that are not ignore_index (the library treated those rows "
                         "as ignored)")


class FusedLinearCrossEntropy(torch.autograd.Function):
    """loss = mean cross-entropy of (H @ W^T, y) with the fused library.  Saves only the
    per-row lse and N_valid for the backward; dW is returned in the weights' dtype.  With
    check_labels (the default) the forward raises ValueError on a label outside [0, V) that
    is not ignore_index, at the cost of one synchronisation; without it such rows are
    treated as ignored."""

    @staticmethod
    def forward(ctx, H, W, y, ignore_index=IGNORE_INDEX, check_labels=True):
        N, D = H.shape
        V = W.shape[0]
        dev = H.device
        ws = torch.empty(flce_workspace_bytes(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        nv = torch.empty(1, dtype=torch.int32, device=dev)
        status = torch.empty(1, dtype=torch.int32, device=dev)
        flce_forward(H, W, y, loss, lse, nv, status, ws, ignore_index)
        if check_labels:
            _check_labels(status)
        ctx.save_for_backward(H, W, y, lse, nv)
        ctx.ignore_index = ignore_index
        return loss[0]

    @staticmethod
    def backward(ctx, g):
        H, W, y, lse, nv = ctx.saved_tensors
        N, D = H.shape
        V = W.shape[0]
        ws = torch.empty(flce_workspace_bytes(N, D, V, H.dtype), dtype=torch.uint8, device=H.device)
        dH = torch.empty_like(H)
        dW = torch.empty(V, D, dtype=torch.float32, device=H.device)
        gl = g.reshape(1).to(torch.float32).contiguous()
        flce_backward(H, W, y, lse, nv, gl, dH, dW, ws, ctx.ignore_index)
        return dH, dW.to(W.dtype), None, None, None


def fused_linear_cross_entropy(H, W, y, ignore_index=IGNORE_INDEX, check_labels=True):
    return FusedLinearCrossEntropy.apply(H, W, y, ignore_index, check_labels)


class NormLinearCrossEntropy(torch.autograd.Function):
    """loss = mean cross-entropy of (RMSNorm(X) * gamma @ W^T, y): the final norm, the lm_head
    and the loss.  Forward saves X, H, rstd, lse and N_valid; the backward's dH feeds the
    norm's backward directly.  dgamma and dW are returned in fp32 cast to the weights'
    dtype.  check_labels as for FusedLinearCrossEntropy."""

    @staticmethod
    def forward(ctx, X, gamma, W, y, eps=0.0, ignore_index=IGNORE_INDEX, check_labels=True):
        N, D = X.shape
        V = W.shape[0]
        dev = X.device
        H = torch.empty_like(X)
        rstd = torch.empty(N, dtype=torch.float32, device=dev)
        flce_rmsnorm_forward(X, gamma, H, rstd, eps)
        ws = torch.empty(flce_workspace_bytes(N, D, V, X.dtype), dtype=torch.uint8, device=dev)
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        nv = torch.empty(1, dtype=torch.int32, device=dev)
        status = torch.empty(1, dtype=torch.int32, device=dev)
        flce_forward(H, W, y, loss, lse, nv, status, ws, ignore_index)
        if check_labels:
            _check_labels(status)
        ctx.save_for_backward(X, gamma, W, y, H, rstd, lse, nv)
        ctx.ignore_index = ignore_index
        return loss[0]

    @staticmethod
    def backward(ctx, g):
        X, gamma, W, y, H, rstd, lse, nv = ctx.saved_tensors
        N, D = X.shape
        V = W.shape[0]
        dev = X.device
        ws = torch.empty(flce_workspace_bytes(N, D, V, X.dtype), dtype=torch.uint8, device=dev)
        dH = torch.empty_like(H)
        dW = torch.empty(V, D, dtype=torch.float32, device=dev)
        gl = g.reshape(1).to(torch.float32).contiguous()
        flce_backward(H, W, y, lse, nv, gl, dH, dW, ws, ctx.ignore_index)
        nws = torch.empty(flce_rmsnorm_workspace_bytes(N, D), dtype=torch.uint8, device=dev)
        dX = torch.empty_like(X)
        dgamma = torch.empty(D, dtype=torch.float32, device=dev)
        flce_rmsnorm_backward(X, gamma, rstd, dH, dX, dgamma, nws)
        return dX, dgamma.to(gamma.dtype), dW.to(W.dtype), None, None, None, None
