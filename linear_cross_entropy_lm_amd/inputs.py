"""Seeded synthetic inputs for the fused lm_head projection + cross-entropy path.

This module only draws and formats inputs; it holds none of the loss or gradient
arithmetic.  Both the HIP path (through the binding) and the fp64 CPU oracle consume
exactly the tensors produced here: bf16 inputs are carried as their raw 16-bit
patterns, and the oracle widens those patterns to fp64 exactly.

Workload shapes follow the vocabulary sizes and batch shapes the pages discuss
("Unsloth Architecture: 5x Faster LLM Training via Triton", section "The Un-Fused
Cross-Entropy Logit Disaster": Llama-2 32,000, Mistral 32,768, Llama-3 128,256,
Qwen-2.5 152,064; a batch of 4 x 4,096 tokens for Llama-3).  No dataset is involved:
hidden states and weights are Gaussian, labels are uniform or Zipf-skewed.

Generation is blockwise: every 4096-row block of a tensor has its own PCG64 stream
keyed by (config seed, tensor id, block index), so blocks fill in parallel threads and
the result does not depend on the thread count.  Normals come from Marsaglia's polar
method with a log built only from integer steps and correctly rounded + - * / sqrt, and
bf16 rounding is done on the bit patterns: the bytes are identical on every host CPU
(library transcendentals and vectorised samplers differ between instruction sets).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch

try:  # numpy >= 2
    from numpy._core.multiarray import _set_madvise_hugepage
except ImportError:  # pragma: no cover
    from numpy.core.multiarray import _set_madvise_hugepage

# Large numpy buffers are otherwise madvise'd for transparent huge pages; on hosts where
# first-touch of such pages is slow this dominates generation time.  Performance only.
_set_madvise_hugepage(False)

IGNORE_INDEX = -100
_BLOCK_ROWS = 4096
_TENSOR_H, _TENSOR_W, _TENSOR_LABELS = 1, 2, 3


@dataclass(frozen=True)
class Config:
    """One synthetic workload: sizes, dtype and input distributions."""

    name: str
    N: int  # tokens (batch x sequence)
    D: int  # hidden size
    V: int  # vocabulary size
    dtype: str  # "f32", "bf16" or "f16"
    seed: int
    h_dist: str = "rms"  # "normal": N(0,1); "rms": N(0,1) rows scaled to unit RMS
    w_std: float = 0.02
    label_dist: str = "uniform"  # "uniform" or "zipf"
    zipf_s: float = 1.1
    ignore_frac: float = 0.05
    ignore_layout: str = "random"  # "random" positions or contiguous "tail"
    batch: int = 1
    seq: int = 0

    @property
    def n_ignored(self) -> int:
        return int(math.floor(self.ignore_frac * self.N + 0.5))

    def describe(self) -> str:
        return (f"{self.name}: N={self.N} (batch {self.batch} x seq {self.seq}), D={self.D}, "
                f"V={self.V}, {self.dtype}")


# The workloads.  The tiny fp32 case is the one the oracle finishes instantly; the next
# four are shaped like the Llama-2, Mistral, Llama-3 and Qwen-2.5 heads.
CONFIGS = {
    "tiny_f32": Config("tiny_f32", N=64, D=256, V=1024, dtype="f32", seed=1001,
                       h_dist="normal", ignore_frac=0.10, batch=1, seq=64),
    "llama2": Config("llama2", N=4096, D=4096, V=32000, dtype="bf16", seed=1002,
                     batch=1, seq=4096),
    "mistral": Config("mistral", N=8192, D=4096, V=32768, dtype="bf16", seed=1003,
                      label_dist="zipf", batch=2, seq=4096),
    "llama3": Config("llama3", N=16384, D=4096, V=128256, dtype="bf16", seed=1004,
                     batch=4, seq=4096),
    "qwen25": Config("qwen25", N=8192, D=3584, V=152064, dtype="bf16", seed=1005,
                     ignore_frac=0.20, ignore_layout="tail", batch=1, seq=8192),
    # fp16 variants of two of them (the pages name fp16 next to bf16)
    "llama2_f16": Config("llama2_f16", N=4096, D=4096, V=32000, dtype="f16", seed=1006,
                         batch=1, seq=4096),
    "llama3_f16": Config("llama3_f16", N=16384, D=4096, V=128256, dtype="f16", seed=1007,
                         batch=4, seq=4096),
}


def case(N: int, D: int, V: int, dtype: str = "bf16", seed: int = 7, **kw) -> Config:
    """A small ad-hoc workload (tests): same distributions, free sizes."""
    base = dict(h_dist="rms", ignore_frac=0.05, ignore_layout="random", batch=1, seq=N)
    base.update(kw)
    return Config(f"case_N{N}_D{D}_V{V}_{dtype}_s{seed}", N=N, D=D, V=V, dtype=dtype,
                  seed=seed, **base)


# Test-only workloads with stored oracle values (tests/golden/fullsize_<name>.npz).
GOLDEN_CASES = {
    # 16640 rows at the Qwen-2.5 vocabulary: one single-pass chunk of every row would span
    # 16640 x 152064 x 2 bytes, past 32-bit offsets, so the single pass runs capped chunks
    "spcap_bf16": case(16640, 64, 152064, "bf16", seed=1010),
    # A 256,000-token vocabulary at a hidden size that puts W and dW past 2^31 elements
    # (2.16e9; 4.33 GB in bf16, 8.65 GB in fp32): the last 503 of the 1000 vocabulary tiles
    # start beyond 2 GiB into W and the last 7 beyond element 2^31, and the single pass is
    # unavailable (one dH contraction over all of W would pass the kernels' 32-bit operand
    # offsets), so the one-call entry point runs the two calls
    "wide_vocab_bf16": case(1100, 8448, 256000, "bf16", seed=1011),
    # Tokens rather than vocabulary past 2^31 elements: H and dH hold 262244 x 8448 = 2.2e9
    # (4.4 GB in bf16), the last token tile ragged; here the single pass is available
    "long_tokens_bf16": case(262244, 8448, 1031, "bf16", seed=1012),
    # The Llama-3-shaped head with fp32 inputs: W and dW are 2.1 GB each, and the single
    # pass's dH contraction over all of W stays just inside the 32-bit operand offsets
    "llama3_f32": replace(CONFIGS["llama3"], name="llama3_f32", dtype="f32", seed=1013),
}


# ---------------------------------------------------------------------------------
# bf16 bit-pattern helpers (format conversion only)
# ---------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (int16/uint16) to fp64."""
    u = bits.view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


_LN2 = 0.6931471805599453
_SQRT_HALF = 0.7071067811865476
_LN_TERMS = [1.0 / (2 * k + 1) for k in range(12)]               # 2 atanh series
_SUB = 1 << 18                                                    # pairs per sub-chunk


def _horner(x2: np.ndarray, coefs) -> np.ndarray:
    acc = np.full_like(x2, coefs[-1])
    for c in reversed(coefs[:-1]):
        acc *= x2
        acc += c
    return acc


def _log(x: np.ndarray) -> np.ndarray:
    """Natural log of x in (0, 1] from exact frexp plus a 2*atanh series, using only
    correctly rounded + - * / so the result is identical on every x86 host."""
    m, e = np.frexp(x)
    small = m < _SQRT_HALF
    m = np.where(small, m * 2.0, m)
    e = np.where(small, e - 1, e).astype(np.float64)
    t = (m - 1.0) / (m + 1.0)
    return e * _LN2 + 2.0 * t * _horner(t * t, _LN_TERMS)


# Faster log for the sampler: m in [0.5, 1) falls in one of
# 256 bins of width 1/512 whose centres c_j are exact; ln c_j comes from the series above.
_LOG_C = 0.5 + (np.arange(256, dtype=np.float64) + 0.5) / 512.0
_LOG_LNC = _log(_LOG_C)


def _log_fast(x: np.ndarray) -> np.ndarray:
    """ln x for x in (0, 1): ln x = e ln 2 + ln c_j + 2 atanh((m - c_j) / (m + c_j)),
    |t| < 1e-3 so four series terms reach full double precision."""
    m, e = np.frexp(x)
    j = ((m - 0.5) * 512.0).astype(np.int64)
    c = _LOG_C[j]
    t = (m - c) / (m + c)
    t2 = t * t
    return e * _LN2 + _LOG_LNC[j] + 2.0 * t * (1.0 + t2 * (1.0 / 3.0 + t2 * (1.0 / 5.0 + t2 * (1.0 / 7.0))))


def _gaussian_block(seed: int, tensor: int, block: int, rows: int, cols: int) -> np.ndarray:
    """Standard normals for one row block by Marsaglia's polar method: PCG64 uniform pairs
    (integer arithmetic) in the unit disc, z = v sqrt(-2 ln s / s), s = |v|^2; accepted
    pairs fill consecutive elements."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, block])))
    n = rows * cols
    need = (n + 1) // 2
    z = np.empty(2 * need)
    filled = 0
    while filled < need:
        v = rng.random((_SUB, 2)) * 2.0 - 1.0
        s = v[:, 0] * v[:, 0] + v[:, 1] * v[:, 1]
        ok = (s > 0.0) & (s < 1.0)
        v, s = v[ok], s[ok]
        k = min(len(s), need - filled)
        v, s = v[:k], s[:k]
        f = np.sqrt(-2.0 * _log_fast(s) / s)
        z[2 * filled:2 * (filled + k)] = (v * f[:, None]).reshape(-1)
        filled += k
    return z[:n].reshape(rows, cols)


def _rne_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even on the bit patterns (finite inputs), as uint16."""
    u = x.view(np.uint32)
    return ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)


def _rne_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE fp16, round to nearest even (numpy's conversion), as uint16 bits."""
    return x.astype(np.float16).view(np.uint16)


_ROUND16 = {"bf16": _rne_bf16, "f16": _rne_f16}


def _normal_rows(rows: int, cols: int, seed: int, tensor: int, threads: int, finish,
                 dtype: str, block_rows: int = _BLOCK_ROWS) -> np.ndarray:
    """[rows, cols] of finish(standard normals) rounded to fp32, then (dtype "bf16" or
    "f16") to 16-bit patterns; block b (block_rows rows) draws from its own stream."""
    out = np.empty((rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)
    nblk = (rows + block_rows - 1) // block_rows

    def fill(b: int) -> None:
        r0, r1 = b * block_rows, min(rows, (b + 1) * block_rows)
        blk = finish(_gaussian_block(seed, tensor, b, r1 - r0, cols)).astype(np.float32)
        out[r0:r1] = blk if dtype == "f32" else _ROUND16[dtype](blk)

    if nblk == 1 or threads <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def _unit_rms(x: np.ndarray) -> np.ndarray:
    """Rows scaled to unit root-mean-square (gamma = 1, eps = 0).  The row sum of squares
    is numpy's pairwise add-reduction: additions only, in a fixed order."""
    ss = np.add.reduce(x * x, axis=1)
    return x / np.sqrt(ss / x.shape[1])[:, None]


@dataclass
class Inputs:
    """Generated inputs.  ``H`` and ``W`` are fp32 tensors for f32 workloads and int16
    bit patterns for bf16 / f16 workloads; ``y`` is int64 with IGNORE_INDEX rows."""

    cfg: Config
    H: torch.Tensor
    W: torch.Tensor
    y: torch.Tensor
    _digest: str | None = field(default=None, repr=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.cfg.dtype]

    def h64(self) -> np.ndarray:
        return self._widen(self.H)

    def w64(self) -> np.ndarray:
        return self._widen(self.W)

    def y64(self) -> np.ndarray:
        return self.y.numpy().astype(np.int64)

    def _widen(self, t: torch.Tensor) -> np.ndarray:
        if self.cfg.dtype == "f32":
            return t.numpy().astype(np.float64)
        if self.cfg.dtype == "f16":
            return t.numpy().view(np.float16).astype(np.float64)
        return bf16_bits_to_f64(t.numpy())

    def device_tensors(self, device) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """(H, W, y) on ``device`` in the workload's element type."""
        if self.cfg.dtype == "f32":
            H, W = self.H, self.W
        else:
            H, W = self.H.view(self.torch_dtype), self.W.view(self.torch_dtype)
        return (H.to(device).contiguous(), W.to(device).contiguous(),
                self.y.to(device).contiguous())

    def digest(self) -> str:
        """Fingerprint of the exact input bytes (xxh3-128 over H, W, y)."""
        if self._digest is None:
            import xxhash
            h = xxhash.xxh3_128()
            for t in (self.H, self.W, self.y):
                h.update(memoryview(t.contiguous().numpy()).cast("B"))
            self._digest = h.hexdigest()
        return self._digest


def _draw_labels(cfg, N: int, V: int) -> np.ndarray:
    """Labels then the ignore mask for a workload (uniform or Zipf over a random vocabulary
    permutation; ignored rows at random positions or as a contiguous tail)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, _TENSOR_LABELS, 0])))
    if cfg.label_dist == "uniform":
        y = rng.integers(0, V, size=N, dtype=np.int64)
    elif cfg.label_dist == "zipf":
        perm = rng.permutation(V)
        # p_k proportional to k^-s, k = 1..V: weights exp(-s ln k) from the same exact-
        # arithmetic log, cumulative sum in order, inverse-CDF draw
        k = np.arange(1, V + 1, dtype=np.float64)
        m, e = np.frexp(k)  # ln k = ln m + e ln 2 with m in [0.5, 1)
        lnk = _log(m) + e.astype(np.float64) * _LN2
        w = _exp_neg(cfg.zipf_s * lnk)
        cdf = np.cumsum(w)
        idx = np.searchsorted(cdf, rng.random(N) * cdf[-1], side="right")
        y = perm[np.minimum(idx, V - 1)].astype(np.int64)
    else:
        raise ValueError(cfg.label_dist)
    k_ign = cfg.n_ignored
    if k_ign:
        if cfg.ignore_layout == "random":
            idx = rng.permutation(N)[:k_ign]
        elif cfg.ignore_layout == "tail":
            idx = np.arange(N - k_ign, N)
        else:
            raise ValueError(cfg.ignore_layout)
        y[idx] = IGNORE_INDEX

    return y


def generate(cfg: Config, threads: int = 8) -> Inputs:
    """Draw H, W, labels and the ignore mask (in that order) for ``cfg``.  Every step is
    integer arithmetic or correctly rounded floating point, so the bytes are the same on
    any host."""
    N, D, V = cfg.N, cfg.D, cfg.V
    if cfg.h_dist == "rms":
        H = _normal_rows(N, D, cfg.seed, _TENSOR_H, threads, _unit_rms, cfg.dtype)
    elif cfg.h_dist == "normal":
        H = _normal_rows(N, D, cfg.seed, _TENSOR_H, threads, lambda z: z, cfg.dtype)
    else:
        raise ValueError(cfg.h_dist)
    W = _normal_rows(V, D, cfg.seed, _TENSOR_W, threads, lambda z: z * cfg.w_std, cfg.dtype)

    y = _draw_labels(cfg, N, V)

    if cfg.dtype in ("bf16", "f16"):
        Ht, Wt = torch.from_numpy(H.view(np.int16)), torch.from_numpy(W.view(np.int16))
    elif cfg.dtype == "f32":
        Ht, Wt = torch.from_numpy(H), torch.from_numpy(W)
    else:
        raise ValueError(cfg.dtype)
    return Inputs(cfg, Ht.contiguous(), Wt.contiguous(), torch.from_numpy(y).contiguous())


# ---------------------------------------------------------------------------------
# Materialised logits (the standalone cross-entropy over logits)
# ---------------------------------------------------------------------------------

_TENSOR_Z = 4
_LOGIT_BLOCK_ROWS = 64  # logit rows are long (V elements): small blocks keep temporaries small


def _logit_block_rows(V: int) -> int:
    """Rows per generator stream: 64 for long rows, more for short ones (>= 2^16 values)."""
    return max(_LOGIT_BLOCK_ROWS, (1 << 16) // max(V, 1))


@dataclass(frozen=True)
class LogitConfig:
    """Logits Z [N, V] ~ N(0, z_std^2) per element (the spread of the Llama-3-shaped head's
    logits, 0.02 sqrt(4096) ~ 1.3, rounded up), labels and ignored rows as for Config.
    ``ld`` > V pads each row (the pad is filled with a large value the kernels must not
    read)."""

    name: str
    N: int
    V: int
    dtype: str
    seed: int
    z_std: float = 2.0
    label_dist: str = "uniform"
    zipf_s: float = 1.1
    ignore_frac: float = 0.05
    ignore_layout: str = "random"
    ld: int = 0

    @property
    def n_ignored(self) -> int:
        return int(math.floor(self.ignore_frac * self.N + 0.5))

    @property
    def pitch(self) -> int:
        return self.ld or self.V

    def describe(self) -> str:
        return f"{self.name}: logits N={self.N}, V={self.V} (pitch {self.pitch}), {self.dtype}"


LOGIT_CONFIGS = {
    "ce_llama3": LogitConfig("ce_llama3", N=16384, V=128256, dtype="bf16", seed=2001),
}


def logit_case(N: int, V: int, dtype: str = "bf16", seed: int = 5, **kw) -> LogitConfig:
    return LogitConfig(f"ce_N{N}_V{V}_{dtype}_s{seed}", N=N, V=V, dtype=dtype, seed=seed, **kw)


@dataclass
class LogitInputs:
    """``Z`` [N, pitch] (fp32, or int16 bit patterns for bf16 / f16) and labels ``y``."""

    cfg: LogitConfig
    Z: torch.Tensor
    y: torch.Tensor
    _digest: str | None = field(default=None, repr=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.cfg.dtype]

    def z64(self, rows=None) -> np.ndarray:
        """Exact fp64 widening of the logits (columns < V), optionally of some rows."""
        t = self.Z.numpy()[:, :self.cfg.V] if rows is None else self.Z.numpy()[rows, :self.cfg.V]
        if self.cfg.dtype == "f32":
            return t.astype(np.float64)
        if self.cfg.dtype == "f16":
            return t.view(np.float16).astype(np.float64)
        return bf16_bits_to_f64(t)

    def y64(self) -> np.ndarray:
        return self.y.numpy().astype(np.int64)

    def device_tensors(self, device) -> tuple[torch.Tensor, torch.Tensor]:
        """(Z [N, V] view with row pitch ``pitch``, y) on ``device``."""
        Z = self.Z if self.cfg.dtype == "f32" else self.Z.view(self.torch_dtype)
        Zd = Z.to(device).contiguous()
        return Zd[:, :self.cfg.V], self.y.to(device).contiguous()

    def digest(self) -> str:
        if self._digest is None:
            import xxhash
            h = xxhash.xxh3_128()
            for t in (self.Z, self.y):
                h.update(memoryview(t.contiguous().numpy()).cast("B"))
            self._digest = h.hexdigest()
        return self._digest


def generate_logits(cfg: LogitConfig, threads: int = 8) -> LogitInputs:
    """Draw Z, then labels and the ignore mask, for ``cfg`` (same exact-arithmetic normals
    and rounding as ``generate``).  Pad columns hold 1e4 (finite, far above any logit)."""
    N, V, P = cfg.N, cfg.V, cfg.pitch
    Z = _normal_rows(N, V, cfg.seed, _TENSOR_Z, threads, lambda z: z * cfg.z_std, cfg.dtype,
                     block_rows=_logit_block_rows(V))
    if P > V:
        pad = np.float32(1e4)
        fill = pad if cfg.dtype == "f32" else _ROUND16[cfg.dtype](np.array([pad], dtype=np.float32))[0]
        Zp = np.empty((N, P), dtype=Z.dtype)
        Zp[:, :V] = Z
        Zp[:, V:] = fill
        Z = Zp
    y = _draw_labels(cfg, N, V)
    Zt = torch.from_numpy(Z if cfg.dtype == "f32" else Z.view(np.int16)).contiguous()
    return LogitInputs(cfg, Zt, torch.from_numpy(y).contiguous())


# ---------------------------------------------------------------------------------
# Pre-norm hidden states (the RMSNorm that produces H)
# ---------------------------------------------------------------------------------

_TENSOR_X, _TENSOR_GAMMA, _TENSOR_DH = 5, 6, 7


@dataclass(frozen=True)
class NormConfig:
    """X [N, D] ~ N(0, x_std^2) (pre-norm hidden states), gamma [D] ~ 1 + N(0, gamma_std^2)
    (a trained norm weight near 1), dH [N, D] ~ N(0, dh_std^2) (the gradient of the norm's
    output; the operation is linear in it, so its scale is free), and eps."""

    name: str
    N: int
    D: int
    dtype: str
    seed: int
    x_std: float = 2.0
    gamma_std: float = 0.1
    dh_std: float = 1.0
    eps: float = 1e-5

    def describe(self) -> str:
        return f"{self.name}: RMSNorm N={self.N}, D={self.D}, {self.dtype}, eps={self.eps:g}"


NORM_CONFIGS = {
    # the final norm before the Llama-3-shaped head: 4 x 4096 tokens, hidden size 4096
    "norm_llama3": NormConfig("norm_llama3", N=16384, D=4096, dtype="bf16", seed=3001),
}


def norm_case(N: int, D: int, dtype: str = "bf16", seed: int = 9, **kw) -> NormConfig:
    return NormConfig(f"norm_N{N}_D{D}_{dtype}_s{seed}", N=N, D=D, dtype=dtype, seed=seed, **kw)


def _widen(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Exact fp64 values of a tensor held as fp32 or as 16-bit patterns."""
    a = t.numpy()
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    return bf16_bits_to_f64(a)


@dataclass
class NormInputs:
    """``X`` [N, D], ``gamma`` [D], ``dH`` [N, D]: fp32, or int16 bit patterns for bf16/f16."""

    cfg: NormConfig
    X: torch.Tensor
    gamma: torch.Tensor
    dH: torch.Tensor

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.cfg.dtype]

    def x64(self) -> np.ndarray:
        return _widen(self.X, self.cfg.dtype)

    def gamma64(self) -> np.ndarray:
        return _widen(self.gamma, self.cfg.dtype)

    def dh64(self) -> np.ndarray:
        return _widen(self.dH, self.cfg.dtype)

    def device_tensors(self, device) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        def dev(t):
            t = t if self.cfg.dtype == "f32" else t.view(self.torch_dtype)
            return t.to(device).contiguous()
        return dev(self.X), dev(self.gamma), dev(self.dH)

    def digest(self) -> str:
        """Fingerprint of the exact input bytes (xxh3-128 over X, gamma, dH)."""
        import xxhash
        h = xxhash.xxh3_128()
        for t in (self.X, self.gamma, self.dH):
            h.update(memoryview(t.contiguous().numpy()).cast("B"))
        return h.hexdigest()


def generate_norm(cfg: NormConfig, threads: int = 8) -> NormInputs:
    """Draw X, gamma, dH for ``cfg`` (same exact-arithmetic normals and rounding as
    ``generate``), each from its own streams."""
    N, D = cfg.N, cfg.D
    br = _logit_block_rows(D)
    X = _normal_rows(N, D, cfg.seed, _TENSOR_X, threads, lambda z: z * cfg.x_std, cfg.dtype, block_rows=br)
    g = _normal_rows(1, D, cfg.seed, _TENSOR_GAMMA, 1, lambda z: 1.0 + z * cfg.gamma_std, cfg.dtype)
    dH = _normal_rows(N, D, cfg.seed, _TENSOR_DH, threads, lambda z: z * cfg.dh_std, cfg.dtype, block_rows=br)

    def t(a):
        return torch.from_numpy(a if cfg.dtype == "f32" else a.view(np.int16)).contiguous()
    return NormInputs(cfg, t(X), t(g).reshape(D), t(dH))


def _exp_neg(x: np.ndarray) -> np.ndarray:
    """exp(-x) for x >= 0 by exact power-of-two reduction and a Taylor series."""
    n = np.floor(x / _LN2)
    r = x - n * _LN2                       # in [0, ln 2) up to rounding
    er = _horner(-r, [1.0 / math.factorial(j) for j in range(20)])
    return np.ldexp(er, -n.astype(np.int64))


def with_labels(inp: Inputs, y: torch.Tensor) -> Inputs:
    """Same H and W with replaced labels (edge-case tests)."""
    return Inputs(replace(inp.cfg, name=inp.cfg.name + "_relabel"), inp.H, inp.W,
                  y.to(torch.int64).contiguous())


def with_weights_scaled(inp: Inputs, factor: float) -> Inputs:
    """Same inputs with W multiplied by ``factor`` (in fp32, then rounded to the workload's
    element type) -- large-logit tests."""
    if inp.cfg.dtype == "f32":
        W = torch.from_numpy(inp.W.numpy() * np.float32(factor))
    elif inp.cfg.dtype == "f16":
        w32 = inp.W.numpy().view(np.float16).astype(np.float32)
        W = torch.from_numpy(_rne_f16(w32 * np.float32(factor)).view(np.int16))
    else:
        w32 = (inp.W.numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        W = torch.from_numpy(_rne_bf16(w32 * np.float32(factor)).view(np.int16))
    return Inputs(replace(inp.cfg, name=inp.cfg.name + f"_wx{factor:g}"), inp.H, W.contiguous(),
                  inp.y)


def worked_example_inputs(total_tokens: int = 2048, d_model: int = 1024,
                          vocab_size: int = 32000, seed: int = 42):
    """The fp32 setup of the numpy walk-through on "Unsloth Architecture: 5x Faster LLM
    Training via Triton" (section "Step 2: Verification and Memory Profiling"): numpy's
    legacy generator seeded with 42 draws standard-normal hidden states, then standard-
    normal weights scaled by 0.02, then uniform integer targets.  Returned as fp32/int64
    numpy arrays."""
    rs = np.random.RandomState(seed)
    hidden = rs.randn(total_tokens, d_model).astype(np.float32)
    weight = rs.randn(vocab_size, d_model).astype(np.float32) * np.float32(0.02)
    targets = rs.randint(0, vocab_size, size=(total_tokens,))
    return hidden, weight, targets.astype(np.int64)
