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

Generation is blockwise: every 4096-row block of a tensor has its own torch CPU
generator whose seed is a fixed function of (config seed, tensor id, block index),
so blocks can be filled in parallel threads and the result does not depend on the
thread count.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch

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
    dtype: str  # "f32" or "bf16"
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


# The five workloads.  The tiny fp32 case is the one the oracle finishes instantly;
# the other four are shaped like the Llama-2, Mistral, Llama-3 and Qwen-2.5 heads.
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
}


def case(N: int, D: int, V: int, dtype: str = "bf16", seed: int = 7, **kw) -> Config:
    """A small ad-hoc workload (tests): same distributions, free sizes."""
    base = dict(h_dist="rms", ignore_frac=0.05, ignore_layout="random", batch=1, seq=N)
    base.update(kw)
    return Config(f"case_N{N}_D{D}_V{V}_{dtype}_s{seed}", N=N, D=D, V=V, dtype=dtype,
                  seed=seed, **base)


# ---------------------------------------------------------------------------------
# bf16 bit-pattern helpers (format conversion only)
# ---------------------------------------------------------------------------------

def f32_to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even fp32 -> bf16, returned as int16 bit patterns."""
    return x.to(torch.bfloat16).view(torch.int16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (int16/uint16) to fp64."""
    u = bits.view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _block_seed(seed: int, tensor: int, block: int) -> int:
    return (seed * 1_000_003 + tensor * 10_007 + block * 97 + 12345) % (2**63 - 1)


def _fill_normal(out: torch.Tensor, seed: int, tensor: int, std: float, threads: int) -> None:
    rows = out.shape[0]
    nblk = (rows + _BLOCK_ROWS - 1) // _BLOCK_ROWS

    def fill(b: int) -> None:
        g = torch.Generator().manual_seed(_block_seed(seed, tensor, b))
        out[b * _BLOCK_ROWS:min(rows, (b + 1) * _BLOCK_ROWS)].normal_(0.0, std, generator=g)

    if nblk == 1 or threads <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))


@dataclass
class Inputs:
    """Generated inputs.  ``H`` and ``W`` are fp32 tensors for f32 workloads and int16
    bf16 bit patterns for bf16 workloads; ``y`` is int64 with IGNORE_INDEX rows."""

    cfg: Config
    H: torch.Tensor
    W: torch.Tensor
    y: torch.Tensor
    _digest: str | None = field(default=None, repr=False)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.cfg.dtype == "f32" else torch.bfloat16

    def h64(self) -> np.ndarray:
        return self._widen(self.H)

    def w64(self) -> np.ndarray:
        return self._widen(self.W)

    def y64(self) -> np.ndarray:
        return self.y.numpy().astype(np.int64)

    def _widen(self, t: torch.Tensor) -> np.ndarray:
        if self.cfg.dtype == "f32":
            return t.numpy().astype(np.float64)
        return bf16_bits_to_f64(t.numpy())

    def device_tensors(self, device) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """(H, W, y) on ``device`` in the workload's element type."""
        if self.cfg.dtype == "f32":
            H, W = self.H, self.W
        else:
            H, W = self.H.view(torch.bfloat16), self.W.view(torch.bfloat16)
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


def generate(cfg: Config, threads: int = 8) -> Inputs:
    """Draw H, W, labels and the ignore mask (in that order) for ``cfg``."""
    N, D, V = cfg.N, cfg.D, cfg.V
    H = torch.empty(N, D, dtype=torch.float32)
    _fill_normal(H, cfg.seed, _TENSOR_H, 1.0, threads)
    if cfg.h_dist == "rms":
        # unit-RMS rows: h / sqrt(mean(h^2)), gamma = 1, eps = 0, in fp32
        H.div_(H.square().mean(dim=1, keepdim=True).sqrt_())
    elif cfg.h_dist != "normal":
        raise ValueError(cfg.h_dist)
    W = torch.empty(V, D, dtype=torch.float32)
    _fill_normal(W, cfg.seed, _TENSOR_W, cfg.w_std, threads)

    g = torch.Generator().manual_seed(_block_seed(cfg.seed, _TENSOR_LABELS, 0))
    if cfg.label_dist == "uniform":
        y = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    elif cfg.label_dist == "zipf":
        perm = torch.randperm(V, generator=g)
        ranks = torch.arange(1, V + 1, dtype=torch.float64)
        p = ranks.pow(-cfg.zipf_s)
        k = torch.multinomial(p / p.sum(), N, replacement=True, generator=g)
        y = perm[k]
    else:
        raise ValueError(cfg.label_dist)
    k_ign = cfg.n_ignored
    if k_ign:
        if cfg.ignore_layout == "random":
            idx = torch.randperm(N, generator=g)[:k_ign]
        elif cfg.ignore_layout == "tail":
            idx = torch.arange(N - k_ign, N)
        else:
            raise ValueError(cfg.ignore_layout)
        y[idx] = IGNORE_INDEX

    if cfg.dtype == "bf16":
        H, W = f32_to_bf16_bits(H), f32_to_bf16_bits(W)
    elif cfg.dtype != "f32":
        raise ValueError(cfg.dtype)
    return Inputs(cfg, H.contiguous(), W.contiguous(), y.contiguous())


def with_labels(inp: Inputs, y: torch.Tensor) -> Inputs:
    """Same H and W with replaced labels (edge-case tests)."""
    return Inputs(replace(inp.cfg, name=inp.cfg.name + "_relabel"), inp.H, inp.W,
                  y.to(torch.int64).contiguous())


def with_weights_scaled(inp: Inputs, factor: float) -> Inputs:
    """Same inputs with W multiplied by ``factor`` before rounding (large-logit tests)."""
    if inp.cfg.dtype == "f32":
        W = inp.W * factor
    else:
        W = f32_to_bf16_bits(inp.W.view(torch.bfloat16).float() * factor)
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
