"""Scratch-memory accounting for the fused path.

The quantity the fused method avoids is the unfused logit tensor: N rows by V columns
of one element each ("Unsloth Architecture: 5x Faster LLM Training via Triton", the
Llama-3 memory box in "The Un-Fused Cross-Entropy Logit Disaster"; section 3 of
"Arquitectura interna de Unsloth y optimización en Triton").  The fused library's peak
scratch is exactly the workspace the caller hands it, so the report is that size as a
fraction of N * V * 2 bytes (the 16-bit logit tensor).
"""
from __future__ import annotations


def unfused_logit_bytes(n_tokens: int, vocab: int, elem_bytes: int = 2) -> int:
    """Bytes of a materialised [n_tokens, vocab] logit tensor."""
    return int(n_tokens) * int(vocab) * int(elem_bytes)


def scratch_fraction(workspace_bytes: int, n_tokens: int, vocab: int) -> float:
    """Workspace as a fraction of the 16-bit unfused logit tensor."""
    return workspace_bytes / unfused_logit_bytes(n_tokens, vocab, 2)
