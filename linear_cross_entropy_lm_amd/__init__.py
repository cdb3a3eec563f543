"""Fused lm_head projection + cross-entropy loss, forward and backward, for AMD MI355X.

The compute path is the C-ABI library ``libflce.so`` (hand-written HIP for gfx950);
``binding`` marshals torch tensors into it.  ``inputs`` draws seeded synthetic
workloads and ``scratch`` does the memory accounting.  Importing this package does not
load the library; importing ``binding`` does, and fails loudly if it was not built.
"""
__all__ = ["binding", "inputs", "scratch"]
