"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .flce_oracle import (IGNORE_INDEX, count_valid, dH_rows, dW_rows, forward_backward,
                          forward_stats, logit_grad, logits, logsumexp_rows)

__all__ = ["IGNORE_INDEX", "count_valid", "dH_rows", "dW_rows", "forward_backward",
           "forward_stats", "logit_grad", "logits", "logsumexp_rows"]
