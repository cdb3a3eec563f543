"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .flce_oracle import (IGNORE_INDEX, ce_from_logits, count_valid, dH_rows, dW_rows,
                          forward_backward, forward_stats, logit_grad, logits, logsumexp_rows)
from .norm_oracle import rmsnorm_backward, rmsnorm_forward, round_to

__all__ = ["IGNORE_INDEX", "ce_from_logits", "count_valid", "dH_rows", "dW_rows",
           "forward_backward", "forward_stats", "logit_grad", "logits", "logsumexp_rows",
           "rmsnorm_backward", "rmsnorm_forward", "round_to"]
