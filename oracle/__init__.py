"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .lce_oracle import (  # noqa: F401
    ForwardResult, backward, compact_valid, dlogits, forward, logits,
    logsumexp_rows, rows_dH, rows_dW, rows_forward, target_logits, valid_mask,
)
