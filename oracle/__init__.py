"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .lce_oracle import (  # noqa: F401
    AttentionGrads, AttentionResult, ForwardResult, attention_backward, attention_forward,
    attention_row_dot, attention_scores, causal_allowed, ShardPartials, backward, compact_valid, dlogits, embed_backward,
    embed_forward, forward, logits,
    logsumexp_rows, merge_partials, optimizer_step, round_to_bf16, rows_dH, rows_dW, rows_forward,
    shard_backward,
    shard_partials, target_logits, valid_mask,
)
