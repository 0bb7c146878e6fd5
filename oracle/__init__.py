"""Float64 CPU oracle (test infrastructure only; see grpo_oracle)."""
from .grpo_oracle import (  # noqa: F401
    group_advantages,
    logits,
    logit_transform,
    logit_transform_slope,
    lse_and_target,
    token_logprobs,
    reverse_kl_k3,
    token_advantages,
    loss_forward,
    loss_coefficients,
    loss_backward,
)
