"""MI355X-native fused, chunked GRPO policy loss.

The loss runs in libgrpo.so (hand-written HIP kernels for gfx950) behind the C
ABI declared in include/grpo.h; this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    GRPO_BF16,
    GRPO_F32,
    GRPO_FP8_E4M3,
    Fp8,
    dequantize_fp8,
    quantize_fp8,
    grpo_ref_logprobs_fp8,
    grpo_loss_fwd_fp8,
    grpo_loss_bwd_fp8,
    GRPO_OP_BWD,
    GRPO_OP_BWD_MIN,
    GRPO_OP_FWD,
    GRPO_OP_REF,
    AGG_SEQUENCE_MEAN,
    AGG_TOKEN_MEAN,
    KL_FORWARD,
    KL_REVERSE,
    KL_REVERSE_Q,
    GrpoError,
    auto_chunk,
    grpo_advantages,
    grpo_gemm_nt,
    grpo_loss_bwd,
    grpo_loss_fwd,
    grpo_ref_logprobs,
    grpo_timing_begin,
    grpo_timing_end,
    grpo_workspace_bytes,
    lib,
)
from .autograd import grpo_loss  # noqa: F401,E402
