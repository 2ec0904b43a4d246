"""Plain fp64 CPU oracle for the top-k routed MXFP4 MoE feed-forward layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package. The GPU library never calls it and shares no code with it.
"""
from .moe_oracle import (  # noqa: F401
    E2M1_BIAS,
    e2m1_value,
    e8m0_value,
    mxfp4_decode,
    bf16_to_f64,
    router_logits,
    topk_select,
    softmax_selected,
    route,
    permute,
    swiglu_clamped,
    expert_ffn,
    experts_from_arrays,
    moe_layer,
    MoEResult,
    rms_norm,
    f64_to_bf16_bits,
    moe_block,
    BlockResult,
    attention_decode,
)
