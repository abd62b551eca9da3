"""fp64 CPU oracle of the gpt-oss MoE FFN layer.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it. The product path never does.
"""
from .moe_oracle import (  # noqa: F401
    E2M1_TABLE,
    SWIGLU_ALPHA,
    SWIGLU_LIMIT,
    bf16_to_f64,
    dequant_mxfp4,
    e8m0_scale,
    expert_mlp,
    expert_parameter_shapes,
    expert_permutation,
    expert_weights,
    forward,
    route,
    router_logits,
    router_logits_f64,
    router_parameter_shapes,
    routing_weights,
    select_topk,
    swiglu,
)
