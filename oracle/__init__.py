"""The CPU oracle of the mixture-of-experts layer.  TEST INFRASTRUCTURE ONLY: imported by
the tests, the smoke check and the benchmark's CPU-baseline leg, never by the GPU path."""
from .moe_oracle import (  # noqa: F401
    OracleOut, Routing, dequant_mxfp4, e2m1_value, e8m0_value, expert_weights, moe_forward,
    moe_forward_prenorm, prenorm_input, promote, rmsnorm,
    round_to_bf16, route, route_sigmoid_shared,
    route_softmax_topk, router_logits, sigmoid, silu, softmax, swiglu_expert,
    top_k_descending,
)
