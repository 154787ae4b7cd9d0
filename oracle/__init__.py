"""CPU oracle of the dropless MoE layer (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (SCORE_SIGMOID, SCORE_SOFTMAX, Routing, backward, capacity_layer, combine, combine_backward,
                         dense_gate_matrix, dense_layer, forward, grouped_gemm, grouped_wgrad,
                         permute, route, router_logits, silu, swiglu, swiglu_backward, to_f64)
