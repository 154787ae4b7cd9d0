"""CPU oracle of the dropless MoE layer (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (SCORE_SIGMOID, SCORE_SOFTMAX, Routing, backward, backward_rows, capacity_layer, combine,
                         combine_backward, dense_gate_matrix, dense_layer, forward, group_of_rows, grouped_gemm,
                         grouped_wgrad, layer_rows, permute, route, router_logits, silu, swiglu,
                         swiglu_backward, to_f64, wgrad_entries)
