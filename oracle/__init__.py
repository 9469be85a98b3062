"""CPU oracle for the MoE sublayer and the FarSkip stack (test infrastructure only).

Only the test suite, the smoke check and the bench's CPU-baseline leg import this package.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (router_logits, select_topk, gate_scores, gate_weights, route, permute,
                         permute_rows, silu, mlp, grouped_mlp, shared_mlp, combine, moe_layer,
                         farskip_stack, moe_stack, attn_moe_stack, attn_moe_layer_stack, round_to_bf16,
                         topk_gap)
from . import mxfp8  # noqa: F401  (MXFP8 numbers of the FP8 expert products)
from . import moe_backward  # noqa: F401  (gradients of one MoE sublayer)
