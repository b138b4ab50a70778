"""CPU oracle of the sparse MoE layer forward (test infrastructure only).

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (as_f64, capacity, router_logits, softmax, topk, route_topk,  # noqa: F401
                         splitmix64, route_rre, dispatch, gather, act_fn, expert_hidden,
                         expert_apply, is_glu,
                         expert_ffn, combine, route, forward, forward_rows,
                         route_and_dispatch, aux_loss)
