"""CPU oracle of the MoE layer forward (test infrastructure only; see
moe_oracle.py).  Nothing under the HIP package imports this."""
from .moe_oracle import (execution_budgets, fold_pool, fold_token,  # noqa: F401
                         forward, forward_routes, kappa_balanced, path_forward, path_route, path_scores, path_sources,
                         permute, proxy_route, proxy_scores, route,
                         router_logits, select_experts, silu, swiglu_expert)
