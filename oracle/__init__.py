"""CPU oracle of the MoE layer forward (test infrastructure only; see
moe_oracle.py).  Nothing under the HIP package imports this."""
from .moe_oracle import (activated_weight_bytes, execution_budgets, forward, permute,  # noqa: F401
                         route, router_logits, select_experts, silu, swiglu_expert)
