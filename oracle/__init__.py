"""fp64 CPU oracle of the Bailing/Ling MoE FFN layer -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .moe_oracle import (OracleConfig, dequant_u8, expert_counts, expert_slots, forward,
                         route, route_token, silu, swiglu_mlp, to_f64)

__all__ = ["OracleConfig", "dequant_u8", "expert_counts", "expert_slots", "forward", "route",
           "route_token", "silu", "swiglu_mlp", "to_f64"]
