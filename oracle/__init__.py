"""CPU oracle (test infrastructure only; see lora_oracle's header)."""
from .lora_oracle import *  # noqa: F401,F403
from .lora_oracle import (Registry, PagedRegistry, OracleError, plan, lora_linear, lora_linear_sampled,
                          dequant_q4, round_to_bf16, Q4_GROUP,
                          base_linear, bf16_bits_to_f64, parity_metrics,
                          MAX_REL_TOL, RELL1_TOL)
