"""CPU oracle (test infrastructure only; see muon_oracle.py)."""
from .muon_oracle import (  # noqa: F401
    NS_A, NS_B, NS_C, NS_STEPS, NS_EPS,
    bf16_round, bf16_bits, bf16_from_bits,
    momentum_ref, ns_ref, ns_ref_heads, split_heads, apply_ref,
    muon_step_ref, rel_fro,
    MINIMAX_LO, MINIMAX_MARGIN, LIMIT_QUINTIC, minimax_quintic, minimax_schedule,
    quintic_eval, sumsq_blocks,
)
