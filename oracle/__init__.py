"""CPU oracle of the DFlash draft-proposal path: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The product path never imports it and shares no code with it.
"""
from .dflash_oracle import (  # noqa: F401
    acceptance_metrics, apply_rope, attention, build_query_block, greedy_verify,
    inject_context_kv, paged_slots, prepare_proposal_inputs, propose_block, rms_norm, round_bf16,
    round_f32, storage_rounding,
)
