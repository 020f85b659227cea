"""libdfa: blockwise exact causal attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libdfa.so`` (hand-written HIP);
``binding`` marshals torch tensors into it.  ``inputs`` holds the seeded
synthetic input generator; ``timeline`` times each (rank, step) slot of a
schedule on its own (measured idle bubble).
"""
from .binding import (  # noqa: F401
    DFA_BF16, DFA_F32, DFA_FWD_FUSED, DFA_FWD_STEPWISE, DFA_OP_BWD, DFA_OP_FWD_FUSED,
    DFA_OP_FWD_STEPWISE, DFA_SCHED_BALANCED, DFA_SCHED_RING, DFA_SCHED_STRIPED, DfaError,
    dfa_attn_block_fwd, dfa_attn_bwd, dfa_attn_fwd, dfa_lse_merge, dfa_rope, dfa_schedule_balance,
    dfa_schedule_build, dfa_schedule_build_striped_blocks, dfa_status_string, dfa_workspace_size,
    make_desc,
)
