"""CPU oracle (test infrastructure only; see attention_ref)."""
from .attention_ref import (  # noqa: F401
    State,
    attention_bwd_ref,
    attention_ref,
    block_state,
    empty_state,
    finalize_state,
    kv_head,
    merge_partials,
    merge_states,
    online_blocked_ref,
)
