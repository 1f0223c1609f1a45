"""Focus oracle (test infrastructure only; see focus_ref's header)."""
from .focus_ref import (  # noqa: F401
    TIE_LOG,
    TIE_REL,
    allowed_keys_asym_ref,
    allowed_keys_ref,
    assign_ref,
    attention_rows_asym_ref,
    attention_rows_ref,
    decode_ref,
    owner_ref,
    pair_count_asym_ref,
    pair_count_ref,
    scores_ref,
    sinkhorn_ref,
    soft_gate_ref,
    topk_ref,
)
