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
from .train_ref import (  # noqa: F401
    biased_attention_ref,
    sinkhorn_iterates_ref,
    soft_affinity_bias_ref,
    soft_assignment_ref,
    soft_train_backward_ref,
    soft_train_forward_ref,
    soft_train_forward_rows_ref,
)
