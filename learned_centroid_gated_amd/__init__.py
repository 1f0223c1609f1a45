"""Focus (learned centroid-gated sparse attention) inference path for AMD MI355X (gfx950).

The compute lives in libfocus.so (hand-written HIP kernels behind the C ABI of
include/focus.h); this package only marshals arguments to it.
"""
from .focus import (  # noqa: F401
    focus_assign,
    focus_assign_workspace_size,
    focus_attention,
    focus_attention_asym,
    focus_attention_asym_workspace_size,
    focus_attention_workspace_size,
    focus_bucket,
    focus_bucket_append,
    focus_bucket_workspace_size,
    focus_decode,
    focus_decode_noalloc,
    focus_decode_paged,
    focus_decode_slots,
    focus_slots_append,
    focus_slots_from_bucket,
    focus_decode_workspace_size,
    focus_soft_attention,
    focus_soft_train_backward,
    focus_soft_train_forward,
    focus_soft_train_workspace_size,
)
from ._lib import LIB_PATH, FocusError, lib, status_string  # noqa: F401
