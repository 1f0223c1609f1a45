"""ctypes view of libfocus.so: the entry points declared in include/focus.h, nothing else.

Loading fails loudly when the library has not been built; there is no fallback path.
"""
import ctypes
import os

# FOCUS_LIB_PATH selects another build of the same library (the host-sanitized one in tests)
LIB_PATH = os.environ.get("FOCUS_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfocus.so")

c_i64, c_int, c_sz, c_f, c_p = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

SIGNATURES = {
    "focus_status_string": (ctypes.c_char_p, [c_int]),
    "focus_version": (c_int, []),
    "focus_assign_workspace_size": (c_sz, [c_i64, c_int, c_int, c_int]),
    "focus_assign": (c_int, [c_p, c_p, c_p, c_i64, c_int, c_int, c_int, c_int, c_int, c_p, c_p,
                             c_p, c_sz, c_p]),
    "focus_bucket_workspace_size": (c_sz, [c_int, c_i64, c_int, c_int]),
    "focus_bucket": (c_int, [c_p, c_int, c_i64, c_int, c_int, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "focus_bucket_append": (c_int, [c_p, c_p, c_int, c_i64, c_int, c_int, c_p, c_p, c_p, c_p, c_p]),
    "focus_attention_workspace_size": (c_sz, [c_i64, c_int, c_int, c_int, c_int, c_int]),
    "focus_attention": (c_int, [c_p, c_p, c_p, c_i64, c_int, c_int, c_int, c_p, c_p, c_p, c_p,
                                c_int, c_int, c_i64, c_f, c_p, c_p, c_p, c_sz, c_p]),
    "focus_attention_ex": (c_int, [c_p, c_p, c_p, c_i64, c_int, c_int, c_int, c_p, c_p, c_p, c_p,
                                   c_int, c_int, c_i64, c_f, c_p, c_p, c_p, c_sz, c_p,
                                   ctypes.POINTER(c_p), c_int]),
    "focus_attention_asym_workspace_size": (c_sz, [c_i64, c_int, c_int, c_int, c_int, c_int]),
    "focus_attention_asym": (c_int, [c_p, c_p, c_p, c_i64, c_int, c_int, c_int, c_p, c_p, c_p,
                                     c_int, c_p, c_p, c_p, c_int, c_i64, c_f, c_p, c_p, c_p,
                                     c_sz, c_p]),
    "focus_soft_attention": (c_int, [c_p, c_p, c_p, c_i64, c_int, c_int, c_int, c_p, c_int, c_int,
                                     c_i64, c_f, c_f, c_p, c_p, c_p]),
    "focus_decode_workspace_size": (c_sz, [c_int, c_i64, c_int, c_int, c_int, c_int, c_int]),
    "focus_slots_from_bucket": (c_int, [c_p, c_p, c_int, c_i64, c_int, c_int, c_int, c_p, c_p,
                                        c_p, c_p]),
    "focus_slots_append": (c_int, [c_p, c_p, c_int, c_int, c_int, c_int, c_p, c_p, c_p, c_p]),
    "focus_decode_slots": (c_int, [c_p, c_p, c_p, c_p, c_i64, c_int, c_p, c_i64, c_p, c_p, c_p,
                                   c_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_i64,
                                   c_f, c_p, c_p, c_p, c_sz, c_p]),
    "focus_decode_paged": (c_int, [c_p, c_p, c_p, c_p, c_i64, c_int, c_p, c_i64, c_p, c_p, c_p,
                                   c_p, c_int, c_int, c_int, c_int, c_int, c_int, c_i64, c_f,
                                   c_p, c_p, c_p, c_sz, c_p]),
    "focus_decode": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_int, c_i64, c_int, c_int,
                             c_int, c_int, c_int, c_i64, c_f, c_p, c_p, c_p, c_sz, c_p]),
    "focus_soft_train_workspace_size": (c_sz, [c_i64, c_int, c_int, c_int, c_int, c_int]),
    "focus_soft_train_forward": (c_int, [c_p, c_p, c_p, c_i64, c_int, c_int, c_int, c_int, c_p,
                                         c_p, c_p, c_int, c_int, c_int, c_i64, c_f, c_f, c_p, c_p,
                                         c_p, c_sz, c_p]),
    "focus_soft_train_backward": (c_int, [c_p, c_p, c_p, c_i64, c_int, c_int, c_int, c_int, c_p,
                                          c_p, c_p, c_int, c_int, c_int, c_i64, c_f, c_f, c_p,
                                          c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]),
    "focus_decode_noalloc_scratch_bytes": (c_sz, []),
    "focus_decode_noalloc": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_int, c_i64, c_int,
                                     c_int, c_int, c_int, c_int, c_i64, c_f, c_p, c_p, c_p]),
}

_lib = None


class FocusError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m learned_centroid_gated_amd.build` (needs ROCm hipcc)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().focus_status_string(status).decode()


def call(name, *args):
    """Call entry point `name`; raise FocusError on a non-zero status."""
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise FocusError(name, st)
    return st
