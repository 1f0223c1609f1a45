"""The Python binding's host-side checks: consistent host tensors are refused as not being on
the device, and a call whose tensors disagree in shape is refused with ValueError before the
library is called (so a mismatch never becomes an out-of-bounds device access). Runs on the
CPU: every check here happens before any device work."""
import pytest
import torch

import learned_centroid_gated_amd as F

# one consistent set of shapes: n tokens, Hq/Hkv heads, head size dh, K groups, top_k
n, Hq, Hkv, dh, K, k = 8, 4, 2, 64, 4, 2
B, L, page, pps, cap = 3, 16, 4, 4, 8


def bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def attn_args(**over):
    a = dict(q=bf(n, Hq, dh), k=bf(n, Hkv, dh), v=bf(n, Hkv, dh), groups=i32(n, k),
             offsets=i32(K + 1), idx=i32(n * k), slot=i32(n, k), K=K, window=2)
    a.update(over)
    return a


def asym_args(**over):
    a = dict(q=bf(n, Hq, dh), k=bf(n, Hkv, dh), v=bf(n, Hkv, dh),
             q_bucket=(i32(K + 1), i32(n * k), i32(n, k)), k_bucket=(i32(K + 1), i32(n), i32(n, 1)),
             K=K, window=2)
    a.update(over)
    return a


def soft_args(**over):
    a = dict(q=bf(n, Hq, dh), k=bf(n, Hkv, dh), v=bf(n, Hkv, dh), groups=i32(n, k), K=K,
             window=2, lam=1.0)
    a.update(over)
    return a


def assign_args(**over):
    a = dict(hidden=f32(n, 16), w_g=f32(16, 8), centroids=f32(K, 8), top_k=k, sinkhorn_iters=2)
    a.update(over)
    return a


def append_args(**over):
    a = dict(new_groups=i32(B, k), cache_len=i32(B), offsets=i32(B, K + 1), idx=i32(B, L * k),
             K=K, Lmax=L)
    a.update(over)
    return a


def decode_args(**over):
    a = dict(q=bf(B, Hq, dh), q_groups=i32(B, k), k_cache=bf(B, L, Hkv, dh),
             v_cache=bf(B, L, Hkv, dh), cache_len=i32(B), cache_groups=i32(B, L, k),
             cache_offsets=i32(B, K + 1), cache_idx=i32(B, L * k), K=K, window=4)
    a.update(over)
    return a


def paged_args(**over):
    a = dict(q=bf(B, Hq, dh), q_groups=i32(B, k), k_pages=bf(10, page, Hkv, dh),
             v_pages=bf(10, page, Hkv, dh), page_table=i32(B, pps), cache_len=i32(B),
             cache_groups=i32(B, pps * page, k), cache_offsets=i32(B, K + 1),
             cache_idx=i32(B, pps * page * k), K=K, window=4)
    a.update(over)
    return a


def slots_decode_args(**over):
    a = dict(q=bf(B, Hq, dh), q_groups=i32(B, k), k_pages=bf(10, page, Hkv, dh),
             v_pages=bf(10, page, Hkv, dh), page_table=i32(B, pps), cache_len=i32(B),
             cache_groups=i32(B, pps * page, k), seg_len=i32(B, K), seg_pos=i32(B, K, cap), K=K,
             window=4)
    a.update(over)
    return a


def from_bucket_args(**over):
    a = dict(offsets=i32(B, K + 1), idx=i32(B, L * k), K=K, Lmax=L, group_cap=cap)
    a.update(over)
    return a


def slots_append_args(**over):
    a = dict(new_groups=i32(B, k), cache_len=i32(B), seg_len=i32(B, K), seg_pos=i32(B, K, cap),
             overflow=i32(1), K=K)
    a.update(over)
    return a


def train_fwd_args(**over):
    a = dict(hidden=f32(n, 16), w_g=f32(16, 8), centroids=f32(K, 8), sinkhorn_iters=2,
             q=bf(n, Hq, dh), k=bf(n, Hkv, dh), v=bf(n, Hkv, dh), window=2, lam=3.0)
    a.update(over)
    return a


def train_bwd_args(**over):
    a = train_fwd_args()
    a.update(out=bf(n, Hq, dh), lse=f32(n, Hq), dout=bf(n, Hq, dh))
    a.update(over)
    return a


WRAPPERS = {
    "focus_soft_train_forward": train_fwd_args, "focus_soft_train_backward": train_bwd_args,
    "focus_assign": assign_args, "focus_bucket": lambda **o: {"groups": i32(n, k), "K": K, **o},
    "focus_attention": attn_args, "focus_attention_asym": asym_args,
    "focus_soft_attention": soft_args, "focus_bucket_append": append_args,
    "focus_decode": decode_args, "focus_decode_paged": paged_args,
    "focus_decode_slots": slots_decode_args, "focus_slots_from_bucket": from_bucket_args,
    "focus_slots_append": slots_append_args,
}


@pytest.mark.parametrize("name", sorted(WRAPPERS))
def test_consistent_host_tensors_are_refused_as_not_on_the_device(name):
    with pytest.raises(ValueError, match="device tensor"):
        getattr(F, name)(**WRAPPERS[name]())


MISMATCHES = [
    # (wrapper, overrides, what the message names)
    ("focus_assign", dict(w_g=f32(15, 8)), "w_g"),
    ("focus_assign", dict(centroids=f32(K, 9)), "centroids"),
    ("focus_assign", dict(groups=i32(n, k + 1)), "groups"),
    ("focus_assign", dict(col_potential=f32(K + 1)), "col_potential"),
    ("focus_bucket", dict(offsets=i32(K)), "offsets"),
    ("focus_bucket", dict(idx=i32(n * k - 1)), "idx"),
    ("focus_bucket", dict(slot=i32(n, k + 1)), "slot"),
    ("focus_attention", dict(k=bf(n - 1, Hkv, dh)), "k"),
    ("focus_attention", dict(v=bf(n, Hkv, dh // 2)), "v"),
    ("focus_attention", dict(groups=i32(n + 1, k)), "groups"),
    ("focus_attention", dict(offsets=i32(K)), "offsets"),
    ("focus_attention", dict(idx=i32(n * k + 4)), "idx"),
    ("focus_attention", dict(slot=i32(n, k + 1)), "slot"),
    ("focus_attention", dict(out=bf(n, Hq, dh + 8)), "out"),
    ("focus_attention", dict(lse=f32(n, Hq - 1)), "lse"),
    ("focus_attention_asym", dict(k_bucket=(i32(K + 1), i32(n - 1), i32(n, 1))), "k_idx"),
    ("focus_attention_asym", dict(q_bucket=(i32(K + 2), i32(n * k), i32(n, k))), "q_offsets"),
    ("focus_attention_asym", dict(k_bucket=(i32(K + 1), i32(n), i32(n, 2))), "one key group"),
    ("focus_attention_asym", dict(q=bf(n + 1, Hq, dh)), "k"),
    ("focus_soft_attention", dict(groups=i32(n - 1, k)), "groups"),
    ("focus_soft_attention", dict(lse=f32(n + 1, Hq)), "lse"),
    ("focus_bucket_append", dict(cache_len=i32(B + 1)), "cache_len"),
    ("focus_bucket_append", dict(idx=i32(B, L * k - 1)), "idx"),
    ("focus_bucket_append", dict(offsets=i32(B, K)), "offsets"),
    ("focus_bucket_append", dict(offsets_out=i32(B - 1, K + 1)), "offsets_out"),
    ("focus_decode", dict(k_cache=bf(B + 1, L, Hkv, dh)), "k_cache"),
    ("focus_decode", dict(v_cache=bf(B, L - 1, Hkv, dh)), "v_cache"),
    ("focus_decode", dict(cache_groups=i32(B, L, k + 1)), "cache_groups"),
    ("focus_decode", dict(cache_idx=i32(B, L * k - 2)), "cache_idx"),
    ("focus_decode", dict(cache_offsets=i32(B, K)), "cache_offsets"),
    ("focus_decode", dict(cache_len=i32(B - 1)), "cache_len"),
    ("focus_decode", dict(q_groups=i32(B, k + 1)), "cache_groups"),
    ("focus_decode_paged", dict(page_table=i32(B + 1, pps)), "page_table"),
    ("focus_decode_paged", dict(v_pages=bf(9, page, Hkv, dh)), "v_pages"),
    ("focus_decode_paged", dict(cache_groups=i32(B, L + 1, k)), "cache_groups"),
    ("focus_decode_paged", dict(cache_idx=i32(B, pps * page * k + 1)), "cache_idx"),
    ("focus_decode_slots", dict(seg_pos=i32(B, K + 1, cap)), "seg_pos"),
    ("focus_decode_slots", dict(seg_len=i32(B, K - 1)), "seg_len"),
    ("focus_decode_slots", dict(out=bf(B, Hq, dh - 1)), "out"),
    ("focus_slots_from_bucket", dict(idx=i32(B, L * k + 3)), "multiple of Lmax"),
    ("focus_slots_from_bucket", dict(offsets=i32(B, K + 3)), "offsets"),
    ("focus_slots_from_bucket", dict(seg_pos=i32(B, K, cap + 1)), "seg_pos"),
    ("focus_slots_from_bucket", dict(top_k=3), "idx"),
    ("focus_slots_append", dict(seg_len=i32(B, K + 1)), "seg_len"),
    ("focus_slots_append", dict(cache_len=i32(B + 2)), "cache_len"),
    ("focus_slots_append", dict(overflow=i32(2)), "overflow"),
    ("focus_soft_train_forward", dict(q=bf(n + 1, Hq, dh)), "k"),
    ("focus_soft_train_forward", dict(hidden=f32(n + 1, 16)), "tokens"),
    ("focus_soft_train_forward", dict(centroids=f32(K, 9)), "centroids"),
    ("focus_soft_train_forward", dict(lse=f32(n, Hq + 1)), "lse"),
    ("focus_soft_train_backward", dict(dout=bf(n, Hq, dh + 8)), "dout"),
    ("focus_soft_train_backward", dict(lse=f32(n - 1, Hq)), "lse"),
    ("focus_soft_train_backward", dict(d_w_g=f32(15, 8)), "d_w_g"),
    ("focus_soft_train_backward", dict(d_hidden=f32(n, 17)), "d_hidden"),
]


@pytest.mark.parametrize("name,over,what", MISMATCHES)
def test_mismatched_shapes_are_refused_before_the_library(name, over, what):
    with pytest.raises(ValueError, match=what):
        getattr(F, name)(**WRAPPERS[name](**over))


def test_every_wrapper_has_a_mismatch_case():
    assert {m[0] for m in MISMATCHES} == set(WRAPPERS)
