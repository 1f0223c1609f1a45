"""Python binding of the Focus C ABI with the same entry-point names.

Argument marshalling only: every step runs in libfocus.so's HIP kernels. torch provides device
memory (outputs and workspace come from its caching allocator) and the current stream.
"""
import torch

from . import _lib

_lib_call = _lib.call


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (the Focus library has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ focus_assign
def focus_assign_workspace_size(n, d, d_g, K):
    return _lib.lib().focus_assign_workspace_size(n, d, d_g, K)


def focus_assign(hidden, w_g, centroids, top_k, sinkhorn_iters, groups=None, col_potential=None,
                 workspace=None, stream=None):
    """Group assignment: returns (groups [n, top_k] int32, col_potential [K] fp32)."""
    dev = hidden.device
    _need(hidden, "hidden", torch.float32)
    _need(w_g, "w_g", torch.float32, dev)
    _need(centroids, "centroids", torch.float32, dev)
    n, d = hidden.shape
    d_g = w_g.shape[1]
    K = centroids.shape[0]
    if w_g.shape[0] != d or centroids.shape[1] != d_g:
        raise ValueError("shape mismatch between hidden, w_g and centroids")
    if groups is None:
        groups = torch.empty((n, top_k), dtype=torch.int32, device=dev)
    if col_potential is None:
        col_potential = torch.empty((K,), dtype=torch.float32, device=dev)
    ws = _workspace(focus_assign_workspace_size(n, d, d_g, K), dev, workspace)
    _lib_call("focus_assign", _ptr(hidden), _ptr(w_g), _ptr(centroids), n, d, d_g, K, top_k,
              sinkhorn_iters, _ptr(groups), _ptr(col_potential), _ptr(ws),
              ws.numel() * ws.element_size(), _stream(stream))
    return groups, col_potential


# ------------------------------------------------------------------ focus_bucket
def focus_bucket_workspace_size(batch, n, K, top_k):
    return _lib.lib().focus_bucket_workspace_size(batch, n, K, top_k)


def focus_bucket(groups, K, offsets=None, idx=None, slot=None, workspace=None, stream=None):
    """groups [n, top_k] or [batch, n, top_k] int32 -> (offsets, idx, slot) with a batch dim
    matching the input."""
    _need(groups, "groups", torch.int32)
    dev = groups.device
    batched = groups.dim() == 3
    g3 = groups if batched else groups.unsqueeze(0)
    batch, n, top_k = g3.shape
    if offsets is None:
        offsets = torch.empty((batch, K + 1), dtype=torch.int32, device=dev)
    if idx is None:
        idx = torch.empty((batch, n * top_k), dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty((batch, n, top_k), dtype=torch.int32, device=dev)
    ws = _workspace(focus_bucket_workspace_size(batch, n, K, top_k), dev, workspace)
    _lib_call("focus_bucket", _ptr(g3), batch, n, K, top_k, _ptr(offsets), _ptr(idx), _ptr(slot),
              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if batched:
        return offsets, idx, slot
    return offsets[0], idx[0], slot[0]


# ------------------------------------------------------------------ focus_attention
def focus_attention_workspace_size(n, Hq, Hkv, d_head, K, top_k):
    return _lib.lib().focus_attention_workspace_size(n, Hq, Hkv, d_head, K, top_k)


def focus_attention(q, k, v, groups, offsets, idx, slot, K, window, scale=0.0, out=None, lse=None,
                    workspace=None, stream=None):
    """Gated sparse causal attention: returns (out [n, Hq, dh] bf16, lse [n, Hq] fp32)."""
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((groups, "groups"), (offsets, "offsets"), (idx, "idx"), (slot, "slot")):
        _need(t, name, torch.int32, dev)
    n, Hq, dh = q.shape
    Hkv = k.shape[1]
    top_k = groups.shape[-1]
    if out is None:
        out = torch.empty((n, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((n, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_attention_workspace_size(n, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_attention", _ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, dh, _ptr(groups),
              _ptr(offsets), _ptr(idx), _ptr(slot), K, top_k, int(window), float(scale), _ptr(out),
              _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    return out, lse


# ------------------------------------------------------------------ focus_attention_asym
def focus_attention_asym_workspace_size(n, Hq, Hkv, d_head, K, top_k):
    return _lib.lib().focus_attention_asym_workspace_size(n, Hq, Hkv, d_head, K, top_k)


def focus_attention_asym(q, k, v, q_bucket, k_bucket, K, window, scale=0.0, out=None, lse=None,
                         workspace=None, stream=None):
    """Asymmetric top-k gated attention: q_bucket = focus_bucket(q_groups [n, top_k]) for the
    groups each token looks at, k_bucket = focus_bucket(k_group [n, 1]) for each token's single
    key group. Returns (out [n, Hq, dh] bf16, lse [n, Hq] fp32)."""
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, dev)
    q_off, q_idx, q_slot = q_bucket
    k_off, k_idx, k_slot = k_bucket
    for t, name in ((q_off, "q_offsets"), (q_idx, "q_idx"), (q_slot, "q_slot"),
                    (k_off, "k_offsets"), (k_idx, "k_idx"), (k_slot, "k_slot")):
        _need(t, name, torch.int32, dev)
    n, Hq, dh = q.shape
    Hkv = k.shape[1]
    top_k = q_slot.shape[-1]
    if k_slot.shape[-1] != 1:
        raise ValueError("k_bucket must come from one key group per token")
    if out is None:
        out = torch.empty((n, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((n, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_attention_asym_workspace_size(n, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_attention_asym", _ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, dh, _ptr(q_off),
              _ptr(q_idx), _ptr(q_slot), top_k, _ptr(k_off), _ptr(k_idx), _ptr(k_slot), K,
              int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
              ws.numel() * ws.element_size(), _stream(stream))
    return out, lse


# ------------------------------------------------------------------ focus_bucket_append
def focus_bucket_append(new_groups, cache_len, offsets, idx, K, Lmax, offsets_out=None,
                        idx_out=None, stream=None):
    """Token cache_len[b] - 1 of every sequence joins its bucketed memberships: returns
    (offsets_out [B, K+1], idx_out [B, Lmax * top_k]) from the inputs for the shorter caches."""
    dev = new_groups.device
    for t, name in ((new_groups, "new_groups"), (cache_len, "cache_len"), (offsets, "offsets"),
                    (idx, "idx")):
        _need(t, name, torch.int32, dev)
    B, top_k = new_groups.shape
    if offsets_out is None:
        offsets_out = torch.empty_like(offsets)
    if idx_out is None:
        idx_out = torch.empty_like(idx)
    _lib_call("focus_bucket_append", _ptr(new_groups), _ptr(cache_len), B, int(Lmax), K, top_k,
              _ptr(offsets), _ptr(idx), _ptr(offsets_out), _ptr(idx_out), _stream(stream))
    return offsets_out, idx_out


# ------------------------------------------------------------------ focus_soft_attention
def focus_soft_attention(q, k, v, groups, K, window, lam, scale=0.0, out=None, lse=None,
                         stream=None):
    """Training-time soft-gated attention over all causal pairs, forward: returns
    (out [n, Hq, dh] bf16, lse [n, Hq] fp32)."""
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, dev)
    _need(groups, "groups", torch.int32, dev)
    n, Hq, dh = q.shape
    Hkv = k.shape[1]
    top_k = groups.shape[-1]
    if out is None:
        out = torch.empty((n, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((n, Hq), dtype=torch.float32, device=dev)
    _lib_call("focus_soft_attention", _ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, dh, _ptr(groups), K,
              top_k, int(window), float(lam), float(scale), _ptr(out), _ptr(lse), _stream(stream))
    return out, lse


# ------------------------------------------------------------------ focus_decode
def focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k):
    return _lib.lib().focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k)


def focus_decode(q, q_groups, k_cache, v_cache, cache_len, cache_groups, cache_offsets, cache_idx,
                 K, window, scale=0.0, out=None, lse=None, workspace=None, stream=None):
    """One token per sequence against its cache: returns (out [B, Hq, dh] bf16, lse [B, Hq])."""
    dev = q.device
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_groups, "q_groups"), (cache_len, "cache_len"),
                    (cache_groups, "cache_groups"), (cache_offsets, "cache_offsets"),
                    (cache_idx, "cache_idx")):
        _need(t, name, torch.int32, dev)
    B, Hq, dh = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    top_k = q_groups.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_decode_workspace_size(B, Lmax, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_decode", _ptr(q), _ptr(q_groups), _ptr(k_cache), _ptr(v_cache),
              _ptr(cache_len), _ptr(cache_groups), _ptr(cache_offsets), _ptr(cache_idx), B, Lmax,
              Hq, Hkv, dh, K, top_k, int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
              ws.numel() * ws.element_size(), _stream(stream))
    return out, lse


def focus_decode_paged(q, q_groups, k_pages, v_pages, page_table, cache_len, cache_groups,
                       cache_offsets, cache_idx, K, window, scale=0.0, out=None, lse=None,
                       workspace=None, stream=None):
    """focus_decode over a paged cache: k_pages / v_pages [num_pages, page_size, Hkv, dh] bf16,
    page_table [B, pages_per_seq] int32; cache_groups [B, pages_per_seq * page_size, top_k].
    Returns (out [B, Hq, dh] bf16, lse [B, Hq])."""
    dev = q.device
    for t, name in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_groups, "q_groups"), (page_table, "page_table"), (cache_len, "cache_len"),
                    (cache_groups, "cache_groups"), (cache_offsets, "cache_offsets"),
                    (cache_idx, "cache_idx")):
        _need(t, name, torch.int32, dev)
    B, Hq, dh = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    pages_per_seq = page_table.shape[1]
    Lmax = pages_per_seq * page_size
    top_k = q_groups.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_decode_workspace_size(B, Lmax, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_decode_paged", _ptr(q), _ptr(q_groups), _ptr(k_pages), _ptr(v_pages),
              num_pages, page_size, _ptr(page_table), pages_per_seq, _ptr(cache_len),
              _ptr(cache_groups), _ptr(cache_offsets), _ptr(cache_idx), B, Hq, Hkv, dh, K, top_k,
              int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
              ws.numel() * ws.element_size(), _stream(stream))
    return out, lse


# ------------------------------------------------------------------ group-slotted memberships
def focus_slots_from_bucket(offsets, idx, K, Lmax, group_cap, seg_len=None, seg_pos=None,
                            overflow=None, stream=None):
    """Rows of group_cap slots per (sequence, group) from a bucket (offsets [B, K+1], idx
    [B, Lmax * top_k]): returns (seg_len [B, K], seg_pos [B, K, group_cap], overflow [1])."""
    for t, name in ((offsets, "offsets"), (idx, "idx")):
        _need(t, name, torch.int32)
    dev = offsets.device
    B = offsets.shape[0]
    top_k = idx.shape[1] // Lmax
    if seg_len is None:
        seg_len = torch.empty((B, K), dtype=torch.int32, device=dev)
    if seg_pos is None:
        seg_pos = torch.empty((B, K, group_cap), dtype=torch.int32, device=dev)
    if overflow is None:
        overflow = torch.zeros((1,), dtype=torch.int32, device=dev)
    _lib_call("focus_slots_from_bucket", _ptr(offsets), _ptr(idx), B, int(Lmax), K, top_k,
              int(group_cap), _ptr(seg_len), _ptr(seg_pos), _ptr(overflow), _stream(stream))
    return seg_len, seg_pos, overflow


def focus_slots_append(new_groups, cache_len, seg_len, seg_pos, overflow, K, stream=None):
    """The newest token of every sequence joins the rows of its groups, in place."""
    for t, name in ((new_groups, "new_groups"), (cache_len, "cache_len"), (seg_len, "seg_len"),
                    (seg_pos, "seg_pos"), (overflow, "overflow")):
        _need(t, name, torch.int32)
    B, top_k = new_groups.shape
    _lib_call("focus_slots_append", _ptr(new_groups), _ptr(cache_len), B, K, top_k,
              seg_pos.shape[2], _ptr(seg_len), _ptr(seg_pos), _ptr(overflow), _stream(stream))


def focus_decode_slots(q, q_groups, k_pages, v_pages, page_table, cache_len, cache_groups, seg_len,
                       seg_pos, K, window, scale=0.0, out=None, lse=None, workspace=None,
                       stream=None):
    """focus_decode_paged with group-slotted cache memberships (seg_len [B, K], seg_pos
    [B, K, group_cap]). Returns (out [B, Hq, dh] bf16, lse [B, Hq])."""
    dev = q.device
    for t, name in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_groups, "q_groups"), (page_table, "page_table"), (cache_len, "cache_len"),
                    (cache_groups, "cache_groups"), (seg_len, "seg_len"), (seg_pos, "seg_pos")):
        _need(t, name, torch.int32, dev)
    B, Hq, dh = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    pages_per_seq = page_table.shape[1]
    Lmax = pages_per_seq * page_size
    top_k = q_groups.shape[-1]
    if out is None:
        out = torch.empty((B, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_decode_workspace_size(B, Lmax, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_decode_slots", _ptr(q), _ptr(q_groups), _ptr(k_pages), _ptr(v_pages),
              num_pages, page_size, _ptr(page_table), pages_per_seq, _ptr(cache_len),
              _ptr(cache_groups), _ptr(seg_len), _ptr(seg_pos), seg_pos.shape[2], B, Hq, Hkv, dh,
              K, top_k, int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
              ws.numel() * ws.element_size(), _stream(stream))
    return out, lse
