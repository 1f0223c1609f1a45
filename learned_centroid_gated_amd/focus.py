"""Python binding of the Focus C ABI with the same entry-point names.

Argument marshalling only: every step runs in libfocus.so's HIP kernels. torch provides device
memory (outputs and workspace come from its caching allocator) and the current stream.

Every wrapper checks, before any library call and in this order: that the tensors' shapes agree
with each other (a host-only check on `.shape`, so a mismatched call raises ValueError on any
machine), then dtype, device and contiguity. The library itself trusts the sizes it is given, so
these checks are what keeps a mismatched call from reading or writing past a device buffer.
"""
import torch

from . import _lib

_lib_call = _lib.call


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ------------------------------------------------------------------ host-only shape checks
def _tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")


def _dims(t, name, ndim):
    """t.shape of a tensor that must have `ndim` dimensions."""
    _tensor(t, name)
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _shape(t, name, shape):
    """Require t.shape == shape (entries None match any size)."""
    if t is None:
        return
    _tensor(t, name)
    got = tuple(t.shape)
    if len(got) != len(shape) or any(e is not None and g != e for g, e in zip(got, shape)):
        want = tuple("*" if e is None else e for e in shape)
        raise ValueError(f"{name} has shape {got}, expected {want}")


def _numel(t, name, count):
    """Require a tensor of exactly `count` elements (index lists accepted flat or with a
    leading batch dimension of 1)."""
    if t is None:
        return
    _tensor(t, name)
    if t.numel() != count:
        raise ValueError(f"{name} has {t.numel()} elements (shape {tuple(t.shape)}), expected {count}")


# ------------------------------------------------------------------ dtype / device checks
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


def _need_opt(t, name, dtype, device):
    if t is not None:
        _need(t, name, dtype, device)


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        if workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, expected {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _ws_bytes(ws):
    return ws.numel() * ws.element_size()


# ------------------------------------------------------------------ focus_assign
def focus_assign_workspace_size(n, d, d_g, K):
    return _lib.lib().focus_assign_workspace_size(n, d, d_g, K)


def focus_assign(hidden, w_g, centroids, top_k, sinkhorn_iters, groups=None, col_potential=None,
                 workspace=None, stream=None):
    """Group assignment: returns (groups [n, top_k] int32, col_potential [K] fp32)."""
    n, d = _dims(hidden, "hidden", 2)
    _, d_g = _dims(w_g, "w_g", 2)
    K, _ = _dims(centroids, "centroids", 2)
    _shape(w_g, "w_g", (d, d_g))
    _shape(centroids, "centroids", (K, d_g))
    _shape(groups, "groups", (n, top_k))
    _shape(col_potential, "col_potential", (K,))
    dev = hidden.device
    _need(hidden, "hidden", torch.float32)
    _need(w_g, "w_g", torch.float32, dev)
    _need(centroids, "centroids", torch.float32, dev)
    _need_opt(groups, "groups", torch.int32, dev)
    _need_opt(col_potential, "col_potential", torch.float32, dev)
    if groups is None:
        groups = torch.empty((n, top_k), dtype=torch.int32, device=dev)
    if col_potential is None:
        col_potential = torch.empty((K,), dtype=torch.float32, device=dev)
    ws = _workspace(focus_assign_workspace_size(n, d, d_g, K), dev, workspace)
    _lib_call("focus_assign", _ptr(hidden), _ptr(w_g), _ptr(centroids), n, d, d_g, K, top_k,
              sinkhorn_iters, _ptr(groups), _ptr(col_potential), _ptr(ws), _ws_bytes(ws),
              _stream(stream))
    return groups, col_potential


# ------------------------------------------------------------------ focus_bucket
def focus_bucket_workspace_size(batch, n, K, top_k):
    return _lib.lib().focus_bucket_workspace_size(batch, n, K, top_k)


def focus_bucket(groups, K, offsets=None, idx=None, slot=None, workspace=None, stream=None):
    """groups [n, top_k] or [batch, n, top_k] int32 -> (offsets, idx, slot) with a batch dim
    matching the input. Caller-given outputs may carry the batch dimension either way."""
    _tensor(groups, "groups")
    batched = groups.dim() == 3
    if groups.dim() not in (2, 3):
        raise ValueError(f"groups must be [n, top_k] or [batch, n, top_k], got {tuple(groups.shape)}")
    g3 = groups if batched else groups.unsqueeze(0)
    batch, n, top_k = g3.shape
    _numel(offsets, "offsets", batch * (K + 1))
    _numel(idx, "idx", batch * n * top_k)
    _numel(slot, "slot", batch * n * top_k)
    _need(groups, "groups", torch.int32)
    dev = groups.device
    for t, name in ((offsets, "offsets"), (idx, "idx"), (slot, "slot")):
        _need_opt(t, name, torch.int32, dev)
    if offsets is None:
        offsets = torch.empty((batch, K + 1), dtype=torch.int32, device=dev)
    if idx is None:
        idx = torch.empty((batch, n * top_k), dtype=torch.int32, device=dev)
    if slot is None:
        slot = torch.empty((batch, n, top_k), dtype=torch.int32, device=dev)
    ws = _workspace(focus_bucket_workspace_size(batch, n, K, top_k), dev, workspace)
    _lib_call("focus_bucket", _ptr(g3), batch, n, K, top_k, _ptr(offsets), _ptr(idx), _ptr(slot),
              _ptr(ws), _ws_bytes(ws), _stream(stream))
    if batched:
        return offsets, idx, slot
    # unbatched input: drop the batch dimension of outputs that carry one
    return (offsets[0] if offsets.dim() == 2 else offsets, idx[0] if idx.dim() == 2 else idx,
            slot[0] if slot.dim() == 3 else slot)


# ------------------------------------------------------------------ focus_attention
def focus_attention_workspace_size(n, Hq, Hkv, d_head, K, top_k):
    return _lib.lib().focus_attention_workspace_size(n, Hq, Hkv, d_head, K, top_k)


def _qkv_shapes(q, k, v):
    n, Hq, dh = _dims(q, "q", 3)
    _, Hkv, _ = _dims(k, "k", 3)
    _shape(k, "k", (n, Hkv, dh))
    _shape(v, "v", (n, Hkv, dh))
    return n, Hq, Hkv, dh


def focus_attention(q, k, v, groups, offsets, idx, slot, K, window, scale=0.0, out=None, lse=None,
                    workspace=None, stream=None):
    """Gated sparse causal attention: returns (out [n, Hq, dh] bf16, lse [n, Hq] fp32)."""
    n, Hq, Hkv, dh = _qkv_shapes(q, k, v)
    _, top_k = _dims(groups, "groups", 2)
    _shape(groups, "groups", (n, top_k))
    _numel(offsets, "offsets", K + 1)
    _numel(idx, "idx", n * top_k)
    _numel(slot, "slot", n * top_k)
    _shape(out, "out", (n, Hq, dh))
    _shape(lse, "lse", (n, Hq))
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((groups, "groups"), (offsets, "offsets"), (idx, "idx"), (slot, "slot")):
        _need(t, name, torch.int32, dev)
    _need_opt(out, "out", torch.bfloat16, dev)
    _need_opt(lse, "lse", torch.float32, dev)
    if out is None:
        out = torch.empty((n, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((n, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_attention_workspace_size(n, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_attention", _ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, dh, _ptr(groups),
              _ptr(offsets), _ptr(idx), _ptr(slot), K, top_k, int(window), float(scale), _ptr(out),
              _ptr(lse), _ptr(ws), _ws_bytes(ws), _stream(stream))
    return out, lse


# ------------------------------------------------------------------ focus_attention_asym
def focus_attention_asym_workspace_size(n, Hq, Hkv, d_head, K, top_k):
    return _lib.lib().focus_attention_asym_workspace_size(n, Hq, Hkv, d_head, K, top_k)


def focus_attention_asym(q, k, v, q_bucket, k_bucket, K, window, scale=0.0, out=None, lse=None,
                         workspace=None, stream=None):
    """Asymmetric top-k gated attention: q_bucket = focus_bucket(q_groups [n, top_k]) for the
    groups each token looks at, k_bucket = focus_bucket(k_group [n, 1]) for each token's single
    key group. Returns (out [n, Hq, dh] bf16, lse [n, Hq] fp32)."""
    n, Hq, Hkv, dh = _qkv_shapes(q, k, v)
    q_off, q_idx, q_slot = q_bucket
    k_off, k_idx, k_slot = k_bucket
    _tensor(q_slot, "q_slot")
    _tensor(k_slot, "k_slot")
    if q_slot.dim() < 2 or k_slot.dim() < 2:
        raise ValueError("q_slot and k_slot must be [n, top_k] (from focus_bucket)")
    top_k = q_slot.shape[-1]
    if k_slot.shape[-1] != 1:
        raise ValueError("k_bucket must come from one key group per token")
    _numel(q_off, "q_offsets", K + 1)
    _numel(q_idx, "q_idx", n * top_k)
    _numel(q_slot, "q_slot", n * top_k)
    _numel(k_off, "k_offsets", K + 1)
    _numel(k_idx, "k_idx", n)
    _numel(k_slot, "k_slot", n)
    _shape(out, "out", (n, Hq, dh))
    _shape(lse, "lse", (n, Hq))
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_off, "q_offsets"), (q_idx, "q_idx"), (q_slot, "q_slot"),
                    (k_off, "k_offsets"), (k_idx, "k_idx"), (k_slot, "k_slot")):
        _need(t, name, torch.int32, dev)
    _need_opt(out, "out", torch.bfloat16, dev)
    _need_opt(lse, "lse", torch.float32, dev)
    if out is None:
        out = torch.empty((n, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((n, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_attention_asym_workspace_size(n, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_attention_asym", _ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, dh, _ptr(q_off),
              _ptr(q_idx), _ptr(q_slot), top_k, _ptr(k_off), _ptr(k_idx), _ptr(k_slot), K,
              int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws), _ws_bytes(ws),
              _stream(stream))
    return out, lse


# ------------------------------------------------------------------ focus_bucket_append
def focus_bucket_append(new_groups, cache_len, offsets, idx, K, Lmax, offsets_out=None,
                        idx_out=None, stream=None):
    """Token cache_len[b] - 1 of every sequence joins its bucketed memberships: returns
    (offsets_out [B, K+1], idx_out [B, Lmax * top_k]) from the inputs for the shorter caches."""
    B, top_k = _dims(new_groups, "new_groups", 2)
    _shape(cache_len, "cache_len", (B,))
    _shape(offsets, "offsets", (B, K + 1))
    _shape(idx, "idx", (B, Lmax * top_k))
    _shape(offsets_out, "offsets_out", (B, K + 1))
    _shape(idx_out, "idx_out", (B, Lmax * top_k))
    dev = new_groups.device
    for t, name in ((new_groups, "new_groups"), (cache_len, "cache_len"), (offsets, "offsets"),
                    (idx, "idx")):
        _need(t, name, torch.int32, dev)
    _need_opt(offsets_out, "offsets_out", torch.int32, dev)
    _need_opt(idx_out, "idx_out", torch.int32, dev)
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
    n, Hq, Hkv, dh = _qkv_shapes(q, k, v)
    _, top_k = _dims(groups, "groups", 2)
    _shape(groups, "groups", (n, top_k))
    _shape(out, "out", (n, Hq, dh))
    _shape(lse, "lse", (n, Hq))
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, dev)
    _need(groups, "groups", torch.int32, dev)
    _need_opt(out, "out", torch.bfloat16, dev)
    _need_opt(lse, "lse", torch.float32, dev)
    if out is None:
        out = torch.empty((n, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((n, Hq), dtype=torch.float32, device=dev)
    _lib_call("focus_soft_attention", _ptr(q), _ptr(k), _ptr(v), n, Hq, Hkv, dh, _ptr(groups), K,
              top_k, int(window), float(lam), float(scale), _ptr(out), _ptr(lse), _stream(stream))
    return out, lse


# ------------------------------------------------------------------ soft-gated training
def focus_soft_train_workspace_size(n, d, d_g, K, Hq, sinkhorn_iters):
    return _lib.lib().focus_soft_train_workspace_size(n, d, d_g, K, Hq, sinkhorn_iters)


def _train_shapes(hidden, w_g, centroids, q, k, v):
    n, d = _dims(hidden, "hidden", 2)
    _, d_g = _dims(w_g, "w_g", 2)
    K, _ = _dims(centroids, "centroids", 2)
    _shape(w_g, "w_g", (d, d_g))
    _shape(centroids, "centroids", (K, d_g))
    nq, Hq, Hkv, dh = _qkv_shapes(q, k, v)
    if nq != n:
        raise ValueError(f"q has {nq} tokens, hidden has {n}")
    return n, d, d_g, K, Hq, Hkv, dh


def _train_need(hidden, w_g, centroids, q, k, v):
    dev = hidden.device
    for t, name in ((hidden, "hidden"), (w_g, "w_g"), (centroids, "centroids")):
        _need(t, name, torch.float32, dev)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, dev)
    return dev


def focus_soft_train_forward(hidden, w_g, centroids, sinkhorn_iters, q, k, v, window, lam,
                             scale=0.0, out=None, lse=None, workspace=None, stream=None):
    """Soft-gated training forward over every causal pair, the gate driven by the soft
    assignment (the balanced Sinkhorn plan): returns (out [n, Hq, dh] bf16, lse [n, Hq])."""
    n, d, d_g, K, Hq, Hkv, dh = _train_shapes(hidden, w_g, centroids, q, k, v)
    _shape(out, "out", (n, Hq, dh))
    _shape(lse, "lse", (n, Hq))
    dev = _train_need(hidden, w_g, centroids, q, k, v)
    _need_opt(out, "out", torch.bfloat16, dev)
    _need_opt(lse, "lse", torch.float32, dev)
    if out is None:
        out = torch.empty((n, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((n, Hq), dtype=torch.float32, device=dev)
    ws = _workspace(focus_soft_train_workspace_size(n, d, d_g, K, Hq, sinkhorn_iters), dev,
                    workspace)
    _lib_call("focus_soft_train_forward", _ptr(hidden), _ptr(w_g), _ptr(centroids), n, d, d_g, K,
              sinkhorn_iters, _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, dh, int(window), float(lam),
              float(scale), _ptr(out), _ptr(lse), _ptr(ws), _ws_bytes(ws), _stream(stream))
    return out, lse


def focus_soft_train_backward(hidden, w_g, centroids, sinkhorn_iters, q, k, v, out, lse, dout,
                              window, lam, scale=0.0, want_hidden=False, d_centroids=None,
                              d_w_g=None, d_hidden=None, workspace=None, stream=None):
    """Gradients of the soft-gated forward with respect to the centroids, the projection and
    (want_hidden or d_hidden given) the hidden states, from the forward's out and lse and the
    upstream gradient dout: returns (d_centroids [K, d_g], d_w_g [d, d_g], d_hidden or None)."""
    n, d, d_g, K, Hq, Hkv, dh = _train_shapes(hidden, w_g, centroids, q, k, v)
    for t, name, shape in ((out, "out", (n, Hq, dh)), (lse, "lse", (n, Hq)),
                           (dout, "dout", (n, Hq, dh))):
        _tensor(t, name)
        _shape(t, name, shape)
    _shape(d_centroids, "d_centroids", (K, d_g))
    _shape(d_w_g, "d_w_g", (d, d_g))
    _shape(d_hidden, "d_hidden", (n, d))
    dev = _train_need(hidden, w_g, centroids, q, k, v)
    _need(out, "out", torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    _need(dout, "dout", torch.bfloat16, dev)
    for t, name in ((d_centroids, "d_centroids"), (d_w_g, "d_w_g"), (d_hidden, "d_hidden")):
        _need_opt(t, name, torch.float32, dev)
    if d_centroids is None:
        d_centroids = torch.empty((K, d_g), dtype=torch.float32, device=dev)
    if d_w_g is None:
        d_w_g = torch.empty((d, d_g), dtype=torch.float32, device=dev)
    if d_hidden is None and want_hidden:
        d_hidden = torch.empty((n, d), dtype=torch.float32, device=dev)
    ws = _workspace(focus_soft_train_workspace_size(n, d, d_g, K, Hq, sinkhorn_iters), dev,
                    workspace)
    _lib_call("focus_soft_train_backward", _ptr(hidden), _ptr(w_g), _ptr(centroids), n, d, d_g,
              K, sinkhorn_iters, _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, dh, int(window), float(lam),
              float(scale), _ptr(out), _ptr(lse), _ptr(dout), _ptr(d_centroids), _ptr(d_w_g),
              _ptr(d_hidden), _ptr(ws), _ws_bytes(ws), _stream(stream))
    return d_centroids, d_w_g, d_hidden


# ------------------------------------------------------------------ focus_decode
def focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k):
    return _lib.lib().focus_decode_workspace_size(B, Lmax, Hq, Hkv, d_head, K, top_k)


def _decode_query_shapes(q, q_groups, out, lse):
    B, Hq, dh = _dims(q, "q", 3)
    _, top_k = _dims(q_groups, "q_groups", 2)
    _shape(q_groups, "q_groups", (B, top_k))
    _shape(out, "out", (B, Hq, dh))
    _shape(lse, "lse", (B, Hq))
    return B, Hq, dh, top_k


def _decode_outputs(B, Hq, dh, out, lse, dev):
    _need_opt(out, "out", torch.bfloat16, dev)
    _need_opt(lse, "lse", torch.float32, dev)
    if out is None:
        out = torch.empty((B, Hq, dh), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    return out, lse


def focus_decode(q, q_groups, k_cache, v_cache, cache_len, cache_groups, cache_offsets, cache_idx,
                 K, window, scale=0.0, out=None, lse=None, workspace=None, stream=None):
    """One token per sequence against its cache: returns (out [B, Hq, dh] bf16, lse [B, Hq])."""
    B, Hq, dh, top_k = _decode_query_shapes(q, q_groups, out, lse)
    _, Lmax, Hkv, _ = _dims(k_cache, "k_cache", 4)
    _shape(k_cache, "k_cache", (B, Lmax, Hkv, dh))
    _shape(v_cache, "v_cache", (B, Lmax, Hkv, dh))
    _shape(cache_len, "cache_len", (B,))
    _shape(cache_groups, "cache_groups", (B, Lmax, top_k))
    _numel(cache_offsets, "cache_offsets", B * (K + 1))
    _numel(cache_idx, "cache_idx", B * Lmax * top_k)
    dev = q.device
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_groups, "q_groups"), (cache_len, "cache_len"),
                    (cache_groups, "cache_groups"), (cache_offsets, "cache_offsets"),
                    (cache_idx, "cache_idx")):
        _need(t, name, torch.int32, dev)
    out, lse = _decode_outputs(B, Hq, dh, out, lse, dev)
    ws = _workspace(focus_decode_workspace_size(B, Lmax, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_decode", _ptr(q), _ptr(q_groups), _ptr(k_cache), _ptr(v_cache),
              _ptr(cache_len), _ptr(cache_groups), _ptr(cache_offsets), _ptr(cache_idx), B, Lmax,
              Hq, Hkv, dh, K, top_k, int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
              _ws_bytes(ws), _stream(stream))
    return out, lse


def focus_decode_noalloc(q, q_groups, k_cache, v_cache, cache_len, cache_groups, cache_offsets,
                         cache_idx, K, window, scale=0.0, out=None, lse=None, stream=None):
    """focus_decode without a workspace: the library's fixed per-GPU scratch serves the call
    (calls overlapping on one GPU race on it). Returns (out [B, Hq, dh] bf16, lse [B, Hq])."""
    B, Hq, dh, top_k = _decode_query_shapes(q, q_groups, out, lse)
    _, Lmax, Hkv, _ = _dims(k_cache, "k_cache", 4)
    _shape(k_cache, "k_cache", (B, Lmax, Hkv, dh))
    _shape(v_cache, "v_cache", (B, Lmax, Hkv, dh))
    _shape(cache_len, "cache_len", (B,))
    _shape(cache_groups, "cache_groups", (B, Lmax, top_k))
    _numel(cache_offsets, "cache_offsets", B * (K + 1))
    _numel(cache_idx, "cache_idx", B * Lmax * top_k)
    dev = q.device
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_groups, "q_groups"), (cache_len, "cache_len"),
                    (cache_groups, "cache_groups"), (cache_offsets, "cache_offsets"),
                    (cache_idx, "cache_idx")):
        _need(t, name, torch.int32, dev)
    out, lse = _decode_outputs(B, Hq, dh, out, lse, dev)
    _lib_call("focus_decode_noalloc", _ptr(q), _ptr(q_groups), _ptr(k_cache), _ptr(v_cache),
              _ptr(cache_len), _ptr(cache_groups), _ptr(cache_offsets), _ptr(cache_idx), B, Lmax,
              Hq, Hkv, dh, K, top_k, int(window), float(scale), _ptr(out), _ptr(lse),
              _stream(stream))
    return out, lse


def _paged_shapes(q, k_pages, v_pages, page_table, cache_len, cache_groups, top_k, B, dh):
    num_pages, page_size, Hkv, _ = _dims(k_pages, "k_pages", 4)
    _shape(k_pages, "k_pages", (num_pages, page_size, Hkv, dh))
    _shape(v_pages, "v_pages", (num_pages, page_size, Hkv, dh))
    _, pages_per_seq = _dims(page_table, "page_table", 2)
    _shape(page_table, "page_table", (B, pages_per_seq))
    Lmax = pages_per_seq * page_size
    _shape(cache_len, "cache_len", (B,))
    _shape(cache_groups, "cache_groups", (B, Lmax, top_k))
    return num_pages, page_size, Hkv, pages_per_seq, Lmax


def focus_decode_paged(q, q_groups, k_pages, v_pages, page_table, cache_len, cache_groups,
                       cache_offsets, cache_idx, K, window, scale=0.0, out=None, lse=None,
                       workspace=None, stream=None):
    """focus_decode over a paged cache: k_pages / v_pages [num_pages, page_size, Hkv, dh] bf16,
    page_table [B, pages_per_seq] int32; cache_groups [B, pages_per_seq * page_size, top_k].
    Returns (out [B, Hq, dh] bf16, lse [B, Hq])."""
    B, Hq, dh, top_k = _decode_query_shapes(q, q_groups, out, lse)
    num_pages, page_size, Hkv, pages_per_seq, Lmax = _paged_shapes(
        q, k_pages, v_pages, page_table, cache_len, cache_groups, top_k, B, dh)
    _numel(cache_offsets, "cache_offsets", B * (K + 1))
    _numel(cache_idx, "cache_idx", B * Lmax * top_k)
    dev = q.device
    for t, name in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_groups, "q_groups"), (page_table, "page_table"), (cache_len, "cache_len"),
                    (cache_groups, "cache_groups"), (cache_offsets, "cache_offsets"),
                    (cache_idx, "cache_idx")):
        _need(t, name, torch.int32, dev)
    out, lse = _decode_outputs(B, Hq, dh, out, lse, dev)
    ws = _workspace(focus_decode_workspace_size(B, Lmax, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_decode_paged", _ptr(q), _ptr(q_groups), _ptr(k_pages), _ptr(v_pages),
              num_pages, page_size, _ptr(page_table), pages_per_seq, _ptr(cache_len),
              _ptr(cache_groups), _ptr(cache_offsets), _ptr(cache_idx), B, Hq, Hkv, dh, K, top_k,
              int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws), _ws_bytes(ws),
              _stream(stream))
    return out, lse


# ------------------------------------------------------------------ group-slotted memberships
def focus_slots_from_bucket(offsets, idx, K, Lmax, group_cap, seg_len=None, seg_pos=None,
                            overflow=None, top_k=None, stream=None):
    """Rows of group_cap slots per (sequence, group) from a bucket (offsets [B, K+1], idx
    [B, Lmax * top_k]): returns (seg_len [B, K], seg_pos [B, K, group_cap], overflow [1]).
    top_k defaults to idx.shape[1] / Lmax, which must then divide exactly."""
    B, _ = _dims(offsets, "offsets", 2)
    _shape(offsets, "offsets", (B, K + 1))
    _, per = _dims(idx, "idx", 2)
    if top_k is None:
        if Lmax < 1 or per % Lmax != 0:
            raise ValueError(f"idx has {per} entries per sequence, not a multiple of Lmax={Lmax}")
        top_k = per // Lmax
    _shape(idx, "idx", (B, Lmax * top_k))
    _shape(seg_len, "seg_len", (B, K))
    _shape(seg_pos, "seg_pos", (B, K, group_cap))
    _numel(overflow, "overflow", 1)
    dev = offsets.device
    for t, name in ((offsets, "offsets"), (idx, "idx")):
        _need(t, name, torch.int32, dev)
    for t, name in ((seg_len, "seg_len"), (seg_pos, "seg_pos"), (overflow, "overflow")):
        _need_opt(t, name, torch.int32, dev)
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
    B, top_k = _dims(new_groups, "new_groups", 2)
    _shape(cache_len, "cache_len", (B,))
    _shape(seg_len, "seg_len", (B, K))
    _, _, gcap = _dims(seg_pos, "seg_pos", 3)
    _shape(seg_pos, "seg_pos", (B, K, gcap))
    _numel(overflow, "overflow", 1)
    dev = new_groups.device
    for t, name in ((new_groups, "new_groups"), (cache_len, "cache_len"), (seg_len, "seg_len"),
                    (seg_pos, "seg_pos"), (overflow, "overflow")):
        _need(t, name, torch.int32, dev)
    _lib_call("focus_slots_append", _ptr(new_groups), _ptr(cache_len), B, K, top_k, gcap,
              _ptr(seg_len), _ptr(seg_pos), _ptr(overflow), _stream(stream))


def focus_decode_slots(q, q_groups, k_pages, v_pages, page_table, cache_len, cache_groups, seg_len,
                       seg_pos, K, window, scale=0.0, out=None, lse=None, workspace=None,
                       stream=None):
    """focus_decode_paged with group-slotted cache memberships (seg_len [B, K], seg_pos
    [B, K, group_cap]). Returns (out [B, Hq, dh] bf16, lse [B, Hq])."""
    B, Hq, dh, top_k = _decode_query_shapes(q, q_groups, out, lse)
    num_pages, page_size, Hkv, pages_per_seq, Lmax = _paged_shapes(
        q, k_pages, v_pages, page_table, cache_len, cache_groups, top_k, B, dh)
    _shape(seg_len, "seg_len", (B, K))
    _, _, gcap = _dims(seg_pos, "seg_pos", 3)
    _shape(seg_pos, "seg_pos", (B, K, gcap))
    dev = q.device
    for t, name in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
        _need(t, name, torch.bfloat16, dev)
    for t, name in ((q_groups, "q_groups"), (page_table, "page_table"), (cache_len, "cache_len"),
                    (cache_groups, "cache_groups"), (seg_len, "seg_len"), (seg_pos, "seg_pos")):
        _need(t, name, torch.int32, dev)
    out, lse = _decode_outputs(B, Hq, dh, out, lse, dev)
    ws = _workspace(focus_decode_workspace_size(B, Lmax, Hq, Hkv, dh, K, top_k), dev, workspace)
    _lib_call("focus_decode_slots", _ptr(q), _ptr(q_groups), _ptr(k_pages), _ptr(v_pages),
              num_pages, page_size, _ptr(page_table), pages_per_seq, _ptr(cache_len),
              _ptr(cache_groups), _ptr(seg_len), _ptr(seg_pos), gcap, B, Hq, Hkv, dh,
              K, top_k, int(window), float(scale), _ptr(out), _ptr(lse), _ptr(ws),
              _ws_bytes(ws), _stream(stream))
    return out, lse
