"""focus_bucket_append on the GPU: appending the newest token's memberships to the bucket of the
shorter caches must give exactly the bucket of the full caches (bit-exact offsets, and index
lists equal up to the new totals), with ragged cache lengths, empty caches, dropped group ids
and several appends in a row."""
import numpy as np
import pytest
import torch

from gpu_util import bucket_expected, i32_dev, say
from synth import random_groups

pytestmark = pytest.mark.gpu


def _bucket_prefix(groups, lens, upto, K):
    """numpy stable-sort bucket of each sequence's tokens 0 .. lens[b] - 1 - upto (capacity Lmax)."""
    B, L, k = groups.shape
    offs, idxs = [], []
    for b in range(B):
        g = groups[b].copy()
        g[max(lens[b] - upto, 0):] = -1  # tokens past the prefix are dropped
        o, i, _ = bucket_expected(g, K)
        offs.append(o)
        idxs.append(i)
    return np.stack(offs), np.stack(idxs)


@pytest.mark.parametrize("B,L,K,k", [(1, 1, 1, 1), (3, 700, 8, 2), (5, 2049, 64, 2), (2, 300, 5, 3),
                                     (4, 513, 200, 4)])
def test_append_equals_rebucket(B, L, K, k):
    from learned_centroid_gated_amd import focus_bucket_append
    rng = np.random.default_rng(B * L + K)
    groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)]).astype(np.int32)
    if K > 4:  # a dropped id in some new tokens
        groups[0, -1, 0] = -1
    lens = np.array([L, 1, 0, L - 3, L // 2][:B], np.int32)
    lens = np.maximum(np.minimum(lens, L), 0)
    say(f"append B={B} L={L} K={K} top_k={k} lens={lens.tolist()}")
    off_in, idx_in = _bucket_prefix(groups, lens, 1, K)
    new_g = np.stack([groups[b, max(lens[b] - 1, 0)] for b in range(B)]).astype(np.int32)
    off_out, idx_out = focus_bucket_append(i32_dev(new_g), i32_dev(lens), i32_dev(off_in),
                                           i32_dev(idx_in), K, L)
    torch.cuda.synchronize()
    off_exp, idx_exp = _bucket_prefix(groups, lens, 0, K)
    oo, io = off_out.cpu().numpy(), idx_out.cpu().numpy()
    np.testing.assert_array_equal(oo, off_exp)
    for b in range(B):
        tot = off_exp[b, K]
        np.testing.assert_array_equal(io[b, :tot], idx_exp[b, :tot])


def test_append_steps_in_a_row():
    from learned_centroid_gated_amd import focus_bucket_append
    B, L, K, k, steps = 4, 1500, 32, 2, 6
    rng = np.random.default_rng(9)
    groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)]).astype(np.int32)
    lens = np.full(B, L - steps, np.int32)
    off_np, idx_np = _bucket_prefix(groups, lens, 0, K)
    off, idx = i32_dev(off_np), i32_dev(idx_np)
    off2, idx2 = torch.empty_like(off), torch.empty_like(idx)
    for s in range(steps):
        lens += 1
        new_g = np.stack([groups[b, lens[b] - 1] for b in range(B)]).astype(np.int32)
        focus_bucket_append(i32_dev(new_g), i32_dev(lens), off, idx, K, L, off2, idx2)
        off, off2, idx, idx2 = off2, off, idx2, idx  # ping-pong
    torch.cuda.synchronize()
    off_exp, idx_exp = _bucket_prefix(groups, lens, 0, K)
    np.testing.assert_array_equal(off.cpu().numpy(), off_exp)
    io = idx.cpu().numpy()
    for b in range(B):
        np.testing.assert_array_equal(io[b, :off_exp[b, K]], idx_exp[b, :off_exp[b, K]])
