"""focus_bucket on the GPU: bit-exact against a stable sort of the memberships by group."""
import numpy as np
import pytest
import torch

from gpu_util import bucket_expected, i32_dev, say, to_np
from synth import random_groups

pytestmark = pytest.mark.gpu


def _bucket(groups_np, K):
    from learned_centroid_gated_amd import focus_bucket
    off, idx, slot = focus_bucket(i32_dev(groups_np), K)
    torch.cuda.synchronize()
    return to_np(off), to_np(idx), to_np(slot)


@pytest.mark.parametrize("n,K,k,skew", [(1, 1, 1, 0), (2, 3, 2, 0), (63, 4, 1, 0), (64, 16, 2, 0),
                                        (65, 7, 3, 1.5), (255, 2, 1, 0), (256, 2, 2, 0),
                                        (257, 100, 2, 1.1), (1000, 1024, 4, 0),
                                        (4097, 64, 2, 1.1), (20000, 256, 1, 0.5),
                                        (70000, 128, 8, 0)])
def test_bucket_exact(n, K, k, skew):
    say(f"bucket n={n} K={K} k={k} skew={skew}")
    g = random_groups(n, K, k, np.random.default_rng(n + K + k), skew=skew)
    off, idx, slot = _bucket(g, K)
    e_off, e_idx, e_slot = bucket_expected(g, K)
    np.testing.assert_array_equal(off, e_off)
    np.testing.assert_array_equal(idx, e_idx)
    np.testing.assert_array_equal(slot, e_slot)


def test_bucket_drops_invalid_ids_and_batches():
    rng = np.random.default_rng(3)
    B, n, K, k = 3, 700, 10, 2
    g = np.stack([random_groups(n, K, k, rng) for _ in range(B)])
    g[1, 5, 0] = -1
    g[2, 17, 1] = K + 3
    from learned_centroid_gated_amd import focus_bucket
    off, idx, slot = focus_bucket(i32_dev(g), K)
    off, idx, slot = to_np(off), to_np(idx), to_np(slot)
    for b in range(B):
        e_off, e_idx, e_slot = bucket_expected(g[b], K)
        np.testing.assert_array_equal(off[b], e_off)
        np.testing.assert_array_equal(idx[b], e_idx)
        np.testing.assert_array_equal(slot[b], e_slot)
    assert slot[1, 5, 0] == -1 and slot[2, 17, 1] == -1


def test_bucket_empty_sequence():
    from learned_centroid_gated_amd import focus_bucket
    off, idx, slot = focus_bucket(torch.zeros((0, 2), dtype=torch.int32, device="cuda"), 5)
    torch.cuda.synchronize()
    assert to_np(off).tolist() == [0] * 6
