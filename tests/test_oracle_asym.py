"""Pins for the oracle's asymmetric top-k variant: every key sits in its top-1 group, every
query looks at its k groups (Dutch summary, Resultaten, 'Inferentie'; Chinese summary,
section 4 table)."""
import numpy as np
import pytest
import torch

from conftest import load_golden
from oracle import (allowed_keys_asym_ref, allowed_keys_ref, assign_ref,
                    attention_rows_asym_ref, attention_rows_ref, pair_count_asym_ref)
from synth import assign_inputs, bf16_bits_to_f32, qkv_inputs, random_groups


def _asym_groups(n, K, kq, rng):
    """Random query groups and, for every token, a key group drawn from its own query groups
    (as top-1 lies inside top-k)."""
    qg = random_groups(n, K, kq, rng)
    kg = qg[np.arange(n), rng.integers(0, kq, size=n)].astype(np.int32)
    return qg, kg


def test_golden_hand_worked_pair_sets_and_q0_outputs():
    g = load_golden("pairs_asym_n7.json")
    n, w = g["n"], g["window"]
    qg = np.array(g["q_groups"], np.int32)
    kg = np.array(g["k_group"], np.int32)
    for i in range(n):
        assert list(allowed_keys_asym_ref(i, qg, kg, w)) == g["allowed"][i]
    # the symmetric rule on the same query groups is a different pair set
    assert list(allowed_keys_ref(3, qg, w)) == g["symmetric_allowed_3"]
    np.testing.assert_array_equal(pair_count_asym_ref(qg, kg, w), g["counts"])
    q = np.zeros((n, 1, 2))
    k = np.random.default_rng(0).normal(size=(n, 1, 2))
    v = np.stack([np.arange(n, dtype=np.float64), np.ones(n)], axis=1)[:, None, :]
    out, lse = attention_rows_asym_ref(q, k, v, qg, kg, w)
    np.testing.assert_allclose(out[:, 0, :], np.array(g["out_q0"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0], np.log(g["counts"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,w", [(64, 0), (203, 5), (400, 17)])
def test_two_of_four_groups_halves_the_far_pairs(n, w):
    """Keys cycle through K = 4 groups (j % 4) and query i looks at groups i % 4 and
    (i + 1) % 4. Closed form: the far keys of group g below i - w + 1 number
    floor((i - w - g) / 4) + 1 when i - w >= g, and over all queries they are half of the
    far causal pairs up to boundary terms -- the 2-of-4 arithmetic of the pages."""
    K = 4
    kg = (np.arange(n) % K).astype(np.int32)
    qg = np.sort(np.stack([np.arange(n) % K, (np.arange(n) + 1) % K], axis=1), axis=1).astype(np.int32)
    counts = pair_count_asym_ref(qg, kg, w)
    far_total = 0
    for i in range(n):
        far = 0
        for g in (i % K, (i + 1) % K):
            if i - w >= g:
                far += (i - w - g) // K + 1
        assert counts[i] == min(i + 1, w) + far
        far_total += far
    causal_far = sum(max(i - w + 1, 0) for i in range(n))
    assert abs(far_total - causal_far / 2) <= n  # boundary terms: at most one key per query
    assert abs(far_total / causal_far - 0.5) < 0.03


@pytest.mark.parametrize("n,K,kq,w", [(50, 3, 2, 4), (120, 8, 3, 0), (97, 5, 4, 9), (64, 6, 1, 3)])
def test_pair_counts_match_the_allowed_sets(n, K, kq, w):
    qg, kg = _asym_groups(n, K, kq, np.random.default_rng(n + K))
    counts = pair_count_asym_ref(qg, kg, w)
    for i in range(n):
        assert len(allowed_keys_asym_ref(i, qg, kg, w)) == counts[i]


@pytest.mark.parametrize("n,K,kq,w", [(80, 5, 2, 3), (64, 4, 3, 0), (90, 7, 4, 6)])
def test_asym_pairs_lie_inside_the_symmetric_pairs(n, K, kq, w):
    """With each key group among the token's own query groups, an asymmetric far pair (key
    group among the query's groups) always shares a group, so it is a symmetric pair too;
    the reverse fails somewhere for kq > 1."""
    qg, kg = _asym_groups(n, K, kq, np.random.default_rng(7 * n + kq))
    strict = False
    for i in range(n):
        a = set(allowed_keys_asym_ref(i, qg, kg, w).tolist())
        s = set(allowed_keys_ref(i, qg, w).tolist())
        assert a <= s
        strict = strict or a != s
    assert strict


def test_single_group_membership_reduces_to_the_symmetric_rule():
    """kq = 1 with k_group = q_groups[:, 0]: both rules read 'same group'."""
    n, Hq, Hkv, dh = 96, 4, 2, 16
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=41)
    qg = random_groups(n, 6, 1, np.random.default_rng(5))
    kg = qg[:, 0].copy()
    for i in range(n):
        np.testing.assert_array_equal(allowed_keys_asym_ref(i, qg, kg, 7),
                                      allowed_keys_ref(i, qg, 7))
    o1, l1 = attention_rows_asym_ref(t["q"], t["k"], t["v"], qg, kg, 7)
    o2, l2 = attention_rows_ref(t["q"], t["k"], t["v"], qg, 7)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def _sdpa_causal(q, k, v, G):
    qt = torch.from_numpy(bf16_bits_to_f32(q).astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(bf16_bits_to_f32(k).astype(np.float64)).permute(1, 0, 2)
    vt = torch.from_numpy(bf16_bits_to_f32(v).astype(np.float64)).permute(1, 0, 2)
    kt = kt.repeat_interleave(G, dim=0)
    vt = vt.repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("case", ["looks_at_every_group", "wide_window"])
def test_reduces_to_full_causal_attention(case):
    n, Hq, Hkv, dh = 96, 4, 2, 16
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=43)
    rng = np.random.default_rng(3)
    if case == "looks_at_every_group":  # K = kq: every key group is looked at
        qg = np.tile(np.arange(3, dtype=np.int32), (n, 1))
        kg = rng.integers(0, 3, size=n).astype(np.int32)
        w = 4
    else:
        qg, kg = _asym_groups(n, 8, 2, rng)
        w = n
    out, _ = attention_rows_asym_ref(t["q"], t["k"], t["v"], qg, kg, w)
    np.testing.assert_allclose(out, _sdpa_causal(t["q"], t["k"], t["v"], Hq // Hkv), atol=1e-12)


def test_q_zero_lse_counts_pairs_and_weights_cover_the_allowed_set():
    """At Q = 0 every allowed key has weight 1 / count: lse = log count (counted by the
    independent position search) and out = the mean of V over the allowed set."""
    n, K, kq, w = 150, 6, 2, 5
    qg, kg = _asym_groups(n, K, kq, np.random.default_rng(11))
    rng = np.random.default_rng(12)
    q = np.zeros((n, 2, 4))
    k = rng.normal(size=(n, 1, 4))
    v = rng.normal(size=(n, 1, 3))
    out, lse = attention_rows_asym_ref(q, k, v, qg, kg, w)
    counts = pair_count_asym_ref(qg, kg, w)
    np.testing.assert_allclose(lse, np.log(counts)[:, None].repeat(2, 1), atol=1e-12)
    for i in range(0, n, 7):
        J = allowed_keys_asym_ref(i, qg, kg, w)
        np.testing.assert_allclose(out[i, 0], v[J, 0].mean(axis=0), atol=1e-12)


def test_group_relabelling_leaves_output_unchanged():
    n, Hq, Hkv, dh, K = 80, 2, 1, 8, 5
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=45)
    qg, kg = _asym_groups(n, K, 2, np.random.default_rng(9))
    perm = np.random.default_rng(10).permutation(K).astype(np.int32)
    o1, l1 = attention_rows_asym_ref(t["q"], t["k"], t["v"], qg, kg, 3)
    o2, l2 = attention_rows_asym_ref(t["q"], t["k"], t["v"], np.sort(perm[qg], axis=1), perm[kg], 3)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_assigned_top1_lies_in_assigned_topk():
    """The key group (top-1 of the balanced scores) is one of the token's top-k groups, with
    the same tie rule, so the assignment stage feeds both sides of the variant."""
    n, d, dg, K = 300, 32, 16, 6
    inp = assign_inputs(n, d, dg, K, mix=K, index=0)
    a1 = assign_ref(inp["hidden"], inp["w_g"], inp["centroids"], 1, 3)["groups"][:, 0]
    a3 = assign_ref(inp["hidden"], inp["w_g"], inp["centroids"], 3, 3)["groups"]
    assert all(a1[i] in a3[i] for i in range(n))


def test_row_without_allowed_keys_has_lse_minus_infinity():
    """Window 0 and a key group outside the token's own query groups: token 1 (key group 1,
    looking at group 0) has no earlier key of group 0 and does not see itself."""
    qg = np.array([[0], [0], [1]], np.int32)
    kg = np.array([0, 1, 1], np.int32)
    assert list(allowed_keys_asym_ref(1, qg, kg, 0)) == [0]
    assert list(allowed_keys_asym_ref(0, qg, kg, 0)) == [0]
    qg2 = np.array([[1], [0], [1]], np.int32)  # token 0 looks at group 1, its key group is 0
    assert len(allowed_keys_asym_ref(0, qg2, kg, 0)) == 0
    q = np.random.default_rng(1).normal(size=(3, 2, 4))
    k = np.random.default_rng(2).normal(size=(3, 1, 4))
    v = np.random.default_rng(3).normal(size=(3, 1, 4))
    out, lse = attention_rows_asym_ref(q, k, v, qg2, kg, 0)
    assert np.all(lse[0] == -np.inf) and np.all(out[0] == 0)
    assert pair_count_asym_ref(qg2, kg, 0)[0] == 0
    # row 2 (looks at group 1) sees keys 1 and 2: an ordinary softmax
    assert np.isfinite(lse[2]).all()
