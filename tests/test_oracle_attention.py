"""Pins for the oracle's gated attention, pair set, decode and soft gate."""
import math

import numpy as np
import pytest
import torch

from conftest import load_golden
from oracle import (allowed_keys_ref, attention_rows_ref, decode_ref, owner_ref,
                    pair_count_ref, soft_gate_ref)
from synth import bf16_bits_to_f32, qkv_inputs, random_groups


def _golden_case(name):
    g = load_golden(name)
    n = g["n"]
    groups = np.array(g["groups"], np.int32)
    q = np.zeros((n, 1, 2))
    k = np.random.default_rng(0).normal(size=(n, 1, 2))
    v = np.stack([np.arange(n, dtype=np.float64), np.ones(n)], axis=1)[:, None, :]
    return g, groups, q, k, v


@pytest.mark.parametrize("name", ["pairs_top1_n8.json", "pairs_top2_n6.json"])
def test_golden_pair_sets_and_q0_outputs(name):
    g, groups, q, k, v = _golden_case(name)
    n, w = g["n"], g["window"]
    for i in range(n):
        assert list(allowed_keys_ref(i, groups, w)) == g["allowed"][i]
    np.testing.assert_array_equal(pair_count_ref(groups, w), g["counts"])
    out, lse = attention_rows_ref(q, k, v, groups, w)
    np.testing.assert_allclose(out[:, 0, :], np.array(g["out_q0"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0], np.log(g["counts"]), rtol=0, atol=1e-12)
    for i in range(n):
        for j in range(i + 1):
            o = owner_ref(i, j, groups, w)
            key = f"{i},{j}"
            if i - j < w:
                assert o == -1
            elif key in g["owners"]:
                assert o == g["owners"][key]
            else:
                assert o is None


def _brute_allowed(i, j, groups, w):
    if j > i:
        return False
    if i - j < w:
        return True
    return len(set(groups[i].tolist()) & set(groups[j].tolist())) > 0


@pytest.mark.parametrize("n,K,k,w", [(64, 4, 1, 3), (64, 6, 2, 0), (50, 5, 3, 5), (64, 1, 1, 1),
                                     (40, 8, 2, 64), (64, 3, 3, 2), (1, 2, 1, 0), (2, 3, 2, 1)])
def test_pair_set_brute_force_and_partition(n, K, k, w):
    rng = np.random.default_rng(n + K * 7 + k * 13 + w)
    groups = random_groups(n, K, k, rng)
    counts = np.zeros(n, np.int64)
    for i in range(n):
        brute = [j for j in range(n) if _brute_allowed(i, j, groups, w)]
        assert list(allowed_keys_ref(i, groups, w)) == brute
        counts[i] = len(brute)
        # owners partition the allowed set: every allowed pair has exactly one owner, and
        # the owner's segment contains both tokens
        for j in range(n):
            o = owner_ref(i, j, groups, w)
            assert (o is not None) == (j in brute)
            if o is not None and o >= 0:
                assert o in groups[i] and o in groups[j]
                assert all(gg >= o for gg in set(groups[i]) & set(groups[j]))
    np.testing.assert_array_equal(pair_count_ref(groups, w), counts)


def _loop_attention(q, k, v, groups, w, scale):
    """Plain loops with math.exp, a second statement of the same definition for tiny n."""
    n, Hq, dh = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((n, Hq, dh))
    lse = np.zeros((n, Hq))
    for i in range(n):
        for h in range(Hq):
            logits = {}
            for j in range(n):
                if _brute_allowed(i, j, groups, w):
                    logits[j] = scale * sum(q[i, h, d] * k[j, h // G, d] for d in range(dh))
            m = max(logits.values())
            z = sum(math.exp(x - m) for x in logits.values())
            lse[i, h] = m + math.log(z)
            for j, x in logits.items():
                out[i, h] += math.exp(x - lse[i, h]) * v[j, h // G]
    return out, lse


@pytest.mark.parametrize("n,Hq,Hkv,K,k,w", [(12, 2, 1, 3, 1, 2), (10, 4, 2, 4, 2, 1), (9, 1, 1, 2, 2, 0)])
def test_attention_matches_plain_loops(n, Hq, Hkv, K, k, w):
    rng = np.random.default_rng(n)
    q = rng.normal(size=(n, Hq, 5))
    kk = rng.normal(size=(n, Hkv, 5))
    v = rng.normal(size=(n, Hkv, 5))
    groups = random_groups(n, K, k, rng)
    out, lse = attention_rows_ref(q, kk, v, groups, w, scale=0.7)
    o2, l2 = _loop_attention(q, kk, v, groups, w, 0.7)
    np.testing.assert_allclose(out, o2, atol=1e-12)
    np.testing.assert_allclose(lse, l2, atol=1e-12)


def _sdpa_causal(q, k, v, G):
    qt = torch.from_numpy(bf16_bits_to_f32(q).astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(bf16_bits_to_f32(k).astype(np.float64)).permute(1, 0, 2)
    vt = torch.from_numpy(bf16_bits_to_f32(v).astype(np.float64)).permute(1, 0, 2)
    kt = kt.repeat_interleave(G, dim=0)
    vt = vt.repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("case", ["one_group", "wide_window"])
def test_reduces_to_full_causal_attention(case):
    n, Hq, Hkv, dh = 96, 4, 2, 16
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=21)
    if case == "one_group":
        groups, w = np.zeros((n, 1), np.int32), 4
    else:
        groups, w = random_groups(n, 8, 1, np.random.default_rng(2)), n
    out, _ = attention_rows_ref(t["q"], t["k"], t["v"], groups, w)
    np.testing.assert_allclose(out, _sdpa_causal(t["q"], t["k"], t["v"], Hq // Hkv), atol=1e-12)


def test_weights_are_a_distribution_on_the_allowed_set():
    # V = one-hot rows (dh = n): out_i is the attention weight vector of row i
    n, K, k, w = 48, 4, 2, 3
    rng = np.random.default_rng(9)
    groups = random_groups(n, K, k, rng)
    q = rng.normal(size=(n, 2, 8))
    kk = rng.normal(size=(n, 1, 8))
    v = np.eye(n)[:, None, :]
    out, _ = attention_rows_ref(q, kk, v, groups, w)
    np.testing.assert_allclose(out.sum(axis=2), 1.0, atol=1e-12)
    for i in range(n):
        support = set(np.nonzero(out[i, 0] > 0)[0].tolist())
        assert support == set(allowed_keys_ref(i, groups, w).tolist())


def test_q_zero_counts_pairs():
    n, K, k, w = 300, 6, 2, 7
    rng = np.random.default_rng(4)
    groups = random_groups(n, K, k, rng)
    q = np.zeros((n, 2, 4))
    kk = rng.normal(size=(n, 2, 4))
    v = rng.normal(size=(n, 2, 4))
    out, lse = attention_rows_ref(q, kk, v, groups, w)
    counts = pair_count_ref(groups, w)
    np.testing.assert_allclose(np.exp(lse), np.repeat(counts[:, None], 2, axis=1), rtol=1e-12)


def test_group_relabelling_leaves_output_unchanged():
    n = 80
    t = qkv_inputs(n, 2, 1, 8, index=0, salt=5)
    groups = random_groups(n, 6, 2, np.random.default_rng(3))
    perm = np.random.default_rng(8).permutation(6)
    o0, l0 = attention_rows_ref(t["q"], t["k"], t["v"], groups, 5)
    o1, l1 = attention_rows_ref(t["q"], t["k"], t["v"], np.sort(perm[groups], axis=1), 5)
    np.testing.assert_allclose(o0, o1, atol=1e-13)
    np.testing.assert_allclose(l0, l1, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    n, Hq, Hkv = 40, 4, 2
    t = qkv_inputs(n, Hq, Hkv, 8, index=0, salt=6)
    groups = random_groups(n, 4, 1, np.random.default_rng(1))
    o_gqa, _ = attention_rows_ref(t["q"], t["k"], t["v"], groups, 3)
    k_rep = np.repeat(t["k"], Hq // Hkv, axis=1)
    v_rep = np.repeat(t["v"], Hq // Hkv, axis=1)
    o_mha, _ = attention_rows_ref(t["q"], k_rep, v_rep, groups, 3)
    np.testing.assert_allclose(o_gqa, o_mha, atol=1e-13)
    # a transposed head map (h % Hkv instead of h // G) would differ
    assert not np.allclose(o_gqa[:, 1], o_mha[:, 2])


def test_decode_equals_last_prefill_row():
    B, L, Hq, Hkv, dh, K, k, w = 3, 70, 4, 2, 8, 5, 2, 6
    rng = np.random.default_rng(12)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=9, lead=(B,))
    cache_groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)])
    q_groups = np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])
    lens = np.array([70, 1, 33])
    qdec = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
    out, lse = decode_ref(qdec, q_groups, t["k"], t["v"], lens, cache_groups, w)
    for b in range(B):
        L_b = lens[b]
        g = cache_groups[b, :L_b].copy()
        g[L_b - 1] = q_groups[b]
        o_p, l_p = attention_rows_ref(t["q"][b, :L_b], t["k"][b, :L_b], t["v"][b, :L_b], g, w,
                                      rows=[L_b - 1])
        np.testing.assert_allclose(out[b], o_p[0], atol=1e-13)
        np.testing.assert_allclose(lse[b], l_p[0], atol=1e-13)


def test_soft_gate_approaches_hard_mask():
    n, Hq, Hkv, dh = 64, 2, 1, 16
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=13)
    groups = random_groups(n, 4, 1, np.random.default_rng(6))
    w = 8
    hard, _ = attention_rows_ref(t["q"], t["k"], t["v"], groups, w)
    errs = [np.abs(soft_gate_ref(t["q"], t["k"], t["v"], groups, w, lam) - hard).max()
            for lam in (1.0, 10.0, 100.0)]
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 1e-9
    # the printed form (gate multiplies the logit) keeps e^0 weight on gated pairs
    lit = np.abs(soft_gate_ref(t["q"], t["k"], t["v"], groups, w, 100.0, literal=True) - hard).max()
    assert lit > 0.05


def test_soft_gate_lse_all_local_is_causal_attention():
    # window >= n: every pair is local, no gate applies, and the soft forward is plain causal
    # attention; its lse must then equal the hard rule's (which also allows every causal pair)
    n, Hq, Hkv, dh = 50, 4, 2, 16
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=21)
    groups = random_groups(n, 6, 2, np.random.default_rng(3))
    out_s, lse_s = soft_gate_ref(t["q"], t["k"], t["v"], groups, n, 7.0, with_lse=True)
    out_h, lse_h = attention_rows_ref(t["q"], t["k"], t["v"], groups, n)
    np.testing.assert_allclose(out_s, out_h, atol=1e-12)
    np.testing.assert_allclose(lse_s, lse_h, atol=1e-12)
    # and lse is the log of the softmax normaliser: the weights recomputed from it sum to one
    _, lse10 = soft_gate_ref(t["q"], t["k"], t["v"], groups, 4, 10.0, with_lse=True)
    assert lse10.shape == (n, Hq) and np.isfinite(lse10).all()
    assert (lse10 <= lse_h + 1e-12).all()  # the gate only removes weight (log sigmoid < 0)
