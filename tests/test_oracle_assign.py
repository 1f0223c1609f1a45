"""Pins for the oracle's group assignment (scores, Sinkhorn, top-k) against what the pages
and the mathematics fix, independently of the oracle's own code."""
import itertools
import math

import numpy as np
import pytest

from conftest import load_golden
from oracle import TIE_LOG, assign_ref, scores_ref, sinkhorn_ref, topk_ref
from synth import assign_inputs


def test_scores_hand_worked():
    g = load_golden("scores_tiny.json")
    S = scores_ref(np.array(g["hidden"], np.float32), np.array(g["w_g"], np.float32),
                   np.array(g["centroids"], np.float32))
    np.testing.assert_array_equal(S, np.array(g["S"], np.float64))


def _sinkhorn_knopp(S, iters):
    """Textbook multiplicative Sinkhorn-Knopp on exp(S): rows to 1, then columns to n/K."""
    n, K = S.shape
    P = np.exp(S)
    for _ in range(iters):
        P = P / P.sum(axis=1, keepdims=True)
        P = P * (n / K) / P.sum(axis=0, keepdims=True)
    return P


@pytest.mark.parametrize("n,K,iters", [(7, 3, 1), (64, 16, 3), (200, 8, 5), (33, 33, 2)])
def test_sinkhorn_matches_multiplicative_scaling(n, K, iters):
    rng = np.random.default_rng(n * 100 + K)
    S = rng.normal(0, 1.5, (n, K))
    u, v = sinkhorn_ref(S, iters)
    np.testing.assert_allclose(S + u[:, None] + v[None, :], np.log(_sinkhorn_knopp(S, iters)),
                               rtol=0, atol=1e-10)


def test_sinkhorn_closed_form_2x2_limit():
    g = load_golden("sinkhorn_2x2.json")
    S = np.array(g["S"])
    u, v = sinkhorn_ref(S, 200)
    np.testing.assert_allclose(np.exp(S + u[:, None] + v[None, :]), np.array(g["plan_limit"]),
                               rtol=0, atol=1e-12)
    groups, _, _ = topk_ref(S + v[None, :], 1)
    np.testing.assert_array_equal(groups, np.array(g["top1_groups"]))


@pytest.mark.parametrize("iters", [1, 2, 3])
def test_column_masses_exact(iters):
    rng = np.random.default_rng(iters)
    n, K = 500, 16
    S = rng.normal(0, 1, (n, K))
    u, v = sinkhorn_ref(S, iters)
    col = np.exp(S + u[:, None] + v[None, :]).sum(axis=0)
    np.testing.assert_allclose(col, n / K, rtol=1e-12)


def test_rows_converge_to_one():
    rng = np.random.default_rng(5)
    n, K = 300, 12
    S = rng.normal(0, 1, (n, K))
    errs = []
    for iters in (1, 5, 50):
        u, v = sinkhorn_ref(S, iters)
        rows = np.exp(S + u[:, None] + v[None, :]).sum(axis=1)
        errs.append(np.abs(rows - 1).max())
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 1e-9


def test_rank_one_scores_balance_to_uniform_and_tie_everywhere():
    rng = np.random.default_rng(11)
    n, K, k = 40, 8, 2
    S = rng.normal(size=n)[:, None] + rng.normal(size=K)[None, :]
    u, v = sinkhorn_ref(S, 1)
    np.testing.assert_allclose(np.exp(S + u[:, None] + v[None, :]), 1.0 / K, atol=1e-12)
    # every balanced row is constant: a near-tie everywhere, resolved to the lowest indices
    groups, tie, _ = topk_ref(S + u[:, None] + v[None, :], k)
    assert tie.all()
    b = np.zeros((n, K))
    groups, tie, _ = topk_ref(b, k)
    np.testing.assert_array_equal(groups, np.tile(np.arange(k), (n, 1)))


def _brute_topk(row, k):
    best = None
    for sub in itertools.combinations(range(len(row)), k):
        s = sum(row[list(sub)])
        if best is None or s > best[0]:
            best = (s, sub)
    return list(best[1])


@pytest.mark.parametrize("K,k", [(5, 1), (6, 2), (7, 3), (4, 4)])
def test_topk_brute_force(K, k):
    rng = np.random.default_rng(K * 10 + k)
    b = rng.normal(size=(50, K))
    groups, tie, _ = topk_ref(b, k)
    for i in range(50):
        assert list(groups[i]) == sorted(_brute_topk(b[i], k))
    assert not tie.any()


def test_tie_flag_window():
    b = np.array([[1.0, 1.0 - 0.5 * TIE_LOG, 0.0],
                  [1.0, 1.0 - 2.0 * TIE_LOG, 0.0],
                  [2.0, 2.0, 2.0]])
    groups, tie, gap = topk_ref(b, 1)
    assert list(tie) == [True, False, True]
    assert groups[2, 0] == 0
    assert math.isclose(TIE_LOG, 1e-5, rel_tol=1e-4)


def test_iters_zero_is_topk_of_raw_scores():
    a = assign_inputs(64, 32, 8, 6, 4, index=0, salt=7)
    r = assign_ref(a["hidden"], a["w_g"], a["centroids"], 2, 0)
    np.testing.assert_array_equal(r["v"], 0.0)
    S = r["S"]
    for i in range(64):
        assert list(r["groups"][i]) == sorted(_brute_topk(S[i], 2))


def test_centroid_permutation_equivariance():
    a = assign_inputs(300, 48, 16, 12, 12, index=0, salt=3)
    perm = np.random.default_rng(1).permutation(12)
    r0 = assign_ref(a["hidden"], a["w_g"], a["centroids"], 2, 3)
    r1 = assign_ref(a["hidden"], a["w_g"], a["centroids"][perm], 2, 3)
    np.testing.assert_allclose(r1["v"], r0["v"][perm], atol=1e-12)
    # group perm[c] of the permuted set is group c... of the original: map back and compare sets
    mapped = np.sort(perm[r1["groups"]], axis=1)
    ok = ~(r0["tie"] | r1["tie"])
    np.testing.assert_array_equal(mapped[ok], r0["groups"][ok])


def test_balanced_groups_are_roughly_equal():
    # Sinkhorn's equal column mass shows up as near-equal hard group sizes on mixture data
    a = assign_inputs(4096, 64, 32, 16, 16, index=0, salt=1)
    r = assign_ref(a["hidden"], a["w_g"], a["centroids"], 1, 3)
    sizes = np.bincount(r["groups"][:, 0], minlength=16)
    assert sizes.min() > 0.5 * 4096 / 16 and sizes.max() < 1.6 * 4096 / 16


def test_balanced_ranking_golden():
    """Hand-worked case in which one Sinkhorn iteration moves token 2's top-1 away from its raw
    argmax: ranking by raw scores, by S - v, or by the row-only plan all fail it."""
    g = load_golden("balanced_rank_n3.json")
    h, w, c = (np.array(g[x], np.float64) for x in ("hidden", "w_g", "centroids"))
    ref = assign_ref(h, w, c, 1, g["iters"])
    np.testing.assert_allclose(ref["v"], np.array(g["v"]), rtol=0, atol=1e-12)
    plan = np.exp(ref["S"] + ref["u"][:, None] + ref["v"][None, :])
    np.testing.assert_allclose(plan, np.array(g["plan"]), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(ref["groups"], np.array(g["top1_groups"]))
    raw = assign_ref(h, w, c, 1, 0)
    np.testing.assert_array_equal(raw["groups"], np.array(g["top1_groups_raw"]))
