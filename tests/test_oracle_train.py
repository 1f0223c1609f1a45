"""Pins for the oracle's training side: the soft-gated forward and the backward to the
centroids, the projection and the hidden states. The backward is checked against central
finite differences of the forward (an independent route to the same derivatives), and the
forward's pieces against hand-worked values, a library attention routine and the inference
oracle's hard gate."""
import math

import numpy as np
import pytest
import torch

from conftest import load_golden
from oracle import soft_gate_ref
from oracle.train_ref import (biased_attention_ref, soft_affinity_bias_ref, soft_assignment_ref,
                              soft_train_backward_ref, soft_train_forward_ref)


def _problem(n, d, dg, K, Hq, Hkv, dh, seed):
    rng = np.random.default_rng(seed)
    return dict(hidden=rng.normal(0, 1, (n, d)), w_g=rng.normal(0, 0.7, (d, dg)),
                centroids=rng.normal(0, 1, (K, dg)), q=rng.normal(0, 1, (n, Hq, dh)),
                k=rng.normal(0, 1, (n, Hkv, dh)), v=rng.normal(0, 1, (n, Hkv, dh)),
                dout=rng.normal(0, 1, (n, Hq, dh)))


def _loss(p, iters, window, lam, **over):
    a = {**p, **over}
    out, _, _ = soft_train_forward_ref(a["hidden"], a["w_g"], a["centroids"], iters, a["q"],
                                       a["k"], a["v"], window, lam)
    return float(np.sum(a["dout"] * out))


def _fd(p, name, iters, window, lam, eps=1e-6):
    x = p[name]
    g = np.empty_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        g[idx] = (_loss(p, iters, window, lam, **{name: xp}) -
                  _loss(p, iters, window, lam, **{name: xm})) / (2 * eps)
    return g


CASES = [
    # n, d, dg, K, Hq, Hkv, dh, iters, window, lam
    (9, 5, 3, 3, 2, 1, 4, 2, 2, 3.0),
    (8, 4, 4, 2, 4, 2, 3, 1, 0, -2.0),
    (7, 3, 2, 4, 1, 1, 5, 3, 1, 8.0),
    (6, 4, 3, 3, 2, 2, 4, 0, 2, 1.5),
]


@pytest.mark.parametrize("n,d,dg,K,Hq,Hkv,dh,iters,window,lam", CASES)
def test_backward_matches_finite_differences(n, d, dg, K, Hq, Hkv, dh, iters, window, lam):
    p = _problem(n, d, dg, K, Hq, Hkv, dh, seed=n * 10 + K)
    g = soft_train_backward_ref(p["hidden"], p["w_g"], p["centroids"], iters, p["q"], p["k"],
                                p["v"], p["dout"], window, lam)
    for name, key in (("centroids", "d_centroids"), ("w_g", "d_w_g"), ("hidden", "d_hidden")):
        fd = _fd(p, name, iters, window, lam)
        scale = max(1.0, np.abs(fd).max())
        np.testing.assert_allclose(g[key], fd, rtol=0, atol=2e-6 * scale, err_msg=name)
        assert np.abs(fd).max() > 1e-4, f"{name}: the case does not exercise the gradient"


def test_no_gradient_without_a_gate_slope_or_far_pairs():
    p = _problem(8, 4, 3, 3, 2, 1, 4, seed=3)
    args = (p["hidden"], p["w_g"], p["centroids"], 2, p["q"], p["k"], p["v"], p["dout"])
    for window, lam in ((2, 0.0), (8, 5.0), (100, -3.0)):  # lambda 0: constant gate; all near
        g = soft_train_backward_ref(*args, window, lam)
        for key in ("d_centroids", "d_w_g", "d_hidden"):
            assert np.all(g[key] == 0.0), (window, lam, key)


def test_centroid_relabelling_permutes_the_centroid_gradient():
    p = _problem(9, 5, 3, 4, 2, 1, 4, seed=11)
    perm = np.array([2, 0, 3, 1])
    base = soft_train_backward_ref(p["hidden"], p["w_g"], p["centroids"], 2, p["q"], p["k"],
                                   p["v"], p["dout"], 2, 4.0)
    perm_g = soft_train_backward_ref(p["hidden"], p["w_g"], p["centroids"][perm], 2, p["q"],
                                     p["k"], p["v"], p["dout"], 2, 4.0)
    np.testing.assert_allclose(perm_g["d_centroids"], base["d_centroids"][perm], atol=1e-12)
    np.testing.assert_allclose(perm_g["d_w_g"], base["d_w_g"], atol=1e-12)


def test_affinity_bias_hand_worked():
    gd = load_golden("soft_affinity_n3.json")
    B = soft_affinity_bias_ref(np.array(gd["g"]), gd["window"], gd["lambda"])
    want = np.array([[-np.inf if x is None else x for x in row] for row in gd["bias_lower"]])
    np.testing.assert_allclose(B, want, rtol=0, atol=1e-15)


def test_biased_attention_matches_sdpa_with_an_additive_mask():
    rng = np.random.default_rng(5)
    n, Hq, Hkv, dh = 11, 4, 2, 8
    q, k, v = rng.normal(size=(n, Hq, dh)), rng.normal(size=(n, Hkv, dh)), rng.normal(size=(n, Hkv, dh))
    bias = np.tril(rng.normal(size=(n, n)))
    bias[np.triu_indices(n, 1)] = -np.inf
    out, lse = biased_attention_ref(q, k, v, bias)
    G = Hq // Hkv
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).permute(1, 0, 2)  # noqa: E731
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(np.repeat(k, G, axis=1)), t(np.repeat(v, G, axis=1)),
        attn_mask=torch.from_numpy(bias))
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), atol=1e-12)
    s = np.einsum("ihd,jhd->hij", q, np.repeat(k, G, axis=1)) / math.sqrt(dh) + bias[None]
    np.testing.assert_allclose(lse.T, np.log(np.exp(s).sum(axis=2)), atol=1e-12)


def test_one_hot_assignments_reduce_to_the_hard_gate():
    """With one-hot rows g, a_ij = 1[same group] - 1/2: the forward is the inference oracle's
    soft gate over top-1 memberships."""
    rng = np.random.default_rng(8)
    n, Hq, Hkv, dh, K = 40, 4, 2, 8, 5
    groups = rng.integers(0, K, size=(n, 1))
    g = np.eye(K)[groups[:, 0]]
    q, k, v = rng.normal(size=(n, Hq, dh)), rng.normal(size=(n, Hkv, dh)), rng.normal(size=(n, Hkv, dh))
    for window, lam in ((3, 4.0), (0, -2.0), (10, 30.0)):
        out, _ = biased_attention_ref(q, k, v, soft_affinity_bias_ref(g, window, lam))
        np.testing.assert_allclose(out, soft_gate_ref(q, k, v, groups, window, lam), atol=1e-12)


def test_soft_assignment_is_the_balanced_plan():
    gd = load_golden("balanced_rank_n3.json")
    g = soft_assignment_ref(*(np.array(gd[x]) for x in ("hidden", "w_g", "centroids")), gd["iters"])
    np.testing.assert_allclose(g, np.array(gd["plan"]), atol=1e-12)


def test_sampled_rows_equal_the_full_forward():
    from oracle.train_ref import soft_train_forward_rows_ref
    p = _problem(30, 6, 4, 3, 4, 2, 5, seed=21)
    out, lse, g = soft_train_forward_ref(p["hidden"], p["w_g"], p["centroids"], 2, p["q"], p["k"],
                                         p["v"], 3, 5.0)
    rows = np.array([0, 1, 7, 29])
    o_r, l_r = soft_train_forward_rows_ref(g, p["q"], p["k"], p["v"], 3, 5.0, rows)
    np.testing.assert_allclose(o_r, out[rows], atol=1e-12)
    np.testing.assert_allclose(l_r, lse[rows], atol=1e-12)
