"""focus_assign on the GPU against the oracle: group sets bit-exact except on tokens whose
k-th and (k+1)-th balanced scores lie within the tie window, where the GPU's set must still be
a valid top-k; the column potential within fp32 tolerance."""
import numpy as np
import pytest
import torch

from gpu_util import dev, f32_dev, say, to_np
from oracle import TIE_LOG, assign_ref
from synth import CONFIGS, assign_inputs

pytestmark = pytest.mark.gpu


def _check_groups(g_gpu, ref, S_plus_v):
    g = np.asarray(g_gpu)
    n, k = g.shape
    assert (np.diff(g, axis=1) > 0).all(), "groups must be ascending and distinct"
    assert g.min() >= 0 and g.max() < S_plus_v.shape[1]
    same = (g == ref["groups"]).all(axis=1)
    bad = ~same & ~ref["tie"]
    say(f"  tokens={n} mismatched={(~same).sum()} flagged={ref['tie'].sum()} unflagged-mismatch={bad.sum()}")
    assert not bad.any(), f"{bad.sum()} unflagged tokens differ, first {np.nonzero(bad)[0][:5]}"
    # where a near-tie flipped the choice, the GPU set must still be a top-k within the window
    for i in np.nonzero(~same)[0]:
        row = S_plus_v[i]
        chosen = row[g[i]]
        others = np.delete(row, g[i])
        assert chosen.min() >= others.max() - 2 * TIE_LOG


def _run(hidden, w_g, cents, top_k, iters):
    d = dev()
    groups, v = focus_assign_dev(f32_dev(hidden), f32_dev(w_g), f32_dev(cents), top_k, iters)
    torch.cuda.synchronize()
    return to_np(groups), to_np(v)


def focus_assign_dev(h, w, c, top_k, iters):
    from learned_centroid_gated_amd import focus_assign
    return focus_assign(h, w, c, top_k, iters)


CASES = [
    # n, d, dg, K, top_k, iters, mix   (ragged n, K not a multiple of 4, d tails, fold/no fold)
    (2048, 768, 64, 16, 1, 3, 16),
    (1, 8, 4, 1, 1, 3, 1),
    (1, 64, 16, 4, 2, 0, 2),
    (63, 36, 12, 3, 1, 2, 3),
    (65, 260, 8, 5, 3, 1, 5),
    (1000, 128, 128, 100, 2, 3, 50),
    (777, 64, 32, 256, 1, 2, 40),
    (300, 96, 64, 1024, 4, 2, 64),
    (4097, 512, 128, 64, 2, 5, 64),
    (2000, 256, 16, 8, 8, 3, 8),
    # one iteration: the potentials come from the score product's fused first row step alone
    (4096, 512, 128, 64, 2, 1, 64),     # folded, 128-column tiles
    (3001, 64, 32, 256, 1, 1, 40),      # two products, 256-column tiles
    # two products with inner size 128 over at least one 256-row tile per compute unit: the
    # persistent score kernel with the centroids resident in LDS (ragged rows, K = 200)
    (70001, 512, 128, 200, 2, 2, 100),
    (66000, 512, 128, 256, 1, 1, 128),
]


@pytest.mark.parametrize("n,d,dg,K,top_k,iters,mix", CASES)
def test_assign_matches_oracle(n, d, dg, K, top_k, iters, mix):
    say(f"assign n={n} d={d} dg={dg} K={K} top_k={top_k} iters={iters}")
    a = assign_inputs(n, d, dg, K, mix, index=0, salt=n + K)
    ref = assign_ref(a["hidden"], a["w_g"], a["centroids"], top_k, iters)
    g, v = _run(a["hidden"], a["w_g"], a["centroids"], top_k, iters)
    np.testing.assert_allclose(v, ref["v"], rtol=0, atol=2e-5)
    _check_groups(g, ref, ref["S"] + ref["v"][None, :])


CROWDED = [
    # n, d, dg, K, top_k, iters, scaled   (fold; two products; K and d_g wider than a block; the
    # bf16 split product for d % 32 != 0; small hidden states)
    (4096, 512, 128, 64, 2, 3, "w_g"),
    (4096, 256, 16, 64, 1, 2, "w_g"),
    (2000, 128, 32, 1024, 8, 2, "w_g"),
    (1500, 64, 512, 300, 3, 2, "w_g"),
    (1000, 260, 8, 5, 3, 1, "w_g"),
    (4096, 512, 128, 64, 2, 3, "hidden"),
    (4096, 256, 16, 64, 1, 2, "hidden"),
]


@pytest.mark.parametrize("n,d,dg,K,top_k,iters,scaled", CROWDED)
def test_assign_crowded_scores(n, d, dg, K, top_k, iters, scaled):
    """One operand scaled by 1e-3 crowds the scores: most tokens' k-th and (k+1)-th balanced
    scores lie within 1e-3 of each other, so score errors far below that would already show as
    mismatches outside the tie window. Scaling the hidden states puts most of their elements
    below fp16's normal range, where the library's fp16 split keeps an absolute error only."""
    say(f"assign crowded n={n} d={d} dg={dg} K={K} top_k={top_k} iters={iters} ({scaled} x 1e-3)")
    a = assign_inputs(n, d, dg, K, K, index=0, salt=3 * n + K)
    h, w = a["hidden"], a["w_g"]
    if scaled == "w_g":
        w = w * np.float32(1e-3)
    else:
        h = h * np.float32(1e-3)
    ref = assign_ref(h, w, a["centroids"], top_k, iters)
    b = -np.sort(-(ref["S"] + ref["v"][None, :]), axis=1)
    near = float((b[:, top_k - 1] - b[:, top_k] < 1e-3).mean())
    say(f"  {near:.0%} of tokens within 1e-3 at the k-th place")
    assert near > 0.5
    g, v = _run(h, w, a["centroids"], top_k, iters)
    np.testing.assert_allclose(v, ref["v"], rtol=0, atol=2e-5)
    _check_groups(g, ref, ref["S"] + ref["v"][None, :])


@pytest.mark.parametrize("n,d,dg,K,top_k,iters", [(3000, 512, 128, 64, 2, 3),
                                                   (3000, 256, 32, 128, 1, 2),
                                                   (66000, 512, 128, 256, 1, 2)])
def test_assign_hidden_beyond_fp16_range(n, d, dg, K, top_k, iters):
    """Some tokens carry hidden values beyond fp16's largest finite value (65504) in three
    channels whose rows of W_g are small (large activations on channels the projection
    damps), so scores stay of order one; other tokens sit at fp16's edge in the same channels.
    The library's fp16 score products cannot represent the former: it lists those tokens and
    recomputes their scores exactly in fp32 before balancing (folded plan and two-product plan,
    where both products list the token). Groups and potentials must still match the oracle."""
    say(f"assign beyond fp16 range n={n} d={d} dg={dg} K={K}")
    a = assign_inputs(n, d, dg, K, K, index=0, salt=7 * n + K)
    h, w = a["hidden"].copy(), a["w_g"].copy()
    w[:3] *= np.float32(1e-4)
    rs = np.random.default_rng(n + d)
    big = rs.choice(n, 40, replace=False)
    for i, r in enumerate(big):
        h[r, :1 + i % 3] = np.float32((1 if i % 2 else -1) * (7e4 + 3e4 * i))
    edge = rs.choice(np.setdiff1d(np.arange(n), big), 20, replace=False)
    h[edge, 0] = np.float32(65504.0)
    h[edge[:10], 1] = np.float32(-65519.0)
    ref = assign_ref(h, w, a["centroids"], top_k, iters)
    assert np.abs(ref["S"]).max() < 50.0
    g, v = _run(h, w, a["centroids"], top_k, iters)
    np.testing.assert_allclose(v, ref["v"], rtol=0, atol=2e-5)
    _check_groups(g, ref, ref["S"] + ref["v"][None, :])


@pytest.mark.parametrize("n,d,dg,K,top_k,iters", [(2500, 512, 128, 100, 2, 3),
                                                   (2100, 256, 32, 128, 1, 2)])
def test_assign_every_row_beyond_fp16_range(n, d, dg, K, top_k, iters):
    """Every token carries one hidden value beyond fp16's range in a damped channel, so the
    fp16 score products list all of them and every score row is recomputed in fp32 (folded
    plan with K not a multiple of the eight columns a wave takes per pass; two-product plan).
    Groups and potentials must match the oracle."""
    say(f"assign every row beyond fp16 range n={n} d={d} dg={dg} K={K}")
    a = assign_inputs(n, d, dg, K, K, index=0, salt=11 * n + K)
    h, w = a["hidden"].copy(), a["w_g"].copy()
    w[:3] *= np.float32(1e-4)
    rs = np.random.default_rng(n + K)
    ch = rs.integers(0, 3, n)
    h[np.arange(n), ch] = (rs.choice([-1.0, 1.0], n) * rs.uniform(7e4, 2e5, n)).astype(np.float32)
    ref = assign_ref(h, w, a["centroids"], top_k, iters)
    assert np.abs(ref["S"]).max() < 50.0
    g, v = _run(h, w, a["centroids"], top_k, iters)
    np.testing.assert_allclose(v, ref["v"], rtol=0, atol=2e-5)
    _check_groups(g, ref, ref["S"] + ref["v"][None, :])


def test_assign_deterministic():
    a = assign_inputs(5000, 256, 64, 32, 32, index=0, salt=77)
    g1, v1 = _run(a["hidden"], a["w_g"], a["centroids"], 2, 3)
    g2, v2 = _run(a["hidden"], a["w_g"], a["centroids"], 2, 3)
    np.testing.assert_array_equal(g1, g2)
    np.testing.assert_array_equal(v1, v2)


@pytest.mark.parametrize("name", ["gpt2s_n2k", "gqa7b_n32k", "gqa70b_n128k"])
def test_assign_full_size(name):
    c = [x for x in CONFIGS if x.name == name][0]
    say(f"assign full size {name}: n={c.n} d={c.d}")
    a = assign_inputs(c.n, c.d, c.dg, c.K, c.mix, c.weights, c.noise_frac, index=c.index)
    g, v = _run(a["hidden"], a["w_g"], a["centroids"], c.top_k, c.iters)
    ref = assign_ref(a["hidden"], a["w_g"], a["centroids"], c.top_k, c.iters)
    np.testing.assert_allclose(v, ref["v"], rtol=0, atol=2e-5)
    _check_groups(g, ref, ref["S"] + ref["v"][None, :])
    # Sinkhorn's balance shows in the hard group sizes
    sizes = np.bincount(g.ravel(), minlength=c.K)
    say(f"  group sizes min={sizes.min()} mean={sizes.mean():.1f} max={sizes.max()}")


def _assign_device_inputs(c, n=None):
    """The workload's inputs drawn on the device (the bench's generator), plus host copies."""
    n = c.n if n is None else n
    a = assign_inputs(n, c.d, c.dg, c.K, c.mix, c.weights, c.noise_frac, index=c.index,
                      device="cuda")
    return a, {x: a[x].cpu().numpy() for x in ("hidden", "w_g", "centroids")}


def _compare_device_run(c, a, host):
    from learned_centroid_gated_amd import focus_assign
    groups, v = focus_assign(a["hidden"], a["w_g"], a["centroids"], c.top_k, c.iters)
    torch.cuda.synchronize()
    g, v = to_np(groups), to_np(v)
    say("  GPU done; oracle ...")
    ref = assign_ref(host["hidden"], host["w_g"], host["centroids"], c.top_k, c.iters)
    np.testing.assert_allclose(v, ref["v"], rtol=0, atol=2e-5)
    _check_groups(g, ref, ref["S"] + ref["v"][None, :])
    sizes = np.bincount(g.ravel(), minlength=c.K)
    say(f"  group sizes min={sizes.min()} mean={sizes.mean():.1f} max={sizes.max()}")


def test_assign_long_context_shapes_at_64k_tokens():
    """The 1M-token workload's shapes (d 4096, d_g 128, K 256, top-1, two iterations, 10% noise
    tokens) at n = 65536: the same two-product plan and kernels as the full size."""
    c = [x for x in CONFIGS if x.name == "long_n1m"][0]
    say(f"assign long_n1m shapes at n=65536: d={c.d} dg={c.dg} K={c.K}")
    a, host = _assign_device_inputs(c, 65536)
    _compare_device_run(c, a, host)


@pytest.mark.timeout(900)
def test_assign_full_size_long_n1m():
    """The 1M-token workload at full size, inputs drawn exactly as the benchmark draws them."""
    c = [x for x in CONFIGS if x.name == "long_n1m"][0]
    say(f"assign full size long_n1m: n={c.n} d={c.d} (17 GB of hidden states; oracle ~1-2 min)")
    a, host = _assign_device_inputs(c)
    _compare_device_run(c, a, host)
