"""focus_soft_attention (the training-time soft gate, forward) on the GPU against the oracle.

Every causal pair is attended; far pairs carry log sigmoid(lambda * (share - 1/2)). Element-wise
on every row, over sweeps of n (ragged tails), window (none, some, all local), top-k, GQA ratio,
head size and lambda; plus the large-lambda limit, which must reach focus_attention's hard
pair rule."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, check_attention, i32_dev, say, to_np
from oracle import soft_gate_ref
from synth import qkv_inputs, random_groups

pytestmark = pytest.mark.gpu

CASES = [
    # n, Hq, Hkv, dh, K, top_k, window, lambda
    (1, 1, 1, 64, 1, 1, 0, 3.0),
    (65, 2, 1, 128, 4, 1, 8, 4.0),
    (257, 4, 2, 128, 8, 1, 16, 4.0),
    (600, 8, 2, 64, 5, 2, 32, 10.0),
    (1000, 16, 4, 128, 16, 2, 0, 1.0),
    (513, 2, 1, 128, 3, 3, 700, 2.0),
    (300, 8, 8, 64, 4, 4, 64, 50.0),
    (777, 8, 1, 128, 12, 2, 100, -3.0),
    # G >= 8 (at most 16 query tokens per tile): the share term on the MFMA bias rows
    (1000, 16, 2, 128, 16, 2, 0, 4.0),
    (2049, 16, 2, 128, 128, 2, 1024, 10.0),
    (900, 16, 1, 64, 7, 4, 1, 6.0),
    (700, 32, 2, 128, 9, 3, 700, 2.0),
    (1300, 8, 1, 64, 5, 1, 37, -8.0),
    (640, 16, 2, 128, 6, 2, 64, 60.0),
    (520, 16, 2, 128, 6, 2, 40, 1000.0),  # the share term's parts must add up to it exactly
    # |lambda| large: each row shifts by the larger bias, so kept logits carry no large offset
    (520, 16, 2, 128, 6, 2, 40, 1e5),
    (530, 16, 2, 128, 6, 2, 40, -1e5),
    (600, 8, 2, 64, 5, 2, 32, 1e5),
    (1100, 32, 2, 128, 9, 1, 0, 3e4),
]


@pytest.mark.parametrize("n,Hq,Hkv,dh,K,k,w,lam", CASES)
def test_soft_matches_oracle(n, Hq, Hkv, dh, K, k, w, lam):
    from learned_centroid_gated_amd import focus_soft_attention
    say(f"soft n={n} Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w} lambda={lam}")
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=500 + n)
    groups = random_groups(n, K, k, np.random.default_rng(n + K))
    out, lse = focus_soft_attention(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]),
                                    i32_dev(groups), K, w, lam)
    torch.cuda.synchronize()
    o_ref, l_ref = soft_gate_ref(t["q"], t["k"], t["v"], groups, w, lam, with_lse=True)
    check_attention(out, lse, o_ref, l_ref, "soft")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (16, 2)])
def test_soft_large_lambda_reaches_hard_rule(Hq, Hkv):
    from learned_centroid_gated_amd import focus_attention, focus_bucket, focus_soft_attention
    n, dh, K, k, w = 1500, 128, 16, 2, 64
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=77)
    groups = random_groups(n, K, k, np.random.default_rng(5))
    q, kk, v, g = bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(groups)
    out_s, lse_s = focus_soft_attention(q, kk, v, g, K, w, 200.0)
    off, idx, slot = focus_bucket(g, K)
    out_h, lse_h = focus_attention(q, kk, v, g, off, idx, slot, K, w)
    torch.cuda.synchronize()
    d = np.abs(to_np(out_s) - to_np(out_h))
    dl = np.abs(to_np(lse_s) - to_np(lse_h))
    say(f"  soft(lambda=200) vs hard: max|dO|={d.max():.2e} max|dLSE|={dl.max():.2e}")
    assert d.max() <= 2e-2 and dl.max() <= 2e-3


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (4, 2)])
def test_soft_custom_scale(Hq, Hkv):
    """A caller-given logit scale: the bias-row path (G >= 8) divides the biases by it and adds
    the row shift back in natural units; the per-element path (G < 8) adds the biases directly.
    Scale 0.3 at head size 64 (logit spread about 2.4), as in the attention tests: at head size
    128 the softmax is so peaked that bf16 weights and outputs alone approach the 2e-2 bound."""
    from learned_centroid_gated_amd import focus_soft_attention
    n, dh, K, k, w, lam, scale = 800, 64, 9, 2, 50, 7.0, 0.3
    say(f"soft custom scale Hq={Hq} Hkv={Hkv} scale={scale}")
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=611)
    groups = random_groups(n, K, k, np.random.default_rng(611))
    out, lse = focus_soft_attention(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]),
                                    i32_dev(groups), K, w, lam, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = soft_gate_ref(t["q"], t["k"], t["v"], groups, w, lam, scale=scale, with_lse=True)
    check_attention(out, lse, o_ref, l_ref, "soft, scale 0.3")
