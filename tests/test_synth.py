"""The seeded generators are reproducible and round to bf16 like torch (nearest, ties even)."""
import numpy as np
import torch

from synth import CONFIGS, assign_inputs, bf16_round, f32_to_bf16_bits, qkv_inputs


def test_reproducible():
    a = assign_inputs(100, 16, 4, 3, 5, index=1)
    b = assign_inputs(100, 16, 4, 3, 5, index=1)
    c = assign_inputs(100, 16, 4, 3, 5, index=2)
    np.testing.assert_array_equal(a["hidden"], b["hidden"])
    assert not np.array_equal(a["hidden"], c["hidden"])
    q1 = qkv_inputs(10, 2, 1, 8, index=3)
    q2 = qkv_inputs(10, 2, 1, 8, index=3)
    for k in "qkv":
        np.testing.assert_array_equal(q1[k], q2[k])


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).normal(0, 3, 100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -2.0078125, 0.0]  # exact ties and zero
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_mixture_shapes_and_noise_share():
    a = assign_inputs(20000, 8, 4, 4, 4, noise_frac=0.1, index=0)
    assert abs(a["is_noise"].mean() - 0.1) < 0.01
    assert a["hidden"].shape == (20000, 8) and a["w_g"].shape == (8, 4)
    np.testing.assert_allclose(np.linalg.norm(a["centroids"], axis=1), 1.0, rtol=1e-6)


def test_configs_are_consistent():
    for c in CONFIGS:
        assert c.Hq % c.Hkv == 0 and 1 <= c.top_k <= c.K and c.n * c.top_k < 2 ** 31
