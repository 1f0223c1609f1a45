"""focus_soft_train_forward and focus_soft_train_backward on the GPU against the training oracle
(soft_train_forward_ref, soft_train_backward_ref), both sides fed the same fp32 hidden states,
projection and centroids and the same bf16 Q/K/V and upstream gradient.

Tolerances: the forward as the attention tests (max |dO| 2e-2, mean 2e-3, |dLSE| 1e-4). The
backward's gradients carry the rounding of the logit gradient to bf16 for the matrix cores
(relative 2^-9 per term, independent across the thousands of terms of each sum), fp32 products
and fp32 atomic accumulation: each gradient must lie within 2e-2 of its own largest entry
everywhere and within 2e-2 relative in the Frobenius norm; exactly zero where the oracle's is
(no far pair, or lambda = 0). Measured: 1.5e-3 to 2.4e-3 relative in the Frobenius norm, and
8.9e-3 for a gradient that is small through cancellation (no Sinkhorn iteration, |dC| < 5e-4),
where the same per-term rounding weighs more against the result."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, check_attention, f32_dev, say, to_np
from oracle import (soft_assignment_ref, soft_train_backward_ref, soft_train_forward_ref,
                    soft_train_forward_rows_ref)
from synth import CONFIGS, assign_inputs, qkv_inputs
from synth.gen import f32_to_bf16_bits, seed_streams

pytestmark = pytest.mark.gpu

GRAD_MAX = 2e-2
GRAD_FRO = 2e-2


def _inputs(n, d, dg, K, Hq, Hkv, dh, cscale, salt, mix=8):
    a = assign_inputs(n, d, dg, K, mix, index=1, salt=salt)
    t = qkv_inputs(n, Hq, Hkv, dh, index=1, salt=salt)
    dout = f32_to_bf16_bits(seed_streams(1, salt + 1)["q"].standard_normal((n, Hq, dh),
                                                                          dtype=np.float32))
    cents = (a["centroids"] * np.float32(cscale)).astype(np.float32)
    return a["hidden"], a["w_g"], cents, t["q"], t["k"], t["v"], dout


def _check_grad(got, ref, name):
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"  {name}: max|ref|={scale:.3e} max|err|={err.max():.3e} rel fro={fro:.3e}")
    assert np.isfinite(got).all(), name
    if scale == 0.0:
        assert np.all(got == 0.0), f"{name}: the oracle's gradient is exactly zero"
        return
    assert err.max() <= GRAD_MAX * scale, name
    assert fro <= GRAD_FRO, name


def _run(h, w, c, iters, q, k, v, dout, window, lam, want_hidden=True):
    from learned_centroid_gated_amd import focus_soft_train_backward, focus_soft_train_forward
    hd, wd, cd = f32_dev(h), f32_dev(w), f32_dev(c)
    qd, kd, vd, dd = bf16_dev(q), bf16_dev(k), bf16_dev(v), bf16_dev(dout)
    out, lse = focus_soft_train_forward(hd, wd, cd, iters, qd, kd, vd, window, lam)
    dc, dw, dh_ = focus_soft_train_backward(hd, wd, cd, iters, qd, kd, vd, out, lse, dd, window,
                                            lam, want_hidden=want_hidden)
    torch.cuda.synchronize()
    return out, lse, to_np(dc), to_np(dw), (to_np(dh_) if dh_ is not None else None)


CASES = [
    # n, d, dg, K, Hq, Hkv, dh, iters, window, lambda, centroid scale
    (1, 8, 4, 1, 1, 1, 64, 1, 0, 3.0, 1.0),
    (65, 64, 16, 3, 2, 1, 128, 2, 8, 4.0, 4.0),
    (257, 128, 32, 16, 4, 2, 128, 3, 16, -3.0, 4.0),
    (300, 64, 16, 5, 8, 2, 64, 0, 32, 10.0, 2.0),
    (1000, 256, 64, 64, 8, 8, 64, 3, 0, 6.0, 6.0),
    (777, 128, 64, 128, 16, 1, 128, 2, 100, 8.0, 6.0),
    (1100, 64, 32, 33, 32, 2, 128, 1, 64, 5.0, 4.0),
    (640, 32, 8, 8, 16, 2, 64, 3, 1, 12.0, 5.0),
    (520, 96, 16, 16, 12, 12, 64, 3, 700, 4.0, 4.0),   # window >= n: no far pair
    (400, 64, 16, 8, 4, 2, 128, 2, 16, 0.0, 4.0),      # lambda 0: a constant gate
    (600, 128, 64, 64, 16, 4, 128, 2, 48, 6.0, 4.0),   # G 4, 32 tokens, K 64: the 32K shape
    (530, 64, 32, 100, 16, 2, 64, 3, 20, -4.0, 3.0),   # G 8, 16 tokens, K 100, head size 64
]


@pytest.mark.parametrize("n,d,dg,K,Hq,Hkv,dh,iters,window,lam,cscale", CASES)
def test_soft_train_matches_oracle(n, d, dg, K, Hq, Hkv, dh, iters, window, lam, cscale):
    say(f"soft train n={n} d={d} dg={dg} K={K} Hq={Hq}/{Hkv} dh={dh} T={iters} w={window} "
        f"lambda={lam}")
    h, w, c, q, k, v, dout = _inputs(n, d, dg, K, Hq, Hkv, dh, cscale, salt=n + K)
    out, lse, dc, dw, dh_ = _run(h, w, c, iters, q, k, v, dout, window, lam)
    o_ref, l_ref, _ = soft_train_forward_ref(h, w, c, iters, q, k, v, window, lam)
    check_attention(out, lse, o_ref, l_ref, "soft train forward")
    g = soft_train_backward_ref(h, w, c, iters, q, k, v, dout, window, lam)
    _check_grad(dc, g["d_centroids"], "d_centroids")
    _check_grad(dw, g["d_w_g"], "d_w_g")
    _check_grad(dh_, g["d_hidden"], "d_hidden")


def test_soft_train_gpt2_workload():
    """The 2K GPT-2-small-shaped workload in full (d 768, d_g 64, K 16, 12 heads of 64, window
    128, three iterations), with lambda 10, inputs drawn as the benchmark draws them."""
    cfg = [x for x in CONFIGS if x.name == "gpt2s_n2k"][0]
    a = assign_inputs(cfg.n, cfg.d, cfg.dg, cfg.K, cfg.mix, cfg.weights, index=cfg.index)
    t = qkv_inputs(cfg.n, cfg.Hq, cfg.Hkv, cfg.dh, index=cfg.index)
    dout = f32_to_bf16_bits(seed_streams(cfg.index, 31)["q"].standard_normal(
        (cfg.n, cfg.Hq, cfg.dh), dtype=np.float32))
    lam = 10.0
    say(f"soft train {cfg.name}: n={cfg.n}")
    out, lse, dc, dw, _ = _run(a["hidden"], a["w_g"], a["centroids"], cfg.iters, t["q"], t["k"],
                               t["v"], dout, cfg.window, lam, want_hidden=False)
    o_ref, l_ref, _ = soft_train_forward_ref(a["hidden"], a["w_g"], a["centroids"], cfg.iters,
                                             t["q"], t["k"], t["v"], cfg.window, lam)
    check_attention(out, lse, o_ref, l_ref, "soft train forward, 2K workload")
    g = soft_train_backward_ref(a["hidden"], a["w_g"], a["centroids"], cfg.iters, t["q"], t["k"],
                                t["v"], dout, cfg.window, lam)
    _check_grad(dc, g["d_centroids"], "d_centroids")
    _check_grad(dw, g["d_w_g"], "d_w_g")


def test_soft_train_forward_7b_workload_sampled_rows():
    """The 32K 7B-shaped workload's forward (d 4096, d_g 128, K 64, 32/8 heads of 128, window
    512) on stratified rows, lambda 10."""
    cfg = [x for x in CONFIGS if x.name == "gqa7b_n32k"][0]
    from learned_centroid_gated_amd import focus_soft_train_forward
    a = assign_inputs(cfg.n, cfg.d, cfg.dg, cfg.K, cfg.mix, cfg.weights, index=cfg.index,
                      device="cuda")
    t = qkv_inputs(cfg.n, cfg.Hq, cfg.Hkv, cfg.dh, index=cfg.index, device="cuda")
    lam = 10.0
    say(f"soft train forward {cfg.name}: n={cfg.n}")
    out, lse = focus_soft_train_forward(a["hidden"], a["w_g"], a["centroids"], cfg.iters, t["q"],
                                        t["k"], t["v"], cfg.window, lam)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(cfg.n - 8, cfg.n),
                                     rng.integers(0, cfg.n, 24)]))
    g = soft_assignment_ref(a["hidden"].cpu().numpy(), a["w_g"].cpu().numpy(),
                            a["centroids"].cpu().numpy(), cfg.iters)
    bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    o_ref, l_ref = soft_train_forward_rows_ref(g, bits(t["q"]), bits(t["k"]), bits(t["v"]),
                                               cfg.window, lam, rows)
    rows_t = torch.from_numpy(rows).cuda()
    check_attention(out[rows_t], lse[rows_t], o_ref, l_ref, "soft train forward, 32K sampled")
