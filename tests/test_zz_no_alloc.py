"""focus_decode_noalloc (decode with the library's fixed per-GPU scratch, for callers that
cannot allocate) through the C ABI, against focus_decode with a workspace: two calls in a row,
the second with fewer and shorter sequences, each bit-identical to the workspace entry point's
result on the same inputs and within tolerance of the oracle. (The refusal of a call that needs
more scratch than the array holds is checked on the host in test_abi.py.)"""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, check_attention, i32_dev, say
from oracle import decode_ref
from synth import qkv_inputs, random_groups

pytestmark = pytest.mark.gpu


def _case(B, L, Hq, Hkv, dh, K, top_k, window, salt):
    rng = np.random.default_rng(salt)
    t = qkv_inputs(L, Hq, Hkv, dh, index=4, salt=salt, lead=(B,))
    cache_groups = np.stack([random_groups(L, K, top_k, rng) for _ in range(B)])
    lens = rng.integers(max(1, L // 2), L + 1, size=B).astype(np.int32)
    lens[0] = L
    q_groups = random_groups(B, K, top_k, rng)
    q = np.ascontiguousarray(t["q"][:, -1])  # one fresh query row per sequence
    return dict(k=t["k"], v=t["v"], q=q, lens=lens, cache_groups=cache_groups, q_groups=q_groups,
                K=K, window=window)


def _run_both(c):
    import learned_centroid_gated_amd as F
    q, k, v = bf16_dev(c["q"]), bf16_dev(c["k"]), bf16_dev(c["v"])
    cg, qg, lens = i32_dev(c["cache_groups"]), i32_dev(c["q_groups"]), i32_dev(c["lens"])
    off, idx, _ = F.focus_bucket(cg, c["K"])
    out_w, lse_w = F.focus_decode(q, qg, k, v, lens, cg, off, idx, c["K"], c["window"])
    out_n, lse_n = F.focus_decode_noalloc(q, qg, k, v, lens, cg, off, idx, c["K"], c["window"])
    torch.cuda.synchronize()
    return out_w, lse_w, out_n, lse_n


def test_noalloc_decode_matches_workspace_decode_twice():
    cases = [_case(6, 1500, 8, 2, 128, 16, 2, 64, 900),   # larger first
             _case(3, 700, 8, 2, 128, 16, 2, 64, 901)]    # then fewer, shorter sequences
    for i, c in enumerate(cases):
        say(f"noalloc decode call {i}: B={len(c['lens'])} Lmax={c['k'].shape[1]}")
        out_w, lse_w, out_n, lse_n = _run_both(c)
        assert torch.equal(out_w.view(torch.int16), out_n.view(torch.int16)), "out differs"
        assert torch.equal(lse_w, lse_n), "lse differs"
        o_ref, l_ref = decode_ref(c["q"], c["q_groups"], c["k"], c["v"], c["lens"],
                                  c["cache_groups"], c["window"])
        check_attention(out_n, lse_n, o_ref, l_ref, f"noalloc decode call {i}")
