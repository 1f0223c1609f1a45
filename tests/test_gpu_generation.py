"""A few generation steps through every piece of incremental decode: each new token's K/V goes
into a paged pool (a fresh page, taken from the pool in a random order, when the last one is
full), its memberships join the bucketed cache memberships through focus_bucket_append, and
focus_decode_paged attends. Every step is checked against the oracle's decode on the logical
caches."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, check_attention, i32_dev, say
from oracle import decode_ref
from synth import qkv_inputs, random_groups

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Hq,Hkv,dh,K,k,w,page", [(16, 2, 128, 12, 2, 24, 16),
                                                  (8, 8, 64, 5, 1, 1, 7),
                                                  (32, 8, 128, 64, 3, 40, 32)])
def test_generation_steps_paged_with_append(Hq, Hkv, dh, K, k, w, page):
    from learned_centroid_gated_amd import focus_bucket, focus_bucket_append, focus_decode_paged
    B, steps = 3, 6
    L0 = np.array([100, 37, 250], np.int32)
    pps = -(-(int(L0.max()) + steps) // page) + 1
    Lmax = pps * page
    say(f"generation Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w} page={page}")
    rng = np.random.default_rng(Hq + K + page)
    t = qkv_inputs(Lmax, Hq, Hkv, dh, index=0, salt=900 + page, lead=(B,))  # logical caches
    groups = np.stack([random_groups(Lmax, K, k, rng) for _ in range(B)]).astype(np.int32)
    kc, vc = bf16_dev(t["k"]), bf16_dev(t["v"])

    num_pages = B * pps + 4
    free = [int(x) for x in rng.permutation(num_pages)]
    table = np.full((B, pps), -1, np.int32)
    kp = torch.zeros((num_pages, page, Hkv, dh), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)

    def store(b, lo, hi):  # K/V of positions [lo, hi) of sequence b into the pool
        for pos in range(lo, hi):
            pg = pos // page
            if table[b, pg] < 0:
                table[b, pg] = free.pop()
            kp[int(table[b, pg]), pos % page] = kc[b, pos]
            vp[int(table[b, pg]), pos % page] = vc[b, pos]

    g_now = groups.copy()
    for b in range(B):
        store(b, 0, int(L0[b]))
        g_now[b, L0[b]:] = -1  # tokens not generated yet
    off, idx, _ = focus_bucket(i32_dev(g_now), K)
    lens = L0.copy()
    for step in range(steps):
        lens = lens + 1
        new_g = np.stack([groups[b, lens[b] - 1] for b in range(B)])
        for b in range(B):
            store(b, int(lens[b]) - 1, int(lens[b]))
            g_now[b, lens[b] - 1] = new_g[b]
        off, idx = focus_bucket_append(i32_dev(new_g), i32_dev(lens), off, idx, K, Lmax)
        qd = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
        out, lse = focus_decode_paged(bf16_dev(qd), i32_dev(new_g), kp, vp, i32_dev(table),
                                      i32_dev(lens), i32_dev(g_now), off, idx, K, w)
        torch.cuda.synchronize()
        o_ref, l_ref = decode_ref(qd, new_g, t["k"], t["v"], lens, g_now, w)
        check_attention(out, lse, o_ref, l_ref, f"generation step {step}, lens {lens.tolist()}")
