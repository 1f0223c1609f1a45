"""focus_decode_paged on the GPU: the caches are scattered into a shared pool of pages in a
random order; results must equal focus_decode on the unpaged caches bit for bit (same keys,
same order, same arithmetic) and the oracle's decode within the attention tolerance."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, check_attention, i32_dev, say
from oracle import decode_ref
from synth import CONFIGS, qkv_inputs, random_groups

pytestmark = pytest.mark.gpu


def page_caches(kc, vc, lens, page, rng, spare=5, clear_unused=False):
    """Scatter [B, Lmax, Hkv, dh] caches into a pool of pages in a random order. Returns
    (k_pages, v_pages, table [B, pages_per_seq]); with clear_unused, table entries of pages
    past a sequence's length are -1."""
    B, Lmax = kc.shape[0], kc.shape[1]
    pps = -(-Lmax // page)
    pad = pps * page - Lmax
    if pad:
        z = torch.zeros((B, pad) + tuple(kc.shape[2:]), dtype=kc.dtype, device=kc.device)
        kc, vc = torch.cat([kc, z], 1), torch.cat([vc, z], 1)
    num_pages = B * pps + spare
    perm = rng.permutation(num_pages)[: B * pps].astype(np.int64)
    shape = (num_pages, page) + tuple(kc.shape[2:])
    kp = torch.zeros(shape, dtype=kc.dtype, device=kc.device)
    vp = torch.zeros(shape, dtype=kc.dtype, device=kc.device)
    pt = torch.from_numpy(perm).to(kc.device)
    kp[pt] = kc.reshape((B * pps, page) + tuple(kc.shape[2:]))
    vp[pt] = vc.reshape((B * pps, page) + tuple(kc.shape[2:]))
    table = perm.reshape(B, pps).astype(np.int32)
    if clear_unused:
        for b in range(B):
            table[b, -(-int(lens[b]) // page):] = -1
    return kp, vp, table


def run_both(qd, q_groups, kc, vc, lens, cache_groups, K, window, page, rng, clear_unused):
    from learned_centroid_gated_amd import focus_bucket, focus_decode, focus_decode_paged
    B, Lmax = kc.shape[0], kc.shape[1]
    kp, vp, table = page_caches(kc, vc, lens, page, rng, clear_unused=clear_unused)
    pps = table.shape[1]
    cg = cache_groups
    if pps * page > Lmax:  # the logical capacity grows to whole pages; the padding is never read
        extra = np.stack([random_groups(pps * page - Lmax, K, cg.shape[2], rng) for _ in range(B)])
        cg = np.concatenate([cg, extra], 1)
    cgd = i32_dev(cg)
    off, idx, _ = focus_bucket(cgd, K)
    out_p, lse_p = focus_decode_paged(qd, q_groups, kp, vp, i32_dev(table), lens, cgd, off, idx, K,
                                      window)
    off0, idx0, _ = focus_bucket(i32_dev(cache_groups), K)
    out_d, lse_d = focus_decode(qd, q_groups, kc, vc, lens, i32_dev(cache_groups), off0, idx0, K,
                                window)
    torch.cuda.synchronize()
    return out_p, lse_p, out_d, lse_d


@pytest.mark.parametrize("B,L,Hq,Hkv,dh,K,k,w,page,clear", [
    (5, 300, 8, 2, 128, 8, 2, 16, 16, False),
    (3, 513, 4, 4, 64, 5, 1, 0, 7, True),
    (4, 1000, 16, 2, 128, 16, 3, 1, 1, False),
    (2, 2000, 32, 8, 128, 64, 2, 256, 64, True),
    (6, 257, 2, 1, 64, 3, 2, 400, 256, True),
    (3, 900, 32, 2, 64, 16, 4, 64, 32, False),
])
def test_paged_decode_equals_unpaged_and_oracle(B, L, Hq, Hkv, dh, K, k, w, page, clear):
    say(f"paged decode B={B} L={L} Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w} "
        f"page={page} clear_unused={clear}")
    rng = np.random.default_rng(B * L + K + page)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=500 + L, lead=(B,))
    cache_groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)])
    q_groups = np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])
    lens = np.array([L, 1, 2, L - 1, max(1, L // 3), 7][:B], np.int32)
    qd = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
    out_p, lse_p, out_d, lse_d = run_both(bf16_dev(qd), i32_dev(q_groups), bf16_dev(t["k"]),
                                          bf16_dev(t["v"]), i32_dev(lens), cache_groups, K, w,
                                          page, rng, clear)
    assert torch.equal(out_p.view(torch.int16), out_d.view(torch.int16))
    assert torch.equal(lse_p, lse_d)
    o_ref, l_ref = decode_ref(qd, q_groups, t["k"], t["v"], lens, cache_groups, w)
    check_attention(out_p, lse_p, o_ref, l_ref, "paged decode")


def test_paged_decode_workload_shape():
    """The decode workload (64 sequences of 65536 cached tokens, 32/8 heads, K = 64, top-2,
    window 256) in 16-token pages: equal to the unpaged decode bit for bit."""
    c = [x for x in CONFIGS if x.name == "decode_b64_l64k"][0]
    B, L = c.batch, c.n
    say(f"paged decode workload B={B} L={L} page=16")
    rng = np.random.default_rng(c.index)
    t = qkv_inputs(L, c.Hq, c.Hkv, c.dh, index=c.index, lead=(B,), device="cuda", which="kv")
    cache_groups = np.stack([random_groups(L, c.K, c.top_k, rng) for _ in range(B)])
    q_groups = np.stack([random_groups(1, c.K, c.top_k, rng)[0] for _ in range(B)])
    lens = rng.integers(L // 2, L + 1, size=B).astype(np.int32)
    qd = torch.randn((B, c.Hq, c.dh), device="cuda").to(torch.bfloat16)
    out_p, lse_p, out_d, lse_d = run_both(qd, i32_dev(q_groups), t["k"], t["v"], i32_dev(lens),
                                          cache_groups, c.K, c.window, 16, rng, True)
    assert torch.equal(out_p.view(torch.int16), out_d.view(torch.int16))
    assert torch.equal(lse_p, lse_d)
    del t
    torch.cuda.empty_cache()
