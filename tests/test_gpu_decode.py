"""focus_decode on the GPU against the oracle's decode, and against the last prefill row."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, check_attention, i32_dev, say, to_np
from oracle import assign_ref, decode_ref
from synth import CONFIGS, assign_inputs, qkv_inputs, random_groups

pytestmark = pytest.mark.gpu


def run_decode(qd, q_groups, kc, vc, lens, cache_groups, K, window):
    from learned_centroid_gated_amd import focus_bucket, focus_decode
    off, idx, _ = focus_bucket(cache_groups, K)
    out, lse = focus_decode(qd, q_groups, kc, vc, lens, cache_groups, off, idx, K, window)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("B,L,Hq,Hkv,dh,K,k,w", [
    (5, 300, 8, 2, 128, 8, 2, 16),
    (3, 513, 4, 4, 64, 5, 1, 0),
    (4, 1000, 16, 2, 128, 16, 3, 1),
    (2, 2000, 32, 8, 128, 64, 2, 256),
    (6, 257, 2, 1, 64, 3, 2, 400),
    (2, 700, 64, 8, 128, 16, 2, 32),
    (3, 900, 32, 2, 64, 16, 1, 64),
    (2, 3000, 16, 1, 64, 1024, 4, 100),  # largest K and top_k, G = 16
])
def test_decode_matches_oracle(B, L, Hq, Hkv, dh, K, k, w):
    say(f"decode B={B} L={L} Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w}")
    rng = np.random.default_rng(B * L + K)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=400 + L, lead=(B,))
    cache_groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)])
    q_groups = np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])
    lens = np.array([L, 1, 2, L - 1, max(1, L // 3), 7][:B], np.int32)
    qd = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
    out, lse = run_decode(bf16_dev(qd), i32_dev(q_groups), bf16_dev(t["k"]), bf16_dev(t["v"]),
                          i32_dev(lens), i32_dev(cache_groups), K, w)
    o_ref, l_ref = decode_ref(qd, q_groups, t["k"], t["v"], lens, cache_groups, w)
    check_attention(out, lse, o_ref, l_ref, "decode")


@pytest.mark.parametrize("B", [200, 520])
def test_decode_large_batch(B):
    """Many short sequences: the key lists are cut into two pieces (200 sequences) or one
    (520), so each sequence's partial covers its whole list; lengths from 1 to L."""
    L, Hq, Hkv, dh, K, k, w = 50, 8, 2, 64, 4, 2, 8
    say(f"decode large batch B={B} L={L} Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w}")
    rng = np.random.default_rng(B)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=450 + B, lead=(B,))
    cache_groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)])
    q_groups = np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])
    lens = rng.integers(1, L + 1, B).astype(np.int32)
    qd = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
    out, lse = run_decode(bf16_dev(qd), i32_dev(q_groups), bf16_dev(t["k"]), bf16_dev(t["v"]),
                          i32_dev(lens), i32_dev(cache_groups), K, w)
    o_ref, l_ref = decode_ref(qd, q_groups, t["k"], t["v"], lens, cache_groups, w)
    check_attention(out, lse, o_ref, l_ref, "decode, large batch")


@pytest.mark.parametrize("B,L,Hq,Hkv,dh,K,k,w", [
    (2, 262144, 8, 2, 64, 64, 2, 1024),  # long caches: 128 pieces of about 135 keys per sequence
    (520, 4096, 4, 1, 64, 2, 1, 64),     # one piece per sequence, resolved 1024 entries at a time
])
def test_decode_long_lists(B, L, Hq, Hkv, dh, K, k, w):
    """Long key lists: caches of 262144 tokens, and a batch large enough that each sequence's
    list of about 2100 keys is one piece that a block resolves in several chunks."""
    say(f"decode long lists B={B} L={L} Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w}")
    rng = np.random.default_rng(B * 7 + L)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=470 + B, lead=(B,), which="kv")
    cache_groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)])
    q_groups = np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])
    lens = rng.integers(L // 2, L + 1, B).astype(np.int32)
    lens[0] = L
    qd = qkv_inputs(1, Hq, Hkv, dh, index=0, salt=480 + B, lead=(B,), which="q")["q"][:, 0]
    out, lse = run_decode(bf16_dev(qd), i32_dev(q_groups), bf16_dev(t["k"]), bf16_dev(t["v"]),
                          i32_dev(lens), i32_dev(cache_groups), K, w)
    o_ref, l_ref = decode_ref(qd, q_groups, t["k"], t["v"], lens, cache_groups, w)
    check_attention(out, lse, o_ref, l_ref, "decode, long lists")


def test_decode_query_groups_invalid_or_repeated():
    """Query groups outside [0, K) match no key and a repeated query group counts once, as in
    the oracle (whose rule compares ids: the caches hold only valid ones); a query with no
    valid group sees its window and itself."""
    B, L, Hq, Hkv, dh, K, k, w = 5, 1500, 8, 2, 128, 16, 3, 64
    say(f"decode with invalid and repeated query groups B={B} L={L} K={K} top_k={k}")
    rng = np.random.default_rng(61)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=461, lead=(B,), which="kv")
    cache_groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)])
    q_groups = np.array([[-1, 3, 7], [5, 5, 9], [20, -4, 2], [-1, -1, -1], [4, 4, 4]], np.int32)
    lens = np.array([L, L - 7, 900, 321, L], np.int32)
    qd = qkv_inputs(1, Hq, Hkv, dh, index=0, salt=462, lead=(B,), which="q")["q"][:, 0]
    out, lse = run_decode(bf16_dev(qd), i32_dev(q_groups), bf16_dev(t["k"]), bf16_dev(t["v"]),
                          i32_dev(lens), i32_dev(cache_groups), K, w)
    o_ref, l_ref = decode_ref(qd, q_groups, t["k"], t["v"], lens, cache_groups, w)
    check_attention(out, lse, o_ref, l_ref, "decode, invalid and repeated query groups")


def test_decode_equals_last_prefill_row_on_gpu():
    from learned_centroid_gated_amd import focus_attention, focus_bucket
    L, Hq, Hkv, dh, K, k, w = 3000, 16, 4, 128, 32, 2, 128
    rng = np.random.default_rng(7)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=71)
    g = random_groups(L, K, k, rng)
    qd, kd, vd = bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"])
    gd = i32_dev(g)
    off, idx, slot = focus_bucket(gd, K)
    out_p, lse_p = focus_attention(qd, kd, vd, gd, off, idx, slot, K, w)
    out_d, lse_d = run_decode(qd[L - 1:L].contiguous(), gd[L - 1:L].contiguous(), kd[None], vd[None],
                              i32_dev([L]), gd[None].contiguous(), K, w)
    torch.cuda.synchronize()
    diff = (out_p[L - 1].float() - out_d[0].float()).abs().max().item()
    ldiff = (lse_p[L - 1] - lse_d[0]).abs().max().item()
    say(f"  decode vs last prefill row: max|dO|={diff:.2e} max|dLSE|={ldiff:.2e}")
    assert diff <= 1e-2 and ldiff <= 1e-4


def test_decode_workload_oracle_memberships():
    """The decode workload's shape (65536-token caches, 32/8 heads, K=64, top-2, window 256) on
    4 sequences whose cached groups come from the oracle's assignment of mixture hidden states;
    the query groups come from the GPU assignment of fresh hidden states, checked first
    against the oracle."""
    from learned_centroid_gated_amd import focus_assign
    c = [x for x in CONFIGS if x.name == "decode_b64_l64k"][0]
    B = 4
    say(f"decode workload shape with B={B}, L={c.n}")
    cache_groups = []
    for b in range(B):
        a = assign_inputs(c.n, c.d, c.dg, c.K, c.mix, c.weights, index=c.index, salt=b + 1)
        cache_groups.append(assign_ref(a["hidden"], a["w_g"], a["centroids"], c.top_k, c.iters)["groups"])
        del a
    cache_groups = np.stack(cache_groups)
    fresh = assign_inputs(B, c.d, c.dg, c.K, c.mix, c.weights, index=c.index, salt=100)
    ref = assign_ref(fresh["hidden"], fresh["w_g"], fresh["centroids"], c.top_k, c.iters)
    qg_dev, _ = focus_assign(*(torch.from_numpy(fresh[x]).cuda() for x in ("hidden", "w_g", "centroids")),
                             c.top_k, c.iters)
    qg = to_np(qg_dev)
    ok = ~ref["tie"]
    np.testing.assert_array_equal(qg[ok], ref["groups"][ok])
    t = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index, lead=(B,))
    lens = np.full(B, c.n, np.int32)
    qd = np.stack([t["q"][b, c.n - 1] for b in range(B)])
    out, lse = run_decode(bf16_dev(qd), i32_dev(qg), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(lens),
                          i32_dev(cache_groups), c.K, c.window)
    o_ref, l_ref = decode_ref(qd, qg, t["k"], t["v"], lens, cache_groups, c.window)
    check_attention(out, lse, o_ref, l_ref, "decode workload")


def test_decode_custom_scale():
    from learned_centroid_gated_amd import focus_bucket, focus_decode
    B, L, Hq, Hkv, dh, K, k, w, scale = 3, 900, 8, 2, 64, 8, 2, 40, 0.3
    rng = np.random.default_rng(31)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=431, lead=(B,))
    cache_groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)])
    q_groups = np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])
    lens = np.array([L, 5, L // 2], np.int32)
    qd = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
    off, idx, _ = focus_bucket(i32_dev(cache_groups), K)
    out, lse = focus_decode(bf16_dev(qd), i32_dev(q_groups), bf16_dev(t["k"]), bf16_dev(t["v"]),
                            i32_dev(lens), i32_dev(cache_groups), off, idx, K, w, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = decode_ref(qd, q_groups, t["k"], t["v"], lens, cache_groups, w, scale=scale)
    check_attention(out, lse, o_ref, l_ref, "decode, scale 0.3")
