"""Group-slotted cache memberships on the GPU: rows filled from a bucket equal the bucket's
segments bit for bit; appends of the newest token, one write per membership, reproduce the rows
of the longer caches; decode over the rows equals decode over the bucket (paged, bit for bit)
and the oracle's decode, also through several generation steps; a too-small capacity raises
the overflow flag."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, bucket_expected, check_attention, i32_dev, say
from oracle import decode_ref
from synth import qkv_inputs, random_groups

pytestmark = pytest.mark.gpu


def _rows_expected(groups, lens, K, cap):
    """numpy: per (sequence, group) the ascending positions of members below lens[b]."""
    B = groups.shape[0]
    rl = np.zeros((B, K), np.int32)
    rp = np.full((B, K, cap), -7, np.int32)
    for b in range(B):
        g = groups[b].copy()
        g[lens[b]:] = -1
        off, idx, _ = bucket_expected(g, K)
        for c in range(K):
            seg = idx[off[c]:off[c + 1]]
            rl[b, c] = len(seg)
            rp[b, c, :len(seg)] = seg
    return rl, rp


def _check_rows(seg_len, seg_pos, rl, rp):
    sl, sp = seg_len.cpu().numpy(), seg_pos.cpu().numpy()
    np.testing.assert_array_equal(sl, rl)
    B, K = sl.shape
    for b in range(B):
        for c in range(K):
            np.testing.assert_array_equal(sp[b, c, :sl[b, c]], rp[b, c, :rl[b, c]])


@pytest.mark.parametrize("B,L,K,k", [(1, 1, 1, 1), (3, 700, 8, 2), (4, 2049, 64, 2), (2, 513, 200, 4)])
def test_rows_from_bucket_and_appends(B, L, K, k):
    from learned_centroid_gated_amd import focus_bucket, focus_slots_append, focus_slots_from_bucket
    rng = np.random.default_rng(B * L + K)
    groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)]).astype(np.int32)
    steps = min(6, L - 1) if L > 1 else 0
    lens = np.full(B, L - steps, np.int32)
    cap = L  # never overflows
    say(f"slots B={B} L={L} K={K} top_k={k} steps={steps}")
    g_prefix = groups.copy()
    for b in range(B):
        g_prefix[b, lens[b]:] = -1
    off, idx, _ = focus_bucket(i32_dev(g_prefix), K)
    seg_len, seg_pos, overflow = focus_slots_from_bucket(off, idx, K, L, cap)
    torch.cuda.synchronize()
    _check_rows(seg_len, seg_pos, *_rows_expected(groups, lens, K, cap))
    for _ in range(steps):
        lens = lens + 1
        new_g = np.stack([groups[b, lens[b] - 1] for b in range(B)]).astype(np.int32)
        focus_slots_append(i32_dev(new_g), i32_dev(lens), seg_len, seg_pos, overflow, K)
    torch.cuda.synchronize()
    _check_rows(seg_len, seg_pos, *_rows_expected(groups, lens, K, cap))
    assert int(overflow.item()) == 0


def test_overflow_flag():
    from learned_centroid_gated_amd import focus_bucket, focus_slots_append, focus_slots_from_bucket
    B, L, K, k = 2, 400, 4, 1
    rng = np.random.default_rng(3)
    groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)]).astype(np.int32)
    g = groups.copy()
    g[:, L - 1] = -1
    off, idx, _ = focus_bucket(i32_dev(g), K)
    sizes = np.stack([np.bincount(g[b, :L - 1, 0], minlength=K) for b in range(B)])
    cap = int(sizes.max())  # room for every member of the prefixes, none for more in the fullest
    bf, gf = np.unravel_index(int(np.argmax(sizes)), sizes.shape)
    seg_len, seg_pos, overflow = focus_slots_from_bucket(off, idx, K, L, cap)
    torch.cuda.synchronize()
    assert int(overflow.item()) == 0
    new_g = np.full((B, 1), gf, np.int32)
    lens = np.where(np.arange(B) == bf, L, 0).astype(np.int32)  # only that sequence grows
    before = seg_len.clone()
    focus_slots_append(i32_dev(new_g), i32_dev(lens), seg_len, seg_pos, overflow, K)
    torch.cuda.synchronize()
    assert int(overflow.item()) == 1
    assert torch.equal(seg_len, before)  # nothing stored
    _, _, ov2 = focus_slots_from_bucket(off, idx, K, L, cap - 1)
    torch.cuda.synchronize()
    assert int(ov2.item()) == 1


def _page_pool(kc, vc, page, rng):
    B, Lmax = kc.shape[0], kc.shape[1]
    pps = Lmax // page
    perm = torch.from_numpy(rng.permutation(B * pps)).cuda()
    kp = torch.empty((B * pps, page) + tuple(kc.shape[2:]), dtype=kc.dtype, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = kc.reshape((B * pps, page) + tuple(kc.shape[2:]))
    vp[perm] = vc.reshape((B * pps, page) + tuple(kc.shape[2:]))
    return kp, vp, perm.to(torch.int32).reshape(B, pps).contiguous()


@pytest.mark.parametrize("B,L,Hq,Hkv,dh,K,k,w,page", [
    (4, 1024, 16, 2, 128, 16, 2, 64, 16),
    (3, 512, 8, 8, 64, 5, 1, 0, 8),
    (2, 2048, 32, 8, 128, 64, 3, 256, 64),
])
def test_decode_slots_equals_bucketed_decode_and_oracle(B, L, Hq, Hkv, dh, K, k, w, page):
    from learned_centroid_gated_amd import (focus_bucket, focus_decode_paged, focus_decode_slots,
                                            focus_slots_from_bucket)
    say(f"decode slots B={B} L={L} Hq={Hq} Hkv={Hkv} K={K} top_k={k} window={w} page={page}")
    rng = np.random.default_rng(L + K)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=950 + L, lead=(B,))
    groups = np.stack([random_groups(L, K, k, rng) for _ in range(B)]).astype(np.int32)
    q_groups = np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])
    lens = np.array([L, 1, L // 3, L - 5][:B], np.int32)
    qd = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
    kp, vp, table = _page_pool(bf16_dev(t["k"]), bf16_dev(t["v"]), page, rng)
    gd = i32_dev(groups)
    off, idx, _ = focus_bucket(gd, K)
    seg_len, seg_pos, overflow = focus_slots_from_bucket(off, idx, K, L, L)
    args = (bf16_dev(qd), i32_dev(q_groups), kp, vp, table, i32_dev(lens), gd)
    out_b, lse_b = focus_decode_paged(*args, off, idx, K, w)
    out_s, lse_s = focus_decode_slots(*args, seg_len, seg_pos, K, w)
    torch.cuda.synchronize()
    assert int(overflow.item()) == 0
    assert torch.equal(out_s.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_s, lse_b)
    o_ref, l_ref = decode_ref(qd, q_groups, t["k"], t["v"], lens, groups, w)
    check_attention(out_s, lse_s, o_ref, l_ref, "decode over slots")


def test_generation_steps_with_slot_appends():
    """Six generation steps: each new token's memberships join their rows in place (one write
    each) and decode reads the rows; every step against the oracle."""
    from learned_centroid_gated_amd import (focus_bucket, focus_decode_slots, focus_slots_append,
                                            focus_slots_from_bucket)
    B, Hq, Hkv, dh, K, k, w, page, steps = 3, 16, 2, 128, 12, 2, 24, 16, 6
    L0 = np.array([100, 37, 250], np.int32)
    Lmax = 272
    rng = np.random.default_rng(77)
    t = qkv_inputs(Lmax, Hq, Hkv, dh, index=0, salt=977, lead=(B,))
    groups = np.stack([random_groups(Lmax, K, k, rng) for _ in range(B)]).astype(np.int32)
    kp, vp, table = _page_pool(bf16_dev(t["k"]), bf16_dev(t["v"]), page, rng)  # K/V all stored
    g_now = groups.copy()
    for b in range(B):
        g_now[b, L0[b]:] = -1
    off, idx, _ = focus_bucket(i32_dev(g_now), K)
    seg_len, seg_pos, overflow = focus_slots_from_bucket(off, idx, K, Lmax, 96)
    lens = L0.copy()
    for step in range(steps):
        lens = lens + 1
        new_g = np.stack([groups[b, lens[b] - 1] for b in range(B)]).astype(np.int32)
        for b in range(B):
            g_now[b, lens[b] - 1] = new_g[b]
        focus_slots_append(i32_dev(new_g), i32_dev(lens), seg_len, seg_pos, overflow, K)
        qd = np.stack([t["q"][b, lens[b] - 1] for b in range(B)])
        out, lse = focus_decode_slots(bf16_dev(qd), i32_dev(new_g), kp, vp, table, i32_dev(lens),
                                      i32_dev(g_now), seg_len, seg_pos, K, w)
        torch.cuda.synchronize()
        o_ref, l_ref = decode_ref(qd, new_g, t["k"], t["v"], lens, g_now, w)
        check_attention(out, lse, o_ref, l_ref, f"slots generation step {step}")
    assert int(overflow.item()) == 0
