"""focus_attention_asym on the GPU against the oracle's asymmetric top-k rule (every key in one
group, every query looking at top_k groups), both fed the same memberships.

Every row at sizes the oracle finishes in seconds (several tiles, ragged tails), sampled rows
at the 128K-token layer in the benchmarked launch configuration, and the Q = 0 pair-count
probe over every row (exp(lse_i) equals the exact number of allowed keys)."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, check_attention, i32_dev, say, to_np
from oracle import assign_ref, attention_rows_asym_ref, pair_count_asym_ref
from synth import CONFIGS, assign_inputs, qkv_inputs, random_groups

pytestmark = pytest.mark.gpu


def run_asym(q, k, v, q_groups_dev, k_group_dev, K, window, scale=0.0):
    from learned_centroid_gated_amd import focus_attention_asym, focus_bucket
    qb = focus_bucket(q_groups_dev, K)
    kb = focus_bucket(k_group_dev.reshape(-1, 1).contiguous(), K)
    out, lse = focus_attention_asym(q, k, v, qb, kb, K, window, scale)
    torch.cuda.synchronize()
    return out, lse


def asym_groups(n, K, kq, seed, skew=0.0, inside=True):
    """Query groups [n, kq] ascending; key group [n]: one of the token's own query groups
    (as top-1 lies in top-k) or, with inside=False, any group."""
    rng = np.random.default_rng(seed)
    qg = random_groups(n, K, kq, rng, skew=skew)
    if inside:
        kg = qg[np.arange(n), rng.integers(0, kq, size=n)]
    else:
        kg = random_groups(n, K, 1, rng, skew=skew)[:, 0]
    return qg, kg.astype(np.int32)


CASES = [
    # n, Hq, Hkv, dh, K, top_k, window, skew, inside
    (1, 1, 1, 64, 1, 1, 1, 0, True),
    (2, 4, 1, 128, 2, 1, 0, 0, True),
    (63, 2, 1, 64, 4, 2, 1, 0, True),
    (65, 16, 1, 128, 3, 3, 2, 0, True),
    (127, 4, 4, 64, 16, 2, 126, 0, True),
    (300, 8, 1, 128, 16, 2, 0, 0, True),
    (1000, 4, 1, 128, 4, 2, 64, 0, True),
    (1000, 12, 12, 64, 16, 1, 128, 0, True),
    (999, 4, 2, 128, 8, 2, 2000, 0, True),
    (4097, 8, 2, 128, 16, 2, 200, 0, True),
    (2000, 64, 8, 128, 128, 2, 1024, 1.1, True),
    (3000, 32, 8, 128, 256, 3, 512, 0, True),
    (1500, 8, 8, 64, 5, 4, 33, 0.7, True),
    (1700, 16, 4, 128, 12, 2, 50, 0, False),
    (3000, 16, 1, 64, 1024, 4, 100, 0, True),   # largest K and top_k, G = 16
    (800, 8, 2, 64, 4, 3, 1, 0, False),
]


@pytest.mark.parametrize("n,Hq,Hkv,dh,K,k,w,skew,inside", CASES)
def test_asym_matches_oracle(n, Hq, Hkv, dh, K, k, w, skew, inside):
    say(f"asym n={n} Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w} skew={skew} "
        f"inside={inside}")
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=3000 + n + K)
    qg, kg = asym_groups(n, K, k, n * 5 + K, skew, inside)
    out, lse = run_asym(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(qg),
                        i32_dev(kg), K, w)
    o_ref, l_ref = attention_rows_asym_ref(t["q"], t["k"], t["v"], qg, kg, w)
    check_attention(out, lse, o_ref, l_ref, f"asym n={n} K={K} k={k} w={w}")


def test_asym_rows_without_allowed_keys():
    """Window 0 with key groups drawn apart from the query groups: rows whose key group is not
    among their own query groups and that meet no earlier key of their groups have no pair at
    all; they must come out with lse -inf and out 0, and every other row as the oracle."""
    n, Hq, Hkv, dh, K, k = 900, 8, 2, 128, 6, 1
    say(f"asym empty rows n={n} K={K} top_k={k} window=0")
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=77)
    qg, kg = asym_groups(n, K, k, 77, inside=False)
    out, lse = run_asym(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(qg),
                        i32_dev(kg), K, 0)
    o_ref, l_ref = attention_rows_asym_ref(t["q"], t["k"], t["v"], qg, kg, 0)
    empty = ~np.isfinite(l_ref[:, 0])
    say(f"  rows without keys: {int(empty.sum())}")
    assert empty.any() and not empty.all()
    lse_h, out_h = to_np(lse), to_np(out)
    assert np.all(lse_h[empty] == -np.inf)
    assert np.all(out_h[empty] == 0)
    keep = torch.from_numpy(np.nonzero(~empty)[0]).cuda()
    check_attention(out[keep], lse[keep], o_ref[~empty], l_ref[~empty], "asym window 0, non-empty rows")


def test_asym_custom_scale():
    n, Hq, Hkv, dh, K, k, w = 700, 4, 2, 64, 8, 2, 40
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=7)
    qg, kg = asym_groups(n, K, k, 7)
    out, lse = run_asym(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(qg),
                        i32_dev(kg), K, w, scale=0.3)
    o_ref, l_ref = attention_rows_asym_ref(t["q"], t["k"], t["v"], qg, kg, w, scale=0.3)
    check_attention(out, lse, o_ref, l_ref, "asym scale=0.3")


@pytest.mark.parametrize("n,Hq,Hkv,K,k,w", [(20000, 8, 2, 16, 2, 100), (9000, 4, 4, 4, 2, 0),
                                            (6000, 16, 1, 7, 4, 300)])
def test_asym_q_zero_counts_every_pair_once(n, Hq, Hkv, K, k, w):
    say(f"asym Q=0 probe n={n} K={K} k={k} w={w}")
    t = qkv_inputs(n, Hq, Hkv, 128, index=0, salt=35)
    q0 = torch.zeros((n, Hq, 128), dtype=torch.bfloat16, device="cuda")
    qg, kg = asym_groups(n, K, k, n + k)
    _, lse = run_asym(q0, bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(qg), i32_dev(kg), K, w)
    counts = pair_count_asym_ref(qg, kg, w).astype(np.float64)
    got = np.exp(to_np(lse).astype(np.float64))
    rel = np.abs(got - counts[:, None]) / counts[:, None]
    say(f"  max rel err of exp(lse) vs pair count: {rel.max():.2e}")
    assert rel.max() < 2e-5


def test_asym_deterministic():
    n, Hq, Hkv, dh, K, k, w = 5000, 16, 4, 128, 32, 2, 256
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=11)
    qg, kg = asym_groups(n, K, k, 11)
    q, kk, v = bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"])
    o1, l1 = run_asym(q, kk, v, i32_dev(qg), i32_dev(kg), K, w)
    o2, l2 = run_asym(q, kk, v, i32_dev(qg), i32_dev(kg), K, w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_asym_workload_with_oracle_memberships():
    """The 2K-token layer with the oracle's own assignment: query groups = top-k, key group =
    top-1 of the same balanced scores; every row."""
    c = [x for x in CONFIGS if x.name == "gpt2s_n2k"][0]
    say(f"asym attention on {c.name} with oracle memberships")
    a = assign_inputs(c.n, c.d, c.dg, c.K, c.mix, c.weights, c.noise_frac, index=c.index)
    kq = max(c.top_k, 2)
    qg = assign_ref(a["hidden"], a["w_g"], a["centroids"], kq, c.iters)["groups"]
    kg = assign_ref(a["hidden"], a["w_g"], a["centroids"], 1, c.iters)["groups"][:, 0]
    del a
    t = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index)
    out, lse = run_asym(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(qg),
                        i32_dev(kg), c.K, c.window)
    o_ref, l_ref = attention_rows_asym_ref(t["q"], t["k"], t["v"], qg, kg, c.window)
    check_attention(out, lse, o_ref, l_ref, c.name)


class _RowsOnly:
    """Stands in for q [n, Hq, dh] when only some rows were copied to the host."""

    def __init__(self, n, rows, values):
        self.shape = (n,) + values.shape[1:]
        self._rows = {int(r): values[i] for i, r in enumerate(rows)}

    def __getitem__(self, i):
        return self._rows[int(i)]


@pytest.mark.parametrize("K,k", [(128, 2), (4, 2)])
def test_asym_full_size_sampled(K, k):
    """The 128K-token 70B-shaped layer in the benchmarked launch configuration (K groups,
    queries looking at k of them): sampled rows against the oracle and the Q = 0 probe over
    every row."""
    c = [x for x in CONFIGS if x.name == "gqa70b_n128k"][0]
    say(f"full-size asym attention {c.name}: n={c.n} K={K} top_k={k}")
    t = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index, device="cuda")
    qg, kg = asym_groups(c.n, K, k, c.index + K)
    qd, kd = i32_dev(qg), i32_dev(kg)
    out, lse = run_asym(t["q"], t["k"], t["v"], qd, kd, K, c.window)
    rng = np.random.default_rng(c.index)
    # at K = 4 a late row attends about half the sequence: fewer rows keep the oracle quick
    nrand, ntail = (30, 6) if K > 8 else (4, 2)
    rows = np.unique(np.concatenate([np.arange(6), np.arange(c.window - 3, c.window + 3),
                                     np.arange(c.n - ntail, c.n),
                                     rng.choice(c.n, nrand, replace=False)]))
    rows_t = torch.from_numpy(rows).cuda()
    q_rows = t["q"][rows_t].view(torch.int16).cpu().numpy().view(np.uint16)
    k_host = t["k"].view(torch.int16).cpu().numpy().view(np.uint16)
    v_host = t["v"].view(torch.int16).cpu().numpy().view(np.uint16)
    o_ref, l_ref = attention_rows_asym_ref(_RowsOnly(c.n, rows, q_rows), k_host, v_host, qg, kg,
                                           c.window, rows=rows)
    check_attention(out[rows_t], lse[rows_t], o_ref, l_ref, f"asym 128K K={K}")
    del out, lse, k_host, v_host
    q0 = torch.zeros_like(t["q"])
    del t["q"]
    torch.cuda.empty_cache()
    _, lse0 = run_asym(q0, t["k"], t["v"], qd, kd, K, c.window)
    counts = pair_count_asym_ref(qg, kg, c.window).astype(np.float64)
    got = np.exp(to_np(lse0).astype(np.float64))
    rel = np.abs(got - counts[:, None]) / counts[:, None]
    say(f"  Q=0 probe over {c.n} rows: max rel err {rel.max():.2e}, pairs={counts.sum():.4e}")
    assert rel.max() < 2e-5
    del q0, lse0, t
    torch.cuda.empty_cache()
