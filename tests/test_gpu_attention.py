"""focus_attention on the GPU against the oracle, both fed the same memberships.

Element-wise on every row at sizes the oracle finishes in seconds (spanning several tiles and
ragged tails), on sampled rows at the full workload sizes, plus the Q = 0 pair-count probe
(exp(lse_i) equals the exact number of allowed keys, so a pair counted twice shows up)."""
import numpy as np
import pytest
import torch

from gpu_util import (bf16_dev, bucket_expected, check_attention, i32_dev, say, to_np)
from oracle import assign_ref, attention_rows_ref, pair_count_ref
from synth import CONFIGS, assign_inputs, qkv_inputs, random_groups

pytestmark = pytest.mark.gpu


def run_focus(q, k, v, groups_dev, K, window, scale=0.0):
    from learned_centroid_gated_amd import focus_attention, focus_bucket
    off, idx, slot = focus_bucket(groups_dev, K)
    out, lse = focus_attention(q, k, v, groups_dev, off, idx, slot, K, window, scale)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # n, Hq, Hkv, dh, K, top_k, window, skew
    (1, 1, 1, 64, 1, 1, 1, 0),
    (2, 4, 1, 128, 2, 1, 0, 0),
    (63, 2, 1, 64, 4, 2, 1, 0),
    (64, 8, 2, 128, 2, 1, 64, 0),
    (65, 16, 1, 128, 3, 3, 2, 0),
    (127, 4, 4, 64, 16, 2, 126, 0),
    (300, 8, 1, 128, 16, 1, 0, 0),
    (1000, 4, 1, 128, 16, 2, 64, 0),
    (1000, 12, 12, 64, 16, 1, 128, 0),
    (999, 4, 2, 128, 8, 1, 2000, 0),
    (4097, 2, 2, 128, 1, 1, 17, 0),
    (4097, 8, 2, 128, 16, 2, 200, 0),
    (2000, 32, 8, 128, 64, 2, 512, 1.1),
    (2000, 64, 8, 128, 128, 2, 1024, 1.1),
    (3000, 32, 8, 128, 256, 1, 512, 0),
    (1500, 8, 8, 64, 5, 4, 33, 0.7),
    (3000, 16, 1, 64, 1024, 4, 100, 0),   # largest K and top_k, G = 16
    (2500, 16, 1, 128, 1024, 3, 0, 0),
    (1200, 4, 4, 128, 12, 4, 50, 0),      # top-4 at d_head 128, per-element ownership test
    (1200, 16, 4, 128, 10, 4, 64, 0),     # top-4 at d_head 128, ownership as bias rows
]


@pytest.mark.parametrize("n,Hq,Hkv,dh,K,k,w,skew", CASES)
def test_attention_matches_oracle(n, Hq, Hkv, dh, K, k, w, skew):
    say(f"attention n={n} Hq={Hq} Hkv={Hkv} dh={dh} K={K} top_k={k} window={w} skew={skew}")
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=1000 + n + K)
    groups = random_groups(n, K, k, np.random.default_rng(n * 3 + K), skew=skew)
    out, lse = run_focus(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(groups), K, w)
    o_ref, l_ref = attention_rows_ref(t["q"], t["k"], t["v"], groups, w)
    check_attention(out, lse, o_ref, l_ref, f"n={n} K={K} k={k} w={w}")


def test_attention_custom_scale():
    n, Hq, Hkv, dh, K, k, w = 700, 4, 2, 64, 8, 2, 40
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=5)
    groups = random_groups(n, K, k, np.random.default_rng(5))
    out, lse = run_focus(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(groups), K, w,
                         scale=0.3)
    o_ref, l_ref = attention_rows_ref(t["q"], t["k"], t["v"], groups, w, scale=0.3)
    check_attention(out, lse, o_ref, l_ref, "scale=0.3")


@pytest.mark.parametrize("n,Hq,Hkv,K,k,w", [(20000, 8, 2, 16, 2, 100), (9000, 4, 4, 7, 3, 0),
                                            (6000, 16, 1, 1, 1, 6000)])
def test_q_zero_counts_every_pair_once(n, Hq, Hkv, K, k, w):
    say(f"Q=0 probe n={n} K={K} k={k} w={w}")
    t = qkv_inputs(n, Hq, Hkv, 128, index=0, salt=33)
    q0 = torch.zeros((n, Hq, 128), dtype=torch.bfloat16, device="cuda")
    groups = random_groups(n, K, k, np.random.default_rng(n + k))
    out, lse = run_focus(q0, bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(groups), K, w)
    counts = pair_count_ref(groups, w).astype(np.float64)
    got = np.exp(to_np(lse).astype(np.float64))
    rel = np.abs(got - counts[:, None]) / counts[:, None]
    say(f"  max rel err of exp(lse) vs pair count: {rel.max():.2e}")
    assert rel.max() < 2e-5
    rows = np.unique(np.concatenate([np.arange(8), np.linspace(0, n - 1, 24).astype(int)]))
    o_ref, l_ref = attention_rows_ref(np.zeros((n, Hq, 128), np.uint16), t["k"], t["v"], groups, w,
                                      rows=rows)
    check_attention(out[rows], lse[rows], o_ref, l_ref, "Q=0 sampled rows")


def test_attention_deterministic():
    n, Hq, Hkv, dh, K, k, w = 5000, 16, 4, 128, 32, 2, 256
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=9)
    groups = i32_dev(random_groups(n, K, k, np.random.default_rng(9)))
    q, kk, v = bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"])
    o1, l1 = run_focus(q, kk, v, groups, K, w)
    o2, l2 = run_focus(q, kk, v, groups, K, w)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


class _RowsOnly:
    """Stands in for q [n, Hq, dh] when only some rows were copied to the host."""

    def __init__(self, n, rows, values):
        self.shape = (n,) + values.shape[1:]
        self._rows = {int(r): values[i] for i, r in enumerate(rows)}

    def __getitem__(self, i):
        return self._rows[int(i)]


def _sample_rows(n, w, count, seed):
    rng = np.random.default_rng(seed)
    head = np.arange(min(n, 6))
    around_w = np.arange(max(0, w - 3), min(n, w + 3))
    tail = np.arange(max(0, n - 6), n)
    rand = rng.choice(n, size=count, replace=False)
    return np.unique(np.concatenate([head, around_w, tail, rand]))


@pytest.mark.parametrize("name", ["gpt2s_n2k", "gqa7b_n32k"])
def test_attention_workload_with_oracle_memberships(name):
    """The workload's own memberships: oracle assign on its hidden states, all rows for the
    2K-token layer, sampled rows for the 32K-token layer."""
    c = [x for x in CONFIGS if x.name == name][0]
    say(f"attention on {name} with oracle memberships")
    a = assign_inputs(c.n, c.d, c.dg, c.K, c.mix, c.weights, c.noise_frac, index=c.index)
    groups = assign_ref(a["hidden"], a["w_g"], a["centroids"], c.top_k, c.iters)["groups"]
    del a
    t = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index)
    out, lse = run_focus(bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"]), i32_dev(groups), c.K,
                         c.window)
    rows = None if c.n <= 4096 else _sample_rows(c.n, c.window, 120, c.index)
    o_ref, l_ref = attention_rows_ref(t["q"], t["k"], t["v"], groups, c.window, rows=rows)
    if rows is not None:
        out, lse = out[torch.from_numpy(rows).cuda()], lse[torch.from_numpy(rows).cuda()]
    check_attention(out, lse, o_ref, l_ref, name)


@pytest.mark.parametrize("name", ["gqa70b_n128k", "long_n1m"])
def test_attention_full_size_sampled(name):
    """Full 128K / 1M-token layers in the benchmarked launch configuration: sampled rows
    against the oracle, and the Q = 0 pair-count probe over every row."""
    c = [x for x in CONFIGS if x.name == name][0]
    say(f"full-size attention {name}: n={c.n}")
    t = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index, device="cuda")
    groups = random_groups(c.n, c.K, c.top_k, np.random.default_rng(c.index))
    gd = i32_dev(groups)
    out, lse = run_focus(t["q"], t["k"], t["v"], gd, c.K, c.window)
    rows = _sample_rows(c.n, c.window, 40, c.index)
    rows_t = torch.from_numpy(rows).cuda()
    q_rows = t["q"][rows_t].view(torch.int16).cpu().numpy().view(np.uint16)
    k_host = t["k"].view(torch.int16).cpu().numpy().view(np.uint16)
    v_host = t["v"].view(torch.int16).cpu().numpy().view(np.uint16)
    # the oracle reads q only at the sampled rows
    o_ref, l_ref = attention_rows_ref(_RowsOnly(c.n, rows, q_rows), k_host, v_host, groups,
                                      c.window, rows=rows)
    check_attention(out[rows_t], lse[rows_t], o_ref, l_ref, name)
    del out, lse
    # Q = 0: exp(lse) is the exact allowed-pair count of every row
    q0 = torch.zeros_like(t["q"])
    del t["q"]
    torch.cuda.empty_cache()
    _, lse0 = run_focus(q0, t["k"], t["v"], gd, c.K, c.window)
    counts = pair_count_ref(groups, c.window).astype(np.float64)
    got = np.exp(to_np(lse0).astype(np.float64))
    rel = np.abs(got - counts[:, None]) / counts[:, None]
    say(f"  Q=0 probe over {c.n} rows: max rel err {rel.max():.2e}, pairs={counts.sum():.4e}")
    assert rel.max() < 2e-5
    del q0, lse0, t
    torch.cuda.empty_cache()
