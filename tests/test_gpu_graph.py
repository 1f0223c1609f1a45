"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed: a decode
step against per-sequence caches, the allocation-free decode, and a whole prefill step (assign,
bucket, attention). Every replay must reproduce an eager call on the same inputs bit for bit.
New inputs are copied into the captured buffers before each replay, and eager work and
synchronisations run between the replays."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, f32_dev, i32_dev, say
from synth import assign_inputs, qkv_inputs, random_groups

pytestmark = pytest.mark.gpu
REPLAYS = 3


def _capture(fn):
    """fn() once eagerly (which also settles the library's cached launch parameters), then
    captured into a graph; returns the graph and the captured call's outputs."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def _replays_match(g, outs, step, new_inputs, names):
    for r in range(1, REPLAYS + 1):
        new_inputs(r)
        g.replay()
        torch.cuda.synchronize()
        filler = torch.randn(1 << 20, device="cuda")  # eager work between the replays
        _ = float(filler.sum())
        eager = step()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, eager):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"
        say(f"  replay {r}: {', '.join(names)} equal to the eager call")


def _decode_setup(B, L, Hq, Hkv, dh, K, k, seed):
    from learned_centroid_gated_amd import focus_bucket
    rng = np.random.default_rng(seed)
    t = qkv_inputs(L, Hq, Hkv, dh, index=0, salt=seed, lead=(B,), which="kv")
    kc, vc = bf16_dev(t["k"]), bf16_dev(t["v"])
    cache_groups = i32_dev(np.stack([random_groups(L, K, k, rng) for _ in range(B)]))
    lens = i32_dev(np.array([L, L - 5, 1000, 3][:B], np.int32))
    off, idx, _ = focus_bucket(cache_groups, K)
    q = torch.empty((B, Hq, dh), dtype=torch.bfloat16, device="cuda")
    qg = torch.empty((B, k), dtype=torch.int32, device="cuda")

    def new_inputs(r):
        qq = qkv_inputs(1, Hq, Hkv, dh, index=r, salt=seed + 1, lead=(B,), which="q")["q"][:, 0]
        q.copy_(bf16_dev(qq))
        qg.copy_(i32_dev(np.stack([random_groups(1, K, k, rng)[0] for _ in range(B)])))
    return kc, vc, cache_groups, lens, off, idx, q, qg, new_inputs


def test_decode_step_graph_replays():
    from learned_centroid_gated_amd import focus_decode
    B, L, Hq, Hkv, dh, K, k, w = 4, 2048, 32, 8, 128, 64, 2, 256
    say(f"graph: decode B={B} L={L} Hq={Hq}/{Hkv} K={K} top_k={k} window={w}")
    kc, vc, cg, lens, off, idx, q, qg, new_inputs = _decode_setup(B, L, Hq, Hkv, dh, K, k, 910)
    new_inputs(0)

    def step():
        return focus_decode(q, qg, kc, vc, lens, cg, off, idx, K, w)
    g, outs = _capture(step)
    _replays_match(g, outs, step, new_inputs, ("out", "lse"))


def test_decode_noalloc_graph_replays():
    from learned_centroid_gated_amd import focus_decode_noalloc
    B, L, Hq, Hkv, dh, K, k, w = 3, 1500, 16, 2, 64, 16, 1, 64
    say(f"graph: allocation-free decode B={B} L={L} Hq={Hq}/{Hkv} K={K} top_k={k} window={w}")
    kc, vc, cg, lens, off, idx, q, qg, new_inputs = _decode_setup(B, L, Hq, Hkv, dh, K, k, 920)
    new_inputs(0)

    def step():
        return focus_decode_noalloc(q, qg, kc, vc, lens, cg, off, idx, K, w)
    g, outs = _capture(step)
    _replays_match(g, outs, step, new_inputs, ("out", "lse"))


def test_prefill_step_graph_replays():
    from learned_centroid_gated_amd import focus_assign, focus_attention, focus_bucket
    n, d, dg, K, k, iters = 4097, 512, 128, 64, 2, 3
    Hq, Hkv, dh, w = 16, 4, 128, 256
    say(f"graph: prefill step n={n} d={d} K={K} top_k={k} Hq={Hq}/{Hkv} window={w}")
    a = assign_inputs(n, d, dg, K, K, index=0, salt=930)
    hidden, w_g, cents = f32_dev(a["hidden"]), f32_dev(a["w_g"]), f32_dev(a["centroids"])
    t = qkv_inputs(n, Hq, Hkv, dh, index=0, salt=931)
    q, kk, v = bf16_dev(t["q"]), bf16_dev(t["k"]), bf16_dev(t["v"])

    def new_inputs(r):
        a2 = assign_inputs(n, d, dg, K, K, index=r, salt=930)
        t2 = qkv_inputs(n, Hq, Hkv, dh, index=r, salt=931)
        hidden.copy_(f32_dev(a2["hidden"]))
        q.copy_(bf16_dev(t2["q"]))
        kk.copy_(bf16_dev(t2["k"]))
        v.copy_(bf16_dev(t2["v"]))

    def step():
        groups, col_v = focus_assign(hidden, w_g, cents, k, iters)
        off, idx, slot = focus_bucket(groups, K)
        out, lse = focus_attention(q, kk, v, groups, off, idx, slot, K, w)
        return groups, col_v, out, lse
    g, outs = _capture(step)
    _replays_match(g, outs, step, new_inputs, ("groups", "col_potential", "out", "lse"))
