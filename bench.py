#!/usr/bin/env python
"""Focus inference-path benchmark on one MI355X.

A step is one pass of the prefill hot path over one synthetic sequence with every input already
resident in HBM: focus_assign (scores, Sinkhorn, top-k) -> focus_bucket -> focus_attention
(gather, group pass, window pass with the merge in its epilogue). The headline line is the
128K-token 70B-shaped GQA layer; the 1M-token prefill, the batched decode, a dense causal
baseline on the same GPU, the training-time soft-gate forward and the asymmetric top-k variant
(keys in their top-1 group) are reported beside it. Kernel
times inside focus_attention come from HIP events the library records on its own stream around
each stage (focus_attention_ex).

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--quick] [--decode]
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from learned_centroid_gated_amd import (focus_assign, focus_assign_workspace_size,  # noqa: E402
                                        focus_attention, focus_attention_asym,
                                        focus_attention_asym_workspace_size,
                                        focus_attention_workspace_size,
                                        focus_bucket, focus_bucket_append,
                                        focus_bucket_workspace_size, focus_decode,
                                        focus_decode_paged, focus_decode_slots,
                                        focus_slots_append, focus_slots_from_bucket,
                                        focus_soft_attention, focus_soft_train_backward,
                                        focus_soft_train_forward,
                                        focus_soft_train_workspace_size)
from learned_centroid_gated_amd import _lib  # noqa: E402
from synth import CONFIGS, assign_inputs, qkv_inputs, random_groups  # noqa: E402

METRIC = "Focus prefill tokens/s/GPU at 128K & 1M; attn TFLOP/s as % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ("gather", "tile_prefix", "group_attention", "window_attention_merge")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ measured counters
KERNEL_SRC = os.path.join(ROOT, "learned_centroid_gated_amd", "csrc", "attention_kernels.hip")
COUNTER_FILES = {name: os.path.join(ROOT, "profiles", f"attention_counters_{name}.md")
                 for name in ("gqa70b_n128k", "long_n1m")}
CALIBRATION_BYTES = 1 << 30  # one fp32 negation over 2^28 elements reads and writes 1 GiB each
FLOP_PER_CLOCK = 1024 * 1024  # bf16 MFMA flop per clock: 1024 per SIMD, 1024 SIMDs (256 CUs)


def source_sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_counters(workload):
    """Per-pass figures of the attention kernels from the counter runs summarised in profiles/
    (HBM bytes per launch from FETCH_SIZE / WRITE_SIZE scaled by a plain copy of known size, the
    clock each pass ran at, MFMA busy); None when there is no summary for the workload or the
    attention kernel source changed since the counters were taken."""
    path = COUNTER_FILES.get(workload)
    if not path or not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != source_sha256(KERNEL_SRC):
        return None
    try:
        return {p: {"traffic": float(vals[f"{p}_traffic_bytes_per_launch"]),
                    "clock_ghz": float(vals[f"{p}_clock_ghz"]),
                    "mfma_busy": float(vals[f"{p}_mfma_busy"])} for p in ("group", "window")}
    except (KeyError, ValueError):
        return None


def calibration_copy():
    """One fp32 negation of 2^28 elements (1 GiB read, 1 GiB written): the known-size kernel
    whose FETCH_SIZE/WRITE_SIZE counters scale the counters of the Focus kernels."""
    x = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y


# ------------------------------------------------------------------ HIP events (ctypes)
class Hip:
    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def attention_ex(hip, q, k, v, groups, off, idx, slot, K, window, out, lse, ws, events):
    n, Hq, dh = q.shape
    arr = (ctypes.c_void_p * 8)(*events)
    _lib.call("focus_attention_ex", q.data_ptr(), k.data_ptr(), v.data_ptr(), n, Hq, k.shape[1], dh,
              groups.data_ptr(), off.data_ptr(), idx.data_ptr(), slot.data_ptr(), K,
              groups.shape[1], int(window), 0.0, out.data_ptr(), lse.data_ptr(), ws.data_ptr(),
              ws.numel(), torch.cuda.current_stream().cuda_stream, arr, 8)


# ------------------------------------------------------------------ prefill
def window_pairs(n, w):
    i = np.arange(n, dtype=np.int64)
    return int(np.minimum(i + 1, w).sum())


def count_allowed_pairs(q, k, v, groups, off, idx, slot, K, window):
    """Exact allowed-pair count from the product path's Q = 0 run: every logit is 0, so
    exp(lse_i) is the number of keys row i attends (the tests pin this against the oracle).
    The run uses the benchmarked shapes, so its kernels match the timed ones."""
    q0 = torch.zeros_like(q)
    _, lse = focus_attention(q0, k, v, groups, off, idx, slot, K, window)
    del q0
    counts = torch.exp(lse[:, 0].double()).round().to(torch.int64)
    return int(counts.sum().item())


def sample_rows(n, window, rng):
    """Stratified query rows for the oracle check: the first rows (inside the first window),
    the last rows, and rows drawn uniformly in between."""
    first = np.arange(min(n, 32))
    last = np.arange(max(0, n - 32), n)
    mid = rng.integers(0, n, size=min(n, 64))
    return np.unique(np.concatenate([first, last, mid]))


def prefill_bench(c, steps, warmup, hip, capture=False):
    log(f"[bench] prefill {c.name}: n={c.n} d={c.d} Hq={c.Hq}/{c.Hkv} dh={c.dh} K={c.K} "
        f"top_k={c.top_k} window={c.window} iters={c.iters}")
    t0 = time.time()
    a = assign_inputs(c.n, c.d, c.dg, c.K, c.mix, c.weights, c.noise_frac, index=c.index,
                      device="cuda")
    t = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index, device="cuda")
    hidden, w_g, cents = a["hidden"], a["w_g"], a["centroids"]
    q, k, v = t["q"], t["k"], t["v"]
    dev = q.device
    groups = torch.empty((c.n, c.top_k), dtype=torch.int32, device=dev)
    vpot = torch.empty((c.K,), dtype=torch.float32, device=dev)
    off = torch.empty((c.K + 1,), dtype=torch.int32, device=dev)
    idx = torch.empty((c.n * c.top_k,), dtype=torch.int32, device=dev)
    slot = torch.empty((c.n, c.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((c.n, c.Hq, c.dh), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((c.n, c.Hq), dtype=torch.float32, device=dev)
    ws_a = torch.empty(focus_assign_workspace_size(c.n, c.d, c.dg, c.K), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(focus_bucket_workspace_size(1, c.n, c.K, c.top_k), dtype=torch.uint8, device=dev)
    ws_t = torch.empty(focus_attention_workspace_size(c.n, c.Hq, c.Hkv, c.dh, c.K, c.top_k),
                       dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"[bench]   inputs resident in {time.time() - t0:.1f}s; workspaces "
        f"{(ws_a.numel() + ws_b.numel() + ws_t.numel()) / 2**30:.1f} GiB")

    stage_ev = [[hip.event() for _ in range(8)] for _ in range(steps)]
    call_ev = [[hip.event() for _ in range(3)] for _ in range(steps)]
    rec = hip.h.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream

    def step(i=None):
        if i is not None:
            rec(call_ev[i][0], stream)
        focus_assign(hidden, w_g, cents, c.top_k, c.iters, groups=groups, col_potential=vpot,
                     workspace=ws_a)
        if i is not None:
            rec(call_ev[i][1], stream)
        focus_bucket(groups, c.K, off[None], idx[None], slot[None], workspace=ws_b)
        if i is not None:
            rec(call_ev[i][2], stream)
        attention_ex(hip, q, k, v, groups, off, idx, slot, c.K, c.window, out, lse, ws_t,
                     stage_ev[i] if i is not None else [None] * 8)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.time()
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.time() - wall0
    total_ms = start.elapsed_time(end)
    ms = total_ms / steps
    # the same step replayed from a HIP graph (its launches captured once), checked bit-exact
    # against the last eager step: what the step costs without host launch overhead
    out_eager, groups_eager = out.clone(), groups.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_eager.view(torch.int16)), "graph replay differs"
    assert torch.equal(groups, groups_eager), "graph replay differs"
    del out_eager, groups_eager
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end) / steps
    del graph
    log(f"[bench]   replayed from a HIP graph: {graph_ms:.3f} ms/step")
    cap = None
    if capture:
        # what the oracle leg needs to check this very step: its inputs, its memberships and
        # column potential, and the timed step's output on stratified sample rows
        rows = sample_rows(c.n, c.window, np.random.default_rng(c.index + 11))
        rows_t = torch.from_numpy(rows).to(dev)
        bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
        cap = {"hidden": hidden.cpu().numpy(), "w_g": w_g.cpu().numpy(),
               "centroids": cents.cpu().numpy(), "v": vpot.cpu().numpy(),
               "q": bits(q), "k": bits(k), "v_in": bits(v), "rows": rows,
               "out_rows": out[rows_t].float().cpu().numpy(), "lse_rows": lse[rows_t].cpu().numpy()}
    assign_ms = np.mean([hip.elapsed_ms(e[0], e[1]) for e in call_ev])
    bucket_ms = np.mean([hip.elapsed_ms(e[1], e[2]) for e in call_ev])
    stage_ms = {name: float(np.mean([hip.elapsed_ms(e[2 * s], e[2 * s + 1]) for e in stage_ev]))
                for s, name in enumerate(STAGES)}
    for e in stage_ev + call_ev:
        for x in e:
            hip.destroy(x)

    # effective FLOPs on the exact allowed-pair count (untimed accounting pass)
    pairs = count_allowed_pairs(q, k, v, groups, off, idx, slot, c.K, c.window)
    wpairs = window_pairs(c.n, c.window)
    gpairs = pairs - wpairs
    flops_pair = 4.0 * c.dh * c.Hq
    sizes = torch.bincount(groups.flatten().long(), minlength=c.K).cpu().numpy()
    nk = c.n * c.top_k
    res = {
        "workload": c.name, "n": c.n, "ms_per_step": ms, "wall_s": wall, "steps": steps,
        "tokens_per_s": c.n / (ms / 1e3),
        "graph_ms_per_step": graph_ms, "graph_tokens_per_s": c.n / (graph_ms / 1e3),
        "assign_ms": float(assign_ms), "bucket_ms": float(bucket_ms),
        "attention_stage_ms": stage_ms,
        "allowed_pairs": pairs, "window_pairs": wpairs, "group_pairs": gpairs,
        "density_vs_causal": pairs / (c.n * (c.n + 1) / 2),
        "segment_sizes": {"min": int(sizes.min()), "mean": float(sizes.mean()), "max": int(sizes.max())},
        "pairs_source": "Q = 0 run of the product path (exp(lse) counts each row's keys)",
    }
    # the memberships, kept on the host for the oracle leg's recount of the allowed pairs
    res["_groups"] = groups.cpu().numpy()
    if cap is not None:
        cap["groups"] = res["_groups"]
        res["_capture"] = cap
    attn_ms = stage_ms["group_attention"] + stage_ms["window_attention_merge"]
    res["attention_tflops"] = flops_pair * pairs / (attn_ms * 1e-3) / 1e12
    res["attention_pct_bf16_peak"] = 100 * res["attention_tflops"] / PEAK_BF16_TFLOPS
    res["group_tflops"] = flops_pair * gpairs / (stage_ms["group_attention"] * 1e-3) / 1e12
    res["window_merge_tflops"] = flops_pair * wpairs / (stage_ms["window_attention_merge"] * 1e-3) / 1e12
    # algorithmic bytes of the HBM-bound gather: K and V rows read and written per membership,
    # plus the 16-byte key record written per membership
    gather_bytes = nk * (2 * c.Hkv * c.dh * 2 * 2 + 16)
    res["gather_GBs"] = gather_bytes / (stage_ms["gather"] * 1e-3) / 1e9
    fold = c.d * c.K <= c.d * c.dg + c.dg * c.K
    assign_flops = 2.0 * c.n * c.d * c.K if fold else 2.0 * c.n * (c.d * c.dg + c.dg * c.K)
    # fp32 score products per second (run as three fp16 part products each on the matrix cores)
    res["assign_score_tflops"] = assign_flops / (assign_ms * 1e-3) / 1e12
    res["assign_hidden_GBs"] = c.n * c.d * 4 / (assign_ms * 1e-3) / 1e9
    # the dominant kernel of the step
    dom = max(("group_attention", "window_attention_merge", "gather"), key=lambda s: stage_ms[s])
    if dom != "gather":
        p = gpairs if dom == "group_attention" else wpairs
        ach = flops_pair * p / (stage_ms[dom] * 1e-3) / 1e12
        cnt = measured_counters(c.name)
        pc = cnt["group" if dom == "group_attention" else "window"] if cnt else None
        res["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                           "traffic": pc["traffic"] if pc else None,
                           "algorithmic_per_launch": flops_pair * p, "avg_launch_ms": stage_ms[dom]}
        if pc:
            # the same against the peak at the clock the pass actually ran at (counters)
            peak_clk = FLOP_PER_CLOCK * pc["clock_ghz"] * 1e9 / 1e12
            res["roofline"].update({"clock_ghz": pc["clock_ghz"], "peak_clock_derived": peak_clk,
                                    "frac_clock_derived": ach / peak_clk,
                                    "mfma_busy": pc["mfma_busy"]})
        if cnt:
            for pname, stage, pp in (("group", "group_attention", gpairs),
                                     ("window", "window_attention_merge", wpairs)):
                tf = flops_pair * pp / (stage_ms[stage] * 1e-3) / 1e12
                peak_clk = FLOP_PER_CLOCK * cnt[pname]["clock_ghz"] * 1e9 / 1e12
                res[f"{pname}_pct_clock_derived_peak"] = 100 * tf / peak_clk
    else:
        ach = gather_bytes / (stage_ms[dom] * 1e-3) / 1e9
        res["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": None,
                           "algorithmic_per_launch": gather_bytes, "avg_launch_ms": stage_ms[dom]}
    log(f"[bench]   {ms:.3f} ms/step  {res['tokens_per_s']:.4g} tok/s  stages {stage_ms} "
        f"assign {assign_ms:.3f} bucket {bucket_ms:.3f}")
    # each token's top-1 group from the same assignment (the key side of the asymmetric variant)
    groups1 = torch.empty((c.n, 1), dtype=torch.int32, device=dev)
    focus_assign(hidden, w_g, cents, 1, c.iters, groups=groups1, workspace=ws_a)
    state = dict(q=q, k=k, v=v, groups=groups, groups1=groups1, off=off, idx=idx, slot=slot,
                 out=out, lse=lse, ws_t=ws_t)
    del hidden, w_g, cents, a, t, ws_a, ws_b
    return res, state


def dense_baseline(c, st, hip, reps=2):
    """Dense causal attention on the same GPU: our window kernel with window = n, and torch's
    scaled_dot_product_attention(is_causal=True) on the same Q/K/V."""
    q, k, v = st["q"], st["k"], st["v"]
    out, lse, ws = st["out"], st["lse"], st["ws_t"]
    ev = [hip.event() for _ in range(8)]
    times = []
    for r in range(reps + 1):
        attention_ex(hip, q, k, v, st["groups"], st["off"], st["idx"], st["slot"], c.K, c.n, out,
                     lse, ws, ev)
        torch.cuda.synchronize()
        if r:
            times.append(hip.elapsed_ms(ev[6], ev[7]))  # window attention with merge
    for e in ev:
        hip.destroy(e)
    own_ms = float(np.mean(times))
    causal_flops = 4.0 * c.dh * c.Hq * c.n * (c.n + 1) / 2
    res = {"own_window_kernel_ms": own_ms,
           "own_window_kernel_tflops": causal_flops / (own_ms * 1e-3) / 1e12}
    # the training-time soft gate's forward over the same inputs: every causal pair, far pairs
    # biased by log sigmoid(lambda * (share - 1/2)) from the same memberships (lambda = 10)
    times = []
    for r in range(reps + 1):
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        focus_soft_attention(q, k, v, st["groups"], c.K, c.window, 10.0, out=out, lse=lse)
        e0.record()
        torch.cuda.synchronize()
        if r:
            times.append(s0.elapsed_time(e0))
    res["soft_gate_forward_ms"] = float(np.mean(times))
    res["soft_gate_forward_tflops"] = causal_flops / (res["soft_gate_forward_ms"] * 1e-3) / 1e12
    try:
        G = c.Hq // c.Hkv
        qt = q.permute(1, 0, 2).unsqueeze(0)
        kt = k.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0)
        vt = v.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0)
        times = []
        for r in range(reps + 1):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
            e.record()
            torch.cuda.synchronize()
            if r:
                times.append(s.elapsed_time(e))
        res["torch_sdpa_causal_ms"] = float(np.mean(times))
        res["torch_sdpa_causal_tflops"] = causal_flops / (res["torch_sdpa_causal_ms"] * 1e-3) / 1e12
        del qt, kt, vt
    except Exception as ex:  # report, do not fail the bench
        res["torch_sdpa_causal_error"] = f"{type(ex).__name__}: {str(ex)[:160]}"
    return res


# ------------------------------------------------------------------ asymmetric top-k
def asym_bench(c, st, dense_ms, sym_attn_ms, reps=3):
    """focus_attention_asym on the same Q/K/V: keys in their top-1 group, queries looking at
    top_k groups. Two memberships: the library's own assignment at K groups (query groups =
    the step's top-2, key group = top-1 of the same scores), and the pages' 2-of-4 setting with
    synthetic balanced memberships (4 groups, each token looking at 2, its key group one of
    them). Times the attention call (gather, plan, group pass, window pass with the merge)."""
    q, k, v, out, lse = st["q"], st["k"], st["v"], st["out"], st["lse"]
    dev = q.device
    rng = np.random.default_rng(c.index + 4)
    g4 = random_groups(c.n, 4, 2, rng)
    k4 = g4[np.arange(c.n), rng.integers(0, 2, size=c.n)]
    cases = {
        f"K{c.K}_top{c.top_k}_assigned": (c.K, st["groups"], st["groups1"]),
        "K4_top2_two_of_four": (4, torch.from_numpy(g4).to(dev),
                                torch.from_numpy(k4.astype(np.int32)[:, None].copy()).to(dev)),
    }
    flops_pair = 4.0 * c.dh * c.Hq
    res = {}
    for name, (K, qg, kg) in cases.items():
        qb = focus_bucket(qg, K)
        kb = focus_bucket(kg, K)
        ws = torch.empty(focus_attention_asym_workspace_size(c.n, c.Hq, c.Hkv, c.dh, K,
                                                             qg.shape[1]),
                         dtype=torch.uint8, device=dev)
        times = []
        for r in range(reps + 1):
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            focus_attention_asym(q, k, v, qb, kb, K, c.window, out=out, lse=lse, workspace=ws)
            e0.record()
            torch.cuda.synchronize()
            if r:
                times.append(s0.elapsed_time(e0))
        ms = float(np.mean(times))
        # exact allowed pairs from a Q = 0 run: exp(lse_i) counts row i's keys
        q0 = torch.zeros_like(q)
        _, l0 = focus_attention_asym(q0, k, v, qb, kb, K, c.window, workspace=ws)
        pairs = int(torch.exp(l0[:, 0].double()).round().to(torch.int64).sum().item())
        del q0, l0, ws
        torch.cuda.empty_cache()
        r = {"attention_ms": ms, "allowed_pairs": pairs,
             "density_vs_causal": pairs / (c.n * (c.n + 1) / 2),
             "attention_tflops": flops_pair * pairs / (ms * 1e-3) / 1e12,
             "speedup_vs_own_dense": dense_ms / ms if dense_ms else None}
        if K == c.K:
            r["symmetric_attention_ms"] = sym_attn_ms
        log(f"[bench] asym {name}: {ms:.3f} ms, density {r['density_vs_causal']:.4f}, "
            f"{r['attention_tflops']:.0f} TFLOP/s")
        res[name] = r
    return res


# ------------------------------------------------------------------ training
def train_bench(c, lam=10.0, reps=3):
    """One soft-gated training step on the workload's shapes: the forward over every causal pair
    (gate from the soft assignment) and the backward to the centroids and the projection, with an
    N(0,1) bf16 upstream gradient. Algorithmic flop: forward 4 dh Hq per causal pair; backward
    4 dh Hq per far pair (the logits and dP once; the kernels recompute them on both sides)."""
    log(f"[bench] training step {c.name}: n={c.n} lambda={lam}")
    a = assign_inputs(c.n, c.d, c.dg, c.K, c.mix, c.weights, c.noise_frac, index=c.index,
                      device="cuda")
    t = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index, device="cuda")
    dout = qkv_inputs(c.n, c.Hq, c.Hkv, c.dh, index=c.index, salt=31, device="cuda", which="q")["q"]
    dev = t["q"].device
    ws = torch.empty(focus_soft_train_workspace_size(c.n, c.d, c.dg, c.K, c.Hq, c.iters),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((c.n, c.Hq, c.dh), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((c.n, c.Hq), dtype=torch.float32, device=dev)
    dc = torch.empty((c.K, c.dg), dtype=torch.float32, device=dev)
    dw = torch.empty((c.d, c.dg), dtype=torch.float32, device=dev)
    args = (a["hidden"], a["w_g"], a["centroids"], c.iters, t["q"], t["k"], t["v"])

    def fwd():
        focus_soft_train_forward(*args, c.window, lam, out=out, lse=lse, workspace=ws)

    def bwd():
        focus_soft_train_backward(*args, out, lse, dout, c.window, lam, d_centroids=dc,
                                  d_w_g=dw, workspace=ws)

    fwd()
    bwd()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    f_ms, b_ms = [], []
    for _ in range(reps):
        ev[0].record()
        fwd()
        ev[1].record()
        bwd()
        ev[2].record()
        torch.cuda.synchronize()
        f_ms.append(ev[0].elapsed_time(ev[1]))
        b_ms.append(ev[1].elapsed_time(ev[2]))
    n, w = c.n, min(c.window, c.n)
    causal = n * (n + 1) / 2
    far = (n - w) * (n - w + 1) / 2 if n > w else 0.0  # pairs with i - j >= window
    fl = 4.0 * c.dh * c.Hq
    fm, bm = float(np.median(f_ms)), float(np.median(b_ms))
    res = {"workload": c.name, "lambda": lam, "forward_ms": fm, "backward_ms": bm,
           "step_ms": fm + bm, "tokens_per_s": n / ((fm + bm) * 1e-3),
           "forward_tflops": fl * causal / (fm * 1e-3) / 1e12,
           "backward_tflops_algorithmic": fl * far / (bm * 1e-3) / 1e12,
           "grad_norms": {"d_centroids": float(dc.norm()), "d_w_g": float(dw.norm())}}
    log(f"[bench]   training {c.name}: forward {fm:.3f} ms ({res['forward_tflops']:.0f} TF), "
        f"backward {bm:.3f} ms ({res['backward_tflops_algorithmic']:.0f} TF algorithmic)")
    del a, t, dout, ws
    return res


# ------------------------------------------------------------------ decode
def decode_bench(c, steps, warmup, batch=None):
    B, L = (batch or c.batch), c.n
    log(f"[bench] decode {c.name}: B={B} L={L} Hq={c.Hq}/{c.Hkv} K={c.K} top_k={c.top_k} "
        f"window={c.window}")
    dev = torch.device("cuda:0")
    cache_groups = torch.empty((B, L, c.top_k), dtype=torch.int32, device=dev)
    for b in range(B):  # cached memberships: assignment of each sequence's mixture hidden states
        a = assign_inputs(L, c.d, c.dg, c.K, c.mix, c.weights, index=c.index, salt=b + 1, device="cuda")
        focus_assign(a["hidden"], a["w_g"], a["centroids"], c.top_k, c.iters, groups=cache_groups[b])
        del a
    fresh = assign_inputs(B, c.d, c.dg, c.K, c.mix, c.weights, index=c.index, salt=100, device="cuda")
    q_groups, _ = focus_assign(fresh["hidden"], fresh["w_g"], fresh["centroids"], c.top_k, c.iters)
    t = qkv_inputs(L, c.Hq, c.Hkv, c.dh, index=c.index, device="cuda", lead=(B,), which="kv")
    qd = qkv_inputs(1, c.Hq, c.Hkv, c.dh, index=c.index, salt=1, device="cuda", lead=(B,),
                    which="q")["q"][:, 0].contiguous()
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    off, idx, _ = focus_bucket(cache_groups, c.K)
    out = torch.empty((B, c.Hq, c.dh), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, c.Hq), dtype=torch.float32, device=dev)

    def step():
        focus_decode(qd, q_groups, t["k"], t["v"], lens, cache_groups, off, idx, c.K, c.window,
                     out=out, lse=lse)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        step()
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1e3 / steps
    # keys per query from a Q = 0 decode: exp(lse) counts the allowed keys
    focus_decode(torch.zeros_like(qd), q_groups, t["k"], t["v"], lens, cache_groups, off, idx, c.K,
                 c.window, out=out, lse=lse)
    keys = torch.exp(lse[:, 0].double()).round().sum().item()
    kv_bytes = keys * c.Hkv * c.dh * 2 * 2
    res = {"workload": c.name, "batch": B, "us_per_step": us, "allowed_keys_per_query": keys / B,
           "kv_GBs": kv_bytes / (us * 1e-6) / 1e9}
    res["kv_pct_hbm_peak"] = 100 * res["kv_GBs"] / PEAK_HBM_GBS
    log(f"[bench]   decode {us:.1f} us/step, {keys / B:.0f} keys/query, {res['kv_GBs']:.0f} GB/s")
    out_ref = out.clone()
    focus_decode(qd, q_groups, t["k"], t["v"], lens, cache_groups, off, idx, c.K, c.window,
                 out=out_ref, lse=lse)

    # the same step replayed from a HIP graph: the launch gaps between its three kernels go
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), "graph replay differs"
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    res["graph_us_per_step"] = s.elapsed_time(e) * 1e3 / steps
    log(f"[bench]   decode replayed from a HIP graph {res['graph_us_per_step']:.1f} us/step")
    del graph

    # the same step over a paged cache: 16-token pages scattered through one pool in a seeded
    # random order (focus_decode_paged), checked equal to the unpaged step
    page = 16
    pps = L // page
    perm = torch.from_numpy(np.random.default_rng(c.index).permutation(B * pps)).to(dev)
    kp = torch.empty((B * pps, page, c.Hkv, c.dh), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    kp[perm] = t["k"].reshape(B * pps, page, c.Hkv, c.dh)
    vp[perm] = t["v"].reshape(B * pps, page, c.Hkv, c.dh)
    table = perm.to(torch.int32).reshape(B, pps).contiguous()

    def step_paged():
        focus_decode_paged(qd, q_groups, kp, vp, table, lens, cache_groups, off, idx, c.K,
                           c.window, out=out, lse=lse)

    step_paged()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), "paged decode differs"
    for _ in range(warmup):
        step_paged()
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        step_paged()
    e.record()
    torch.cuda.synchronize()
    res["paged16_us_per_step"] = s.elapsed_time(e) * 1e3 / steps
    res["paged16_kv_GBs"] = kv_bytes / (res["paged16_us_per_step"] * 1e-6) / 1e9
    log(f"[bench]   paged decode (16-token pages) {res['paged16_us_per_step']:.1f} us/step, "
        f"{res['paged16_kv_GBs']:.0f} GB/s")

    # group-slotted memberships (a row of slots per sequence and group): decode over them, and
    # the O(top_k) append of a new token's memberships
    sizes = (off[:, 1:] - off[:, :-1]).max().item()
    gcap = 1 << int(math.ceil(math.log2(sizes + 64)))
    seg_len, seg_pos, overflow = focus_slots_from_bucket(off, idx, c.K, L, gcap)

    def step_slots():
        focus_decode_slots(qd, q_groups, kp, vp, table, lens, cache_groups, seg_len, seg_pos, c.K,
                           c.window, out=out, lse=lse)

    step_slots()
    torch.cuda.synchronize()
    assert int(overflow.item()) == 0, "slot rows overflowed"
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), "slotted decode differs"
    for _ in range(warmup):
        step_slots()
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        step_slots()
    e.record()
    torch.cuda.synchronize()
    res["slots_paged16_us_per_step"] = s.elapsed_time(e) * 1e3 / steps
    res["slots_group_cap"] = gcap
    log(f"[bench]   decode over slot rows (16-token pages) {res['slots_paged16_us_per_step']:.1f} "
        f"us/step (group capacity {gcap})")
    del kp, vp, perm, table, out_ref

    # membership maintenance per step: the newest token of every cache joins the bucketed
    # memberships of the others (focus_bucket_append), against bucketing every cache again
    lens_prev = lens - 1
    g_prev = cache_groups.clone()
    g_prev[:, L - 1, :] = -1  # the newest token not yet assigned
    off_p, idx_p, _ = focus_bucket(g_prev, c.K)
    new_g = cache_groups[:, L - 1, :].contiguous()
    off_o, idx_o = torch.empty_like(off_p), torch.empty_like(idx_p)

    def time_us(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(reps):
            fn()
        e0.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(e0) * 1e3 / reps

    res["append_us"] = time_us(lambda: focus_bucket_append(new_g, lens, off_p, idx_p, c.K, L,
                                                           off_o, idx_o))
    res["rebucket_us"] = time_us(lambda: focus_bucket(cache_groups, c.K))
    moved = 2 * 4 * float(off_p[:, c.K].sum().item())  # index entries read and written
    res["append_GBs"] = moved / (res["append_us"] * 1e-6) / 1e9
    assert torch.equal(off_o, off), "appended offsets differ from the full bucket"
    del lens_prev, g_prev
    log(f"[bench]   append {res['append_us']:.1f} us/step ({res['append_GBs']:.0f} GB/s) vs "
        f"re-bucketing {res['rebucket_us']:.1f} us")
    # the slotted append writes one position per membership (timed on rows that then hold the
    # newest token again; they are not read afterwards)
    res["slots_append_us"] = time_us(lambda: focus_slots_append(new_g, lens, seg_len, seg_pos,
                                                                overflow, c.K))
    log(f"[bench]   slot-row append {res['slots_append_us']:.1f} us/step")
    del seg_len, seg_pos, overflow
    return res


# ------------------------------------------------------------------ oracle on the host
def cpu_baseline(c, cap, prefill):
    """The oracle leg, on the host cores of the same run. It times the untuned oracle on a bounded
    sample of the headline workload and checks the timed step against it:
      - assign_ref over the step's full hidden states (groups bit-exact outside the tie window,
        column potential), timed per token;
      - attention_rows_ref on stratified rows of the full sequence with the step's memberships,
        timed per row and compared with the step's output on those rows;
      - pair_count_ref over every benchmarked workload's memberships, which must equal the
        allowed-pair count behind its effective FLOPs.
    tokens/s = 1 / (assign seconds per token + attention seconds per row)."""
    from oracle import TIE_LOG, assign_ref, attention_rows_ref, pair_count_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:
        threads = None
    cores = len(os.sched_getaffinity(0))
    t0 = time.time()
    ref = assign_ref(cap["hidden"], cap["w_g"], cap["centroids"], c.top_k, c.iters)
    t_assign = time.time() - t0
    same = (ref["groups"] == cap["groups"]).all(axis=1)
    unflagged = int((~same & ~ref["tie"]).sum())
    v_err = float(np.abs(ref["v"] - cap["v"]).max())
    del cap["hidden"]
    rows = cap["rows"]
    t0 = time.time()
    o_ref, l_ref = attention_rows_ref(cap["q"], cap["k"], cap["v_in"], cap["groups"], c.window,
                                      rows=rows)
    t_rows = time.time() - t0
    err = np.abs(cap["out_rows"] - o_ref)
    lerr = np.abs(cap["lse_rows"] - l_ref)
    t0 = time.time()
    pair_checks = {}
    for name, (groups, window, q0_pairs) in prefill.items():
        exact = int(pair_count_ref(groups, window).sum())
        pair_checks[name] = {"pair_count_ref": exact, "q0_run": q0_pairs, "equal": exact == q0_pairs}
    t_pairs = time.time() - t0
    checks = {
        "assign_full_size": {"tokens": c.n, "unflagged_group_mismatches": unflagged,
                             "tie_window_tokens": int(ref["tie"].sum()),
                             "tie_window_mismatches": int((~same & ref["tie"]).sum()),
                             "col_potential_max_abs_err": v_err},
        "attention_rows": {"rows": int(len(rows)), "max_abs_err_out": float(err.max()),
                           "mean_abs_err_out": float(err.mean()),
                           "max_abs_err_lse": float(lerr.max())},
        "allowed_pairs": pair_checks, "pair_count_s": t_pairs,
    }
    log(f"[bench] oracle checks: {json.dumps(checks)}")
    assert unflagged == 0, "the timed step's groups differ from the oracle outside the tie window"
    assert v_err <= 2e-5, "the timed step's column potential differs from the oracle"
    assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-4, "attention rows differ"
    assert all(x["equal"] for x in pair_checks.values()), "Q = 0 pair counts differ from the oracle"
    tok_s = 1.0 / (t_assign / c.n + t_rows / len(rows))
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "blas_threads": threads,
            "kind": "oracle",
            "sample": f"assign_ref over all {c.n} tokens of the {c.name} step ({t_assign:.1f}s) + "
                      f"attention_rows_ref on {len(rows)} stratified rows (first, last and uniform) "
                      f"of the full sequence ({t_rows:.1f}s); tokens/s = 1/(s/token + s/row)",
            "checks": checks}


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--decode", action="store_true",
                    help="only the batched decode workload (prints its own JSON line)")
    ap.add_argument("--decode-batch", type=int, default=None,
                    help="with --decode: sequences per step in place of the workload's 64")
    ap.add_argument("--workload", default=None,
                    help="time one prefill workload only, e.g. long_n1m (prints its own JSON line)")
    ap.add_argument("--train", default=None,
                    help="time the soft-gated training step of one workload only, e.g. gqa7b_n32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB copy, to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the Focus path here runs on a single MI355X and has no "
              "multi-GPU mode (no collectives or sharding are built); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.decode:
        cfg = {x.name: x for x in CONFIGS}
        print(json.dumps(decode_bench(cfg["decode_b64_l64k"], 20, 3, args.decode_batch)),
              flush=True)
        return
    hip = Hip()
    if args.calibrate_copy:
        calibration_copy()
    cfg = {x.name: x for x in CONFIGS}
    if args.train:
        print(json.dumps(train_bench(cfg[args.train])), flush=True)
        return
    if args.workload:
        res, st = prefill_bench(cfg[args.workload], args.steps, args.warmup, hip)
        res.pop("_groups")
        del st
        print(json.dumps(res), flush=True)
        return
    c3 = cfg["gqa70b_n128k"]
    res3, st3 = prefill_bench(c3, args.steps, args.warmup, hip, capture=not args.no_cpu_baseline)
    extra = {}
    prefill = {}  # workload -> (memberships, window, Q = 0 pair count), for the oracle leg

    def keep(c, res):
        prefill[c.name] = (res.pop("_groups"), c.window, res["allowed_pairs"])
        return res
    cap3 = res3.pop("_capture", None)
    keep(c3, res3)
    if not args.quick:
        extra["dense_baseline_128k"] = dense_baseline(c3, st3, hip)
        extra["dense_baseline_128k"]["focus_speedup_vs_own_dense"] = (
            extra["dense_baseline_128k"]["own_window_kernel_ms"] / res3["ms_per_step"])
        sym_attn = sum(res3["attention_stage_ms"].values())
        extra["asym_128k"] = asym_bench(c3, st3, extra["dense_baseline_128k"]["own_window_kernel_ms"],
                                        sym_attn)
    del st3
    torch.cuda.empty_cache()
    if not args.quick:
        res4, st4 = prefill_bench(cfg["long_n1m"], max(3, args.steps // 2), 1, hip)
        extra["long_n1m"] = keep(cfg["long_n1m"], res4)
        del st4
        torch.cuda.empty_cache()
        # the two smaller prefill workloads (2K GPT-2-small-shaped MHA, 32K 7B-shaped GQA)
        for name in ("gpt2s_n2k", "gqa7b_n32k"):
            r, st = prefill_bench(cfg[name], max(args.steps, 20), args.warmup, hip)
            extra[name] = keep(cfg[name], r)
            del st
            torch.cuda.empty_cache()
        extra["decode_b64_l64k"] = decode_bench(cfg["decode_b64_l64k"], 20, 3)
        torch.cuda.empty_cache()
        extra["training_step"] = {name: train_bench(cfg[name]) for name in ("gpt2s_n2k",
                                                                             "gqa7b_n32k")}
        torch.cuda.empty_cache()
    line = {
        "metric": METRIC, "value": res3["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res3["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded Gaussian-mixture fp32 hidden states, N(0,1) bf16 Q/K/V",
        "config": {"workload": c3.name, "n": c3.n, "d_model": c3.d, "q_heads": c3.Hq,
                   "kv_heads": c3.Hkv, "d_head": c3.dh, "d_g": c3.dg, "K": c3.K,
                   "top_k": c3.top_k, "window": c3.window, "sinkhorn_iters": c3.iters,
                   "global_batch": 1, "seq_len": c3.n, "parallelism": "single GPU"},
        "roofline": res3.pop("roofline"),
        "attention_tflops": res3["attention_tflops"],
        "attention_pct_bf16_peak": res3["attention_pct_bf16_peak"],
        "detail_128k": res3,
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(c3, cap3, prefill)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
