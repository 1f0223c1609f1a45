"""Seeded generators for the Focus workloads.

Every array here is random data with a stated distribution; nothing computes any step of
the method. Host arrays come from numpy's PCG64 streams derived from
SeedSequence(20261202 + workload index); device arrays (for sizes where drawing on the
host would take minutes) come from torch's CUDA Philox generator seeded the same way.
Either way both the oracle and the HIP path receive the very same values: device-drawn
inputs are copied to the host before the oracle sees them.

Distributions:
  hidden   h_i = mu_{c_i} + sigma * eps_i, mu unit-norm random directions in R^d,
           c_i drawn i.i.d. from the mixture weights (uniform, or c**-1.1 for c = 1..M);
           a noise token (probability noise_frac, i.i.d.) is sigma * eps_i with no mean.
  W_g      N(0, 1/d) entries, shape [d, d_g].
  C        random unit rows, shape [K, d_g].
  Q, K, V  N(0, 1) drawn in fp32, rounded to bf16 (round to nearest even).
"""
import numpy as np

BASE_SEED = 20261202
STREAMS = ("means", "comps", "noise", "w_g", "centroids", "q", "k", "v")


def seed_streams(index, salt=0):
    """Eight independent PCG64 streams for workload `index` (optionally salted)."""
    ss = np.random.SeedSequence([BASE_SEED + index, salt])
    return dict(zip(STREAMS, (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(8))))


def _stream_seed(index, salt, name):
    """A 63-bit integer seed for torch generators, derived from the same SeedSequence."""
    ss = np.random.SeedSequence([BASE_SEED + index, salt, STREAMS.index(name)])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


# ---------------------------------------------------------------- bf16 helpers (bit-level)
def f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Finite inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ---------------------------------------------------------------- mixture weights
def mixture_weights(mix, weights):
    if weights == "uniform":
        w = np.ones(mix)
    elif weights == "zipf":
        w = np.arange(1, mix + 1, dtype=np.float64) ** -1.1
    else:
        raise ValueError(weights)
    return w / w.sum()


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=1, keepdims=True)


# ---------------------------------------------------------------- assignment inputs
def assign_inputs(n, d, dg, K, mix, weights="uniform", noise_frac=0.0, sigma=0.5,
                  index=0, salt=0, device="cpu"):
    """Hidden states [n, d], W_g [d, dg] and centroids [K, dg], all fp32.

    device="cpu" returns numpy arrays. device="cuda" returns torch tensors on cuda:0 whose
    bulk noise is drawn there; the small parameters are still drawn on the host.
    """
    rs = seed_streams(index, salt)
    means = _unit_rows(rs["means"].standard_normal((mix, d))).astype(np.float32)
    comps = rs["comps"].choice(mix, size=n, p=mixture_weights(mix, weights))
    is_noise = rs["comps"].random(n) < noise_frac if noise_frac > 0 else np.zeros(n, bool)
    w_g = (rs["w_g"].standard_normal((d, dg)) / np.sqrt(d)).astype(np.float32)
    cents = _unit_rows(rs["centroids"].standard_normal((K, dg))).astype(np.float32)
    if device == "cpu":
        hidden = rs["noise"].standard_normal((n, d), dtype=np.float32)
        hidden *= np.float32(sigma)
        keep = ~is_noise
        hidden[keep] += means[comps[keep]]
        return dict(hidden=hidden, w_g=w_g, centroids=cents, comps=comps, is_noise=is_noise)
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(_stream_seed(index, salt, "noise"))
    hidden = torch.empty((n, d), dtype=torch.float32, device="cuda")
    rows = max(1, (1 << 28) // d)  # draw in slabs to bound temporaries
    means_t = torch.from_numpy(means).cuda()
    comps_t = torch.from_numpy(comps.astype(np.int64)).cuda()
    keep_t = torch.from_numpy((~is_noise).astype(np.float32)).cuda()
    for r0 in range(0, n, rows):
        r1 = min(n, r0 + rows)
        slab = torch.randn((r1 - r0, d), dtype=torch.float32, device="cuda", generator=g)
        slab.mul_(sigma)
        slab.add_(means_t[comps_t[r0:r1]] * keep_t[r0:r1, None])
        hidden[r0:r1] = slab
    return dict(hidden=hidden, w_g=torch.from_numpy(w_g).cuda(),
                centroids=torch.from_numpy(cents).cuda(), comps=comps, is_noise=is_noise)


# ---------------------------------------------------------------- attention inputs
def qkv_inputs(n, Hq, Hkv, dh, index=0, salt=0, device="cpu", lead=(), which="qkv"):
    """Q [*lead, n, Hq, dh], K and V [*lead, n, Hkv, dh], N(0,1) rounded to bf16.

    device="cpu": numpy uint16 bf16 bit patterns. device="cuda": torch bfloat16 on cuda:0.
    `which` selects the tensors to draw (each has its own stream, so a subset draws the same
    values as the full set).
    """
    lead = tuple(lead)
    shapes = {"q": lead + (n, Hq, dh), "k": lead + (n, Hkv, dh), "v": lead + (n, Hkv, dh)}
    shapes = {x: shp for x, shp in shapes.items() if x in which}
    if device == "cpu":
        rs = seed_streams(index, salt)
        return {name: f32_to_bf16_bits(rs[name].standard_normal(shp, dtype=np.float32))
                for name, shp in shapes.items()}
    import torch
    out = {}
    for name, shp in shapes.items():
        g = torch.Generator(device="cuda")
        g.manual_seed(_stream_seed(index, salt, name))
        t = torch.empty(shp, dtype=torch.bfloat16, device="cuda")
        flat = t.view(-1, shp[-2] * shp[-1])
        rows = max(1, (1 << 28) // flat.shape[1])  # fp32 temporaries of at most 1 GiB
        for r0 in range(0, flat.shape[0], rows):
            r1 = min(flat.shape[0], r0 + rows)
            flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), dtype=torch.float32, device="cuda",
                                      generator=g).to(torch.bfloat16)
        out[name] = t
    return out


def random_groups(n, K, top_k, rng, skew=0.0):
    """Random memberships: top_k distinct groups per token, listed in ascending order.

    With skew > 0 group c is drawn with weight (c+1)**-skew, giving unequal segment sizes.
    """
    w = np.arange(1, K + 1, dtype=np.float64) ** -skew
    w /= w.sum()
    out = np.empty((n, top_k), np.int32)
    if top_k == 1:
        out[:, 0] = rng.choice(K, size=n, p=w)
        return out
    # weighted sampling without replacement: the top_k of log(w) + Gumbel noise per token
    logw = np.log(w)[None, :]
    for r0 in range(0, n, 65536):
        r1 = min(n, r0 + 65536)
        keys = logw + rng.gumbel(size=(r1 - r0, K))
        out[r0:r1] = np.sort(np.argpartition(-keys, top_k - 1, axis=1)[:, :top_k], axis=1)
    return out
