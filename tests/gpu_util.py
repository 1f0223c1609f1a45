"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and comparing
HIP-path outputs with the oracle. Holds no arithmetic of the method."""
import sys

import numpy as np
import torch

TOL_MAX_ABS = 2e-2   # attention output, bf16 inputs against the fp64 oracle
TOL_MEAN_ABS = 2e-3
TOL_LSE = 1e-4       # the log-sum-exp is accumulated in fp32 from exact bf16 products; one
                     # double-counted or missing pair in a row of m keys moves it by about 1/m


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def bf16_dev(bits):
    """numpy uint16 bf16 bit patterns -> torch bfloat16 on the device."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bucket_expected(groups, K):
    """offsets / idx / slot of a stable sort of the memberships by group (numpy's stable sort)."""
    g = np.asarray(groups, np.int64)
    n, k = g.shape
    flat = g.ravel()
    valid = (flat >= 0) & (flat < K)
    tok = np.repeat(np.arange(n), k)
    order = np.argsort(np.where(valid, flat, K), kind="stable")[: valid.sum()]
    counts = np.bincount(flat[valid], minlength=K)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    idx = np.full(n * k, -1, np.int32)
    idx[: len(order)] = tok[order]
    slot = np.full(n * k, -1, np.int32)
    slot[order] = np.arange(len(order))
    return offsets, idx, slot.reshape(n, k)


def check_attention(out_gpu, lse_gpu, out_ref, lse_ref, what=""):
    o = to_np(out_gpu)
    l = to_np(lse_gpu)
    err = np.abs(o - out_ref)
    lerr = np.abs(l - lse_ref)
    msg = (f"{what}: max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} max|dLSE|={lerr.max():.3e}")
    say(msg)
    assert np.isfinite(o).all() and np.isfinite(l).all(), msg
    assert err.max() <= TOL_MAX_ABS, msg
    assert err.mean() <= TOL_MEAN_ABS, msg
    assert lerr.max() <= TOL_LSE, msg
