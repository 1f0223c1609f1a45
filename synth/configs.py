"""The five workloads of the Focus inference path, as plain data.

Shapes follow the workloads quoted for the method: a GPT-2-small-shaped MHA layer, a
7B-shaped and a 70B-shaped GQA layer, a 1M-token prefill and a batched decode against
65536-token caches. Fields a workload does not state are filled with the values of the
7B-shaped layer (decode: model width 4096, group dimension 128, three Sinkhorn iterations,
a uniform 64-component mixture).
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    index: int            # position in the workload list; seeds derive from it
    n: int                # tokens per sequence (decode: cache length L)
    d: int                # model width of the hidden states
    Hq: int
    Hkv: int
    dh: int
    dg: int               # group-space dimension
    K: int                # number of centroids
    top_k: int
    window: int
    iters: int            # Sinkhorn iterations
    mix: int              # Gaussian-mixture components of the hidden states
    weights: str          # "uniform" or "zipf" (weight of component c is c**-1.1)
    noise_frac: float = 0.0   # share of tokens drawn as isotropic noise with no mean
    sigma: float = 0.5        # per-dimension standard deviation around a mean
    batch: int = 1            # decode batch (one fresh query per sequence)
    decode: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def G(self):
        return self.Hq // self.Hkv


CONFIGS = [
    Config("gpt2s_n2k", 0, n=2048, d=768, Hq=12, Hkv=12, dh=64, dg=64, K=16, top_k=1,
           window=128, iters=3, mix=16, weights="uniform"),
    Config("gqa7b_n32k", 1, n=32768, d=4096, Hq=32, Hkv=8, dh=128, dg=128, K=64, top_k=2,
           window=512, iters=3, mix=64, weights="zipf"),
    Config("gqa70b_n128k", 2, n=131072, d=8192, Hq=64, Hkv=8, dh=128, dg=128, K=128, top_k=2,
           window=1024, iters=3, mix=128, weights="zipf"),
    Config("long_n1m", 3, n=1048576, d=4096, Hq=32, Hkv=8, dh=128, dg=128, K=256, top_k=1,
           window=512, iters=2, mix=256, weights="uniform", noise_frac=0.1),
    Config("decode_b64_l64k", 4, n=65536, d=4096, Hq=32, Hkv=8, dh=128, dg=128, K=64, top_k=2,
           window=256, iters=3, mix=64, weights="uniform", batch=64, decode=True),
]


def config_by_name(name):
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
