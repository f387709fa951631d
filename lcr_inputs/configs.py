"""Workload shapes.

Sizes follow the route-layer description of "Prefilling-dLLM v2: Learned Chunk
Routing for Long-Context Diffusion Language Models" (Figure 3 caption; Table 3,
layer configurations: local radius 256, 32 remote chunks of 64, SWA radius 1280
on the other layers) and the 7B backbone shape (28 query heads, 4 KV heads,
head dim 128, hidden 3584). The tiny case is a reduced version for exhaustive
checks. Each config has an integer id that seeds its random draws.
"""
from dataclasses import dataclass, field
import math

SLOTS = 64      # slots per chunk
CONTENT = 63    # content tokens per chunk (the 64th slot is the routing mask)


@dataclass(frozen=True)
class Config:
    name: str
    cid: int                 # seed id
    kind: str                # "prefill" | "decode" | "stack"
    B: int
    N: int                   # chunks
    Hq: int
    Hkv: int
    d: int
    r: int                   # residual rank
    D: int                   # hidden size feeding the residual
    K: int                   # remote chunks kept per (KV group, query)
    R: int                   # local window radius (content index space)
    beta: float              # entropy weight
    dtype: str               # "bf16" | "fp32"
    ab_std: float = 0.02     # std of the residual factors A and B
    key_offset_std: float = 0.0   # per-chunk shared key offset (entropy workload)
    n_tail: int = 0          # decode: fresh queries at the tail
    steps: int = 1           # decode: steps timed
    needles: int = 0         # decode: planted chunks per KV group
    needle_shift: float = 0.5     # decode: shift in units of sqrt(d) along u_g
    layers: int = 1          # stack: layers
    route_every: int = 4     # stack: route layer when l % route_every == route_every - 1
    swa_radius: int = 0      # stack: SWA radius in slot space
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def L(self) -> int:
        return self.N * SLOTS

    @property
    def T(self) -> int:
        return self.N * CONTENT

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def q0(self) -> int:
        return self.T - self.n_tail if self.kind == "decode" else 0

    @property
    def nq(self) -> int:
        return self.n_tail if self.kind == "decode" else self.T


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny_fp32", 1, "prefill", B=1, N=16, Hq=2, Hkv=1, d=64, r=8, D=128,
               K=4, R=64, beta=0.0, dtype="fp32"),
        Config("prefill_16k", 2, "prefill", B=1, N=256, Hq=28, Hkv=4, d=128, r=64, D=3584,
               K=32, R=256, beta=0.0, dtype="bf16"),
        Config("decode_128k", 3, "decode", B=1, N=2048, Hq=28, Hkv=4, d=128, r=64, D=3584,
               K=32, R=256, beta=0.0, dtype="bf16", n_tail=32, steps=64, needles=8),
        Config("prefill_32k_entropy", 4, "prefill", B=2, N=512, Hq=28, Hkv=4, d=128, r=64,
               D=3584, K=32, R=256, beta=0.5, dtype="bf16", key_offset_std=0.3),
        Config("stack_64k", 5, "stack", B=1, N=1024, Hq=28, Hkv=4, d=128, r=64, D=3584,
               K=32, R=256, beta=0.0, dtype="bf16", layers=28, swa_radius=1280),
    ]
}


def get_config(name: str, **overrides) -> Config:
    base = CONFIGS[name]
    if not overrides:
        return base
    kw = {f: getattr(base, f) for f in base.__dataclass_fields__}
    kw.update(overrides)
    return Config(**kw)
