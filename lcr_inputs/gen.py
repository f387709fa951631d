"""Seeded draws for every workload.

Draws are made in float32 with numpy's default_rng seeded by
[config id, tag, layer, step] and, for bf16 workloads, rounded to bfloat16
(round to nearest even). bf16 arrays are carried as uint16 bit patterns so the
oracle and the GPU consume identical bits. The 64K stack is too large for host
generation and uses a torch generator on the device instead.
"""
import numpy as np

from .configs import Config, SLOTS, CONTENT

TAG_Q, TAG_K, TAG_V, TAG_X, TAG_A, TAG_B, TAG_NEEDLE, TAG_OFFSET = 1, 2, 3, 4, 5, 6, 7, 8
TAG_DO, TAG_SCORE, TAG_ZSEL, TAG_DS, TAG_DH = 9, 10, 11, 12, 13


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern (uint16) -> float64, exact."""
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact upcast of a stored input (uint16 = bf16 bits, or float32/float64)."""
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def _rng(cfg: Config, tag: int, layer: int = 0, step: int = 0):
    return np.random.default_rng([cfg.cid, tag, layer, step])


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def route_inputs(cfg: Config, layer: int = 0, step: int = 0) -> dict:
    """Full route-layer inputs: q [B,Hq,L,d], k,v [B,Hkv,L,d], x [B,L,D], A [D,r], Bm [r,Hq*d].

    The entropy workload adds to every key a per-(batch, KV head, chunk) offset
    vector shared by all 64 slots of the chunk.
    """
    B, Hq, Hkv, L, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d
    out = {}
    out["q"] = _store(_normal(_rng(cfg, TAG_Q, layer, step), (B, Hq, L, d)), cfg.dtype)
    k = _normal(_rng(cfg, TAG_K, layer, step), (B, Hkv, L, d))
    if cfg.key_offset_std > 0:
        off = _normal(_rng(cfg, TAG_OFFSET, layer, step), (B, Hkv, cfg.N, 1, d), cfg.key_offset_std)
        k = (k.reshape(B, Hkv, cfg.N, SLOTS, d) + off).reshape(B, Hkv, L, d)
    out["k"] = _store(k, cfg.dtype)
    del k
    out["v"] = _store(_normal(_rng(cfg, TAG_V, layer, step), (B, Hkv, L, d)), cfg.dtype)
    out["x"] = _store(_normal(_rng(cfg, TAG_X, layer, step), (B, L, cfg.D)), cfg.dtype)
    out["A"] = _store(_normal(_rng(cfg, TAG_A, layer, 0), (cfg.D, cfg.r), cfg.ab_std), cfg.dtype)
    out["Bm"] = _store(_normal(_rng(cfg, TAG_B, layer, 0), (cfg.r, Hq * d), cfg.ab_std), cfg.dtype)
    return out


def _remote_prefix_chunks(cfg: Config) -> int:
    """Chunks lying wholly left of the earliest tail query's window."""
    first = cfg.T - cfg.n_tail
    n = 0
    while CONTENT * n + CONTENT - 1 < first - cfg.R:
        n += 1
    return n


def decode_cache(cfg: Config) -> dict:
    """Cached K/V for the decode workload, the mask-slot queries and the planted needles.

    For every KV group g a random unit direction u_g is drawn and `needles`
    distinct chunks (among those remote for every tail query) get
    needle_shift * sqrt(d) * u_g added to their 63 content keys.
    Returns k, v [1,Hkv,L,d]; q_mask [1,Hq,N,d] (the queries at slots 64c+63);
    needles [Hkv, n]; u [Hkv, d].
    """
    B, Hq, Hkv, L, d, N = cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, cfg.N
    k = _normal(_rng(cfg, TAG_K), (B, Hkv, L, d))
    rng = _rng(cfg, TAG_NEEDLE)
    n_remote = _remote_prefix_chunks(cfg)
    needles = np.zeros((Hkv, cfg.needles), dtype=np.int64)
    u = np.zeros((Hkv, d), dtype=np.float64)
    for g in range(Hkv):
        ug = rng.standard_normal(d)
        ug /= np.linalg.norm(ug)
        u[g] = ug
        needles[g] = np.sort(rng.choice(n_remote, size=cfg.needles, replace=False))
        shift = (cfg.needle_shift * np.sqrt(d) * ug).astype(np.float32)
        for c in needles[g]:
            k[:, g, SLOTS * c: SLOTS * c + CONTENT, :] += shift
    out = {"k": _store(k, cfg.dtype)}
    del k
    out["v"] = _store(_normal(_rng(cfg, TAG_V), (B, Hkv, L, d)), cfg.dtype)
    out["q_mask"] = _store(_normal(_rng(cfg, TAG_Q), (B, Hq, N, d)), cfg.dtype)
    out["A"] = _store(_normal(_rng(cfg, TAG_A), (cfg.D, cfg.r), cfg.ab_std), cfg.dtype)
    out["Bm"] = _store(_normal(_rng(cfg, TAG_B), (cfg.r, Hq * d), cfg.ab_std), cfg.dtype)
    out["needles"] = needles
    out["u"] = u
    out["n_remote"] = n_remote
    return out


def decode_step(cfg: Config, step: int) -> dict:
    """Fresh decode-block inputs: q_tail [1,Hq,n_tail,d] and x_tail [1,n_tail,D] for
    content positions T-n_tail .. T-1 (in order)."""
    B, Hq, d, n = cfg.B, cfg.Hq, cfg.d, cfg.n_tail
    return {
        "q_tail": _store(_normal(_rng(cfg, TAG_Q, 0, step + 1), (B, Hq, n, d)), cfg.dtype),
        "x_tail": _store(_normal(_rng(cfg, TAG_X, 0, step + 1), (B, n, cfg.D)), cfg.dtype),
    }


def stack_layer_torch(cfg: Config, layer: int, device, route: bool):
    """Per-layer inputs of the 64K stack drawn on the device (bf16 ~ N(0,1)).

    Seeds: torch generator seeded with a fixed function of (config id, tag, layer).
    Returns dict of torch tensors q, k, v (and x, A, Bm for route layers).
    """
    import torch

    def draw(tag, shape, std=1.0):
        g = torch.Generator(device=device)
        g.manual_seed(((cfg.cid * 1000003 + tag) * 1000003 + layer) & 0x7FFFFFFFFFFFFFFF)
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(torch.bfloat16)

    B, Hq, Hkv, L, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d
    out = {"q": draw(TAG_Q, (B, Hq, L, d)), "k": draw(TAG_K, (B, Hkv, L, d)),
           "v": draw(TAG_V, (B, Hkv, L, d))}
    if route:
        out["x"] = draw(TAG_X, (B, L, cfg.D))
        out["A"] = draw(TAG_A, (cfg.D, cfg.r), cfg.ab_std)
        out["Bm"] = draw(TAG_B, (cfg.r, Hq * d), cfg.ab_std)
    return out


def backward_draws(cfg: Config, q0: int, nq: int, layer: int = 0) -> dict:
    """Draws for the gradient workloads of queries q0 .. q0+nq-1:
    dO [B,Hq,L,d] (upstream gradient on the route-layer output, stored like q);
    score [B,Hkv,nq,N] float32 (random chunk scores: ranking them over the
    remote chunks gives a synthetic selection); zsel [B,Hq,nq,K] float32
    (chunk logits for the selected entries); ds [B,Hq,N,d] and dH [B,Hq,N]
    float32 (upstream gradients on the summaries and entropies)."""
    B, Hq, Hkv, L, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d
    out = {}
    out["dO"] = _store(_normal(_rng(cfg, TAG_DO, layer), (B, Hq, L, d)), cfg.dtype)
    out["score"] = _normal(_rng(cfg, TAG_SCORE, layer), (B, Hkv, nq, cfg.N))
    out["zsel"] = _normal(_rng(cfg, TAG_ZSEL, layer), (B, Hq, nq, cfg.K))
    out["ds"] = _normal(_rng(cfg, TAG_DS, layer), (B, Hq, cfg.N, d))
    out["dH"] = _normal(_rng(cfg, TAG_DH, layer), (B, Hq, cfg.N))
    return out


def sample_query_blocks(T: int, n_blocks: int = 16, block: int = 64, seed: int = 0) -> np.ndarray:
    """Content positions of `n_blocks` blocks of `block` consecutive queries at
    seeded offsets, always including the first and the last block."""
    rng = np.random.default_rng([seed, 99])
    n_all = (T + block - 1) // block
    if n_all <= n_blocks:
        return np.arange(T)
    mid = rng.choice(np.arange(1, n_all - 1), size=n_blocks - 2, replace=False)
    starts = np.concatenate([[0], np.sort(mid) * block, [T - block]])
    idx = np.unique(np.concatenate([np.arange(s, min(s + block, T)) for s in starts]))
    return idx
