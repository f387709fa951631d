"""HIP path against the fp64 oracle, through the C ABI (needs an MI355X).

Sizes: the tiny float32 layer in full; the 16K prefill layer at full size in the
launch configuration the benchmark times, checked on sampled query blocks; the
128K decode step in full (32 queries); the 32K entropy layer (batch 2) on
sampled blocks; ragged and degenerate cases (window only, no remote chunk,
fewer candidates than K, single and eight-head groups, partial query ranges).
"""
import numpy as np
import pytest
import torch

import learned_chunk_routed_amd as lcr
from lcr_inputs import as_f64, get_config, route_inputs, decode_cache, decode_step, sample_query_blocks
from oracle import route as O
from gpu_util import (to_dev, f64, check_selection, max_err, OUT_TOL, LSE_TOL, Z_TOL)

pytestmark = pytest.mark.gpu


def _f(inp):
    return {k: as_f64(v) for k, v in inp.items() if isinstance(v, np.ndarray) and v.dtype != np.int64}


def route_parity(cfg, queries=None, q0=0, nq=None, label=""):
    """Run the full route layer on the GPU and compare with the oracle on `queries`."""
    print(f"[case] {label or cfg.name}: B={cfg.B} N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} K={cfg.K} "
          f"R={cfg.R} beta={cfg.beta} dtype={cfg.dtype} q0={q0} nq={nq}", flush=True)
    inp = route_inputs(cfg)
    dev = {k: to_dev(v) for k, v in inp.items()}
    nq = cfg.T - q0 if nq is None else nq
    res = lcr.route_layer(dev["q"], dev["k"], dev["v"], dev["x"], dev["A"], dev["Bm"], K=cfg.K, radius=cfg.R,
                          beta=cfg.beta, scale=cfg.scale, q0=q0, nq=nq, want_lse=True)
    torch.cuda.synchronize()
    f = _f(inp)
    if queries is None:
        queries = np.arange(q0, q0 + nq)
    queries = np.asarray(queries)
    t = queries - q0
    ref = O.route_layer(f["q"], f["k"], f["v"], f["x"], f["A"], f["Bm"], K=cfg.K, R=cfg.R, beta=cfg.beta,
                        scale=cfg.scale, queries=queries)
    tol_o, tol_l, tol_z = OUT_TOL[cfg.dtype], LSE_TOL[cfg.dtype], Z_TOL[cfg.dtype]

    s_err = max_err(f64(res["s"]), ref["s"]) / max(1.0, np.abs(ref["s"]).max())
    H_err = max_err(f64(res["H"]), ref["H"])
    assert s_err < 1e-5 and H_err < 1e-5, f"summaries: s {s_err:.2e}, H {H_err:.2e}"

    idx_gpu = res["idx"].cpu().numpy()[:, :, t].astype(np.int64)
    same = check_selection(idx_gpu, ref, cfg.K, label or cfg.name)
    zref = O.gather_zsel(ref["z"], idx_gpu, cfg.G)
    zsel_gpu = f64(res["zsel"])[:, :, t]
    fin = np.isfinite(zref)
    assert np.array_equal(fin, np.isfinite(zsel_gpu)), "zsel padding"
    z_err = max_err(zsel_gpu[fin], zref[fin])
    assert z_err < tol_z * max(1.0, np.abs(zref[fin]).max() if fin.any() else 1.0), f"zsel error {z_err:.2e}"

    o_ref, lse_ref = ref["o"].copy(), ref["lse"].copy()
    diff_t = np.nonzero(~same.all(axis=(0, 1)))[0]
    if len(diff_t):
        qr = f["q"][:, :, O.slot_of(queries[diff_t])]
        o2, l2 = O.routed_attention(qr, f["k"], f["v"], idx_gpu[:, :, diff_t], zref[:, :, diff_t], cfg.R,
                                    cfg.scale, queries[diff_t])
        o_ref[:, :, diff_t], lse_ref[:, :, diff_t] = o2, l2
    o_gpu = f64(res["o"])[:, :, O.slot_of(queries)]
    o_err = max_err(o_gpu, o_ref)
    l_err = max_err(f64(res["lse"])[:, :, t], lse_ref)
    print(f"    rows={len(queries)} gated={int((ref['margin'] > 1e-3).sum())} "
          f"idx_same={int(same.sum())}/{same.size} o_err={o_err:.2e} lse_err={l_err:.2e} z_err={z_err:.2e}",
          flush=True)
    assert o_err < tol_o, f"output error {o_err:.3e} > {tol_o}"
    assert l_err < tol_l, f"lse error {l_err:.3e} > {tol_l}"
    return res


# ----------------------------------------------------------------------------- summaries

@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_16k"])
def test_chunk_summary(name):
    cfg = get_config(name)
    print(f"[case] chunk_summary {name}", flush=True)
    inp = route_inputs(cfg)
    s, H = lcr.chunk_summary(to_dev(inp["q"]), to_dev(inp["k"]), cfg.scale)
    torch.cuda.synchronize()
    rs, rH = O.chunk_summary(as_f64(inp["q"]), as_f64(inp["k"]), cfg.scale)
    assert max_err(f64(s), rs) < 1e-5 * max(1.0, np.abs(rs).max())
    assert max_err(f64(H), rH) < 1e-5


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_16k"])
def test_chunk_summary_mean(name):
    """Mean summaries against the oracle, and bit for bit equal to mask-query pooling
    with zero mask queries (the kernel's own special case)."""
    cfg = get_config(name)
    print(f"[case] chunk_summary_mean {name}", flush=True)
    inp = route_inputs(cfg)
    k = to_dev(inp["k"])
    s, H = lcr.chunk_summary_mean(k, cfg.Hq)
    q0 = torch.zeros(inp["q"].shape, dtype=k.dtype, device="cuda")
    s0, H0 = lcr.chunk_summary(q0, k, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(s, s0) and torch.equal(H, H0)
    rs, rH = O.chunk_summary_mean(as_f64(inp["k"]), cfg.Hq)
    assert max_err(f64(s), rs) < 1e-5 * max(1.0, np.abs(rs).max())
    assert max_err(f64(H), rH) < 1e-5


def test_chunk_summary_refresh_after_keys_change():
    """A decode step rewrites the keys of the block being decoded: refreshing only that
    chunk's summaries must give what a whole recompute gives (bit for bit), and the
    other rows must stay untouched."""
    from lcr_inputs import bf16_round
    cfg = get_config("tiny_fp32", N=32, Hq=8, Hkv=2, d=128, dtype="bf16")
    print("[case] chunk_summary refresh of one chunk", flush=True)
    inp = route_inputs(cfg)
    q = to_dev(inp["q"])
    s, H = lcr.chunk_summary(q, to_dev(inp["k"]), cfg.scale)
    s_old, H_old = s.clone(), H.clone()
    c = cfg.N - 2                                   # an interior chunk's keys change
    k2 = inp["k"].copy()
    rng = np.random.default_rng(99)
    k2[:, :, 64 * c:64 * c + 63] = bf16_round(rng.standard_normal(k2[:, :, 64 * c:64 * c + 63].shape,
                                                                  dtype=np.float32))
    k = to_dev(k2)
    lcr.chunk_summary(q, k, cfg.scale, s=s, H=H, chunks=(c, 1))
    s_full, H_full = lcr.chunk_summary(q, k, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(s, s_full) and torch.equal(H, H_full)
    keep = [i for i in range(cfg.N) if i != c]
    assert torch.equal(s[:, :, keep], s_old[:, :, keep]) and torch.equal(H[:, :, keep], H_old[:, :, keep])
    assert not torch.equal(s[:, :, c], s_old[:, :, c])
    rs, rH = O.chunk_summary(as_f64(inp["q"]), as_f64(k2), cfg.scale)
    assert max_err(f64(s)[:, :, c], rs[:, :, c]) < 1e-5 * max(1.0, np.abs(rs).max())
    assert max_err(f64(H)[:, :, c], rH[:, :, c]) < 1e-5


# ----------------------------------------------------------------------------- full layers

def test_route_layer_tiny_fp32_full():
    route_parity(get_config("tiny_fp32"))


def test_route_layer_prefill_16k_sampled():
    cfg = get_config("prefill_16k")
    route_parity(cfg, queries=sample_query_blocks(cfg.T, n_blocks=6, block=64, seed=2))


def test_route_layer_entropy_32k_sampled():
    cfg = get_config("prefill_32k_entropy")
    route_parity(cfg, queries=sample_query_blocks(cfg.T, n_blocks=4, block=64, seed=4))


def test_decode_128k_step():
    cfg = get_config("decode_128k")
    print("[case] decode_128k step 0", flush=True)
    cache = decode_cache(cfg)
    st = decode_step(cfg, 0)
    B, Hq, L, d, N = cfg.B, cfg.Hq, cfg.L, cfg.d, cfg.N
    q = torch.zeros((B, Hq, L, d), dtype=torch.bfloat16, device="cuda")
    qv = q.view(B, Hq, N, 64, d)
    qv[:, :, :, 63] = to_dev(cache["q_mask"])
    slots = O.slot_of(np.arange(cfg.q0, cfg.T))
    q[:, :, torch.from_numpy(slots).cuda()] = to_dev(st["q_tail"])
    x = torch.zeros((B, L, cfg.D), dtype=torch.bfloat16, device="cuda")
    x[:, torch.from_numpy(slots).cuda()] = to_dev(st["x_tail"])
    k, v = to_dev(cache["k"]), to_dev(cache["v"])
    res = lcr.route_layer(q, k, v, x, to_dev(cache["A"]), to_dev(cache["Bm"]), K=cfg.K, radius=cfg.R,
                          beta=cfg.beta, scale=cfg.scale, q0=cfg.q0, nq=cfg.nq, want_lse=True)
    torch.cuda.synchronize()
    kf, vf = as_f64(cache["k"]), as_f64(cache["v"])
    queries = np.arange(cfg.q0, cfg.T)
    ref = O.route_layer_rows(as_f64(st["q_tail"]), as_f64(cache["q_mask"]), kf, vf, as_f64(st["x_tail"]),
                             as_f64(cache["A"]), as_f64(cache["Bm"]), K=cfg.K, R=cfg.R, beta=cfg.beta,
                             scale=cfg.scale, queries=queries)
    idx_gpu = res["idx"].cpu().numpy().astype(np.int64)
    same = check_selection(idx_gpu, ref, cfg.K, "decode_128k")
    zref = O.gather_zsel(ref["z"], idx_gpu, cfg.G)
    o_ref, l_ref = O.routed_attention(as_f64(st["q_tail"]), kf, vf, idx_gpu, zref, cfg.R, cfg.scale, queries)
    o_err = max_err(f64(res["o"])[:, :, slots], o_ref)
    l_err = max_err(f64(res["lse"]), l_ref)
    hits = np.mean([np.isin(cache["needles"][g], idx_gpu[0, g]).mean() for g in range(cfg.Hkv)])
    print(f"    idx_same={int(same.sum())}/{same.size} gated={int((ref['margin'] > 1e-3).sum())} "
          f"needle_hit_rate={hits:.2f} o_err={o_err:.2e} lse_err={l_err:.2e}", flush=True)
    assert o_err < OUT_TOL["bf16"] and l_err < LSE_TOL["bf16"]


# ----------------------------------------------------------------------------- edge cases

EDGE = [
    ("window only (K=0)", dict(K=0)),
    ("window covers everything", dict(R=4000)),
    ("fewer candidates than K", dict(N=6, K=8, R=100)),
    ("ragged query range", dict(), 137, 201),
    ("single-head groups", dict(Hq=3, Hkv=3)),
    ("eight-head groups", dict(Hq=16, Hkv=2)),
    ("radius zero", dict(R=0)),
    ("large K", dict(N=40, K=64, R=30)),
    ("entropy weight", dict(beta=0.8)),
    ("32 queries, rank 64", dict(r=64, D=256), 700, 32),
    ("5 queries at the end, ragged hidden", dict(), 1507, 5),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_route_layer_edge(case, dtype):
    name, over = case[0], case[1]
    q0, nq = (case[2], case[3]) if len(case) > 2 else (0, None)
    base = dict(N=24, Hq=4, Hkv=2, d=64 if dtype == "fp32" else 128, r=16, D=96, K=4, R=64, beta=0.0,
                dtype=dtype)
    base.update(over)
    cfg = get_config("tiny_fp32", **base)
    route_parity(cfg, q0=q0, nq=nq, label=f"{name} [{dtype}]")


# Prefill-sized edge cases (enough query blocks for the prefill kernel), checked on
# sampled query blocks: first, last and a middle block of the queried range.
PREFILL_EDGE = [
    ("window only (K=0)", dict(K=0)),
    ("ragged query range", dict(), 1000, 5001),
    ("eight-head groups", dict(Hq=16, Hkv=2)),
    ("single-head groups", dict(Hq=4, Hkv=4)),
    ("head dim 64", dict(d=64)),
    ("K=64", dict(K=64, R=30)),
    ("radius zero", dict(R=0)),
    ("wide window", dict(R=3000)),
    # past 512 chunks the fused scoring takes 32-query blocks with 16 keys per lane
    ("700 chunks, entropy term", dict(N=700, K=32, beta=0.5)),
    ("1024 chunks, head dim 64", dict(N=1024, d=64, K=32)),
]


@pytest.mark.parametrize("beta", [-0.5, 0.25, 1.0, 2.0])
def test_route_layer_beta_sweep(beta):
    """Entropy weights around and beyond the published one, on keys with per-chunk
    offsets so that the pooling entropies spread; a negative weight prefers the
    chunks whose summaries are least peaked."""
    cfg = get_config("tiny_fp32", N=128, Hq=8, Hkv=2, d=128, r=16, D=96, K=8, R=128, beta=beta, dtype="bf16",
                     key_offset_std=0.3)
    queries = np.unique(np.concatenate([np.arange(64), np.arange(4000, 4064), np.arange(cfg.T - 64, cfg.T)]))
    route_parity(cfg, queries=queries, label=f"beta {beta}")


@pytest.mark.parametrize("case", PREFILL_EDGE, ids=[c[0] for c in PREFILL_EDGE])
def test_route_layer_prefill_edge(case):
    name, over = case[0], case[1]
    q0, nq = (case[2], case[3]) if len(case) > 2 else (0, None)
    base = dict(N=128, Hq=8, Hkv=2, d=128, r=16, D=96, K=8, R=128, beta=0.0, dtype="bf16")
    base.update(over)
    cfg = get_config("tiny_fp32", **base)
    nq_eff = cfg.T - q0 if nq is None else nq
    lo, hi = q0, q0 + nq_eff
    mid = lo + (nq_eff // 2) // 64 * 64
    queries = np.unique(np.concatenate([np.arange(lo, lo + 64), np.arange(mid, mid + 64), np.arange(hi - 64, hi)]))
    route_parity(cfg, queries=queries, q0=q0, nq=nq, label=f"prefill {name}")


def test_determinism_and_decode_split_matches_prefill():
    """Two runs are bitwise identical; the split (decode) plan equals the unsplit plan."""
    cfg = get_config("tiny_fp32", N=64, Hq=8, Hkv=2, d=128, r=32, D=256, K=8, R=128, dtype="bf16")
    print("[case] determinism", flush=True)
    inp = route_inputs(cfg)
    dev = {k: to_dev(v) for k, v in inp.items()}
    a = lcr.route_layer(dev["q"], dev["k"], dev["v"], dev["x"], dev["A"], dev["Bm"], K=cfg.K, radius=cfg.R,
                        scale=cfg.scale)
    b = lcr.route_layer(dev["q"], dev["k"], dev["v"], dev["x"], dev["A"], dev["Bm"], K=cfg.K, radius=cfg.R,
                        scale=cfg.scale)
    torch.cuda.synchronize()
    for key in ["s", "H", "idx", "zsel", "o"]:
        assert torch.equal(a[key], b[key]), key
    # 20 tail queries take the split plan; their rows must match the prefill run closely
    q0 = cfg.T - 20
    c = lcr.routed_attention(dev["q"], dev["k"], dev["v"], a["idx"][:, :, q0:].contiguous(),
                             a["zsel"][:, :, q0:].contiguous(), radius=cfg.R, scale=cfg.scale, q0=q0, nq=20)
    torch.cuda.synchronize()
    sl = torch.from_numpy(O.slot_of(np.arange(q0, cfg.T))).cuda()
    assert max_err(f64(c[:, :, sl]), f64(a["o"][:, :, sl])) < 1e-2


# ----------------------------------------------------------------------------- SWA

SWA_CASES = [
    ("fp32 tiny", dict(B=1, Hq=2, Hkv=1, L=1024, d=64, R=64, dtype="fp32")),
    ("fp32 ragged L", dict(B=2, Hq=4, Hkv=2, L=333, d=64, R=50, dtype="fp32")),
    ("bf16 radius 1280", dict(B=1, Hq=28, Hkv=4, L=8192, d=128, R=1280, dtype="bf16")),
    ("bf16 dense", dict(B=1, Hq=8, Hkv=1, L=700, d=128, R=5000, dtype="bf16")),
    ("bf16 radius 0", dict(B=1, Hq=4, Hkv=4, L=256, d=128, R=0, dtype="bf16")),
    # two loading waves (3 heads per group), d = 64, ragged last tile and block, batch 2
    ("bf16 d64 ragged", dict(B=2, Hq=6, Hkv=2, L=333, d=64, R=100, dtype="bf16")),
    # a sequence shorter than one 64-slot tile
    ("bf16 short", dict(B=1, Hq=4, Hkv=2, L=40, d=128, R=10, dtype="bf16")),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("L,R,label", [(65536, 1280, "64K radius 1280"), (16384, 16384, "16K dense"),
                                       (131072, 131072, "128K dense")])
def test_swa_full_size_sampled(L, R, label):
    """The bench's SWA layer (65,536 slots, radius 1280) and dense layers (16,384 and
    131,072 slots, R >= L), 28/4 heads, d = 128, bf16, in the launch configuration the
    bench times; the oracle computes 120 sampled rows (both ends and random interior
    slots)."""
    from lcr_inputs import bf16_round
    print(f"[case] swa full size {label}", flush=True)
    B, Hq, Hkv, d = 1, 28, 4, 128
    rng = np.random.default_rng([88, L, R])
    q = bf16_round(rng.standard_normal((B, Hq, L, d), dtype=np.float32))
    k = bf16_round(rng.standard_normal((B, Hkv, L, d), dtype=np.float32))
    v = bf16_round(rng.standard_normal((B, Hkv, L, d), dtype=np.float32))
    scale = 1.0 / np.sqrt(d)
    o, lse = lcr.swa_attention(to_dev(q), to_dev(k), to_dev(v), radius=R, scale=scale, want_lse=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(40), np.arange(L - 40, L), rng.choice(L, size=40, replace=False)]))
    ro, rl = O.swa_attention(_RowView(q), as_f64(k), as_f64(v), R, scale, rows)
    o_err = max_err(f64(o[:, :, torch.from_numpy(rows).cuda()]), ro)
    l_err = max_err(f64(lse[:, :, torch.from_numpy(rows).cuda()]), rl)
    print(f"    o_err={o_err:.2e} lse_err={l_err:.2e}", flush=True)
    assert o_err < OUT_TOL["bf16"] and l_err < LSE_TOL["bf16"]


class _RowView:
    """q for the oracle without upcasting all of it: shape, and rows upcast on access."""

    def __init__(self, q):
        self.q, self.shape = q, q.shape

    def __getitem__(self, ix):
        return as_f64(self.q[ix])


@pytest.mark.parametrize("case", SWA_CASES, ids=[c[0] for c in SWA_CASES])
def test_swa(case):
    name, c = case
    print(f"[case] swa {name} {c}", flush=True)
    rng = np.random.default_rng([77, c["L"], c["R"]])
    shape_q = (c["B"], c["Hq"], c["L"], c["d"])
    shape_k = (c["B"], c["Hkv"], c["L"], c["d"])
    from lcr_inputs import bf16_round
    mk = (lambda s: bf16_round(rng.standard_normal(s, dtype=np.float32))) if c["dtype"] == "bf16" else \
        (lambda s: rng.standard_normal(s, dtype=np.float32))
    q, k, v = mk(shape_q), mk(shape_k), mk(shape_k)
    scale = 1.0 / np.sqrt(c["d"])
    o, lse = lcr.swa_attention(to_dev(q), to_dev(k), to_dev(v), radius=c["R"], scale=scale, want_lse=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, min(70, c["L"])), np.arange(max(0, c["L"] - 70), c["L"]),
                                     rng.choice(c["L"], size=min(100, c["L"]), replace=False)]))
    ro, rl = O.swa_attention(as_f64(q), as_f64(k), as_f64(v), c["R"], scale, rows)
    o_err = max_err(f64(o)[:, :, rows], ro)
    l_err = max_err(f64(lse)[:, :, rows], rl)
    print(f"    o_err={o_err:.2e} lse_err={l_err:.2e}", flush=True)
    assert o_err < OUT_TOL[c["dtype"]] and l_err < LSE_TOL[c["dtype"]]


@pytest.mark.timeout(600)
def test_stack_64k_route_layer_sampled():
    """A route layer of the 64K stack (N = 1,024 chunks: scoring takes the general path, the
    routed kernel its chunk pool with 1,024 positions), inputs drawn on the device; the
    oracle gets the same bits copied back (mask-query rows, sampled query and x rows, K, V)."""
    from lcr_inputs import stack_layer_torch
    cfg = get_config("stack_64k")
    print(f"[case] stack_64k route layer 3: N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} K={cfg.K} R={cfg.R}", flush=True)
    t = stack_layer_torch(cfg, 3, "cuda", route=True)
    res = lcr.route_layer(t["q"], t["k"], t["v"], t["x"], t["A"], t["Bm"], K=cfg.K, radius=cfg.R, beta=cfg.beta,
                          scale=cfg.scale, want_lse=True)
    torch.cuda.synchronize()
    queries = sample_query_blocks(cfg.T, n_blocks=4, block=32, seed=11)
    slots = torch.from_numpy(O.slot_of(queries)).cuda()
    q_rows = f64(t["q"][:, :, slots])
    q_mask = f64(t["q"].view(cfg.B, cfg.Hq, cfg.N, 64, cfg.d)[:, :, :, 63])
    x_rows = f64(t["x"][:, slots])
    k, v, A, Bm = f64(t["k"]), f64(t["v"]), f64(t["A"]), f64(t["Bm"])
    ref = O.route_layer_rows(q_rows, q_mask, k, v, x_rows, A, Bm, K=cfg.K, R=cfg.R, beta=cfg.beta, scale=cfg.scale,
                             queries=queries)
    tq = queries
    idx_gpu = res["idx"][:, :, torch.from_numpy(tq).cuda()].cpu().numpy().astype(np.int64)
    same = check_selection(idx_gpu, ref, cfg.K, "stack_64k")
    fin = np.isfinite(ref["zsel"])
    zg = f64(res["zsel"][:, :, torch.from_numpy(tq).cuda()])
    sm = np.broadcast_to(np.repeat(same, cfg.G, axis=1)[..., None], fin.shape) & fin
    z_err = max_err(zg[sm], ref["zsel"][sm])
    rows_same = same.all(axis=(0, 1))
    o_gpu = f64(res["o"][:, :, slots])
    o_err = max_err(o_gpu[:, :, rows_same], ref["o"][:, :, rows_same])
    l_err = max_err(f64(res["lse"][:, :, torch.from_numpy(tq).cuda()])[:, :, rows_same], ref["lse"][:, :, rows_same])
    print(f"    rows={len(tq)} same={int(rows_same.sum())} o_err={o_err:.2e} lse_err={l_err:.2e} z_err={z_err:.2e}",
          flush=True)
    assert rows_same.sum() >= len(tq) // 2, "too few rows with the oracle's own selection to compare"
    assert o_err < OUT_TOL["bf16"] and l_err < LSE_TOL["bf16"]
    assert z_err < Z_TOL["bf16"] * max(1.0, np.abs(ref["zsel"][sm]).max())
