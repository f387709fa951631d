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
    # batch 2 over few rounds of blocks: the pooled kernel takes fewer than 44 queries per block
    ("batch 2", dict(B=2, beta=0.5)),
    # past 512 chunks the fused scoring takes 32-query blocks with 16 keys per lane
    ("700 chunks, entropy term", dict(N=700, K=32, beta=0.5)),
    ("1024 chunks, head dim 64", dict(N=1024, d=64, K=32)),
    # past 1,024 chunks the one-sweep scoring: batches of 64 chunks, or of 32 for groups of 8 heads
    ("1100 chunks, entropy term", dict(N=1100, K=32, beta=0.5)),
    ("1100 chunks, eight-head groups", dict(N=1100, Hq=16, Hkv=2, K=32)),
    ("1100 chunks, head dim 64, K=17, ragged query range", dict(N=1100, d=64, K=17), 20000, 3001),
    ("1100 chunks, K=1", dict(N=1100, K=1)),
    ("1100 chunks, batch 2", dict(N=1100, B=2, K=8, beta=0.25)),
    # float32 past 1,024 chunks: per-head scores through memory, the block-tiled routed kernel
    ("1100 chunks, float32", dict(N=1100, Hq=2, Hkv=1, d=64, K=8, dtype="fp32")),
    # K = 64 with groups of 8 heads does not fit the one-sweep kernel: the general path
    ("1100 chunks, eight-head groups, K=64", dict(N=1100, Hq=16, Hkv=2, K=64, R=30)),
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


@pytest.mark.parametrize("N", [600, 1200])
def test_topk_exact_ties_many_chunks(N):
    """Exact ties in the group maximum at N = 600 (the two-sweep fused scoring, 16 keys per
    lane) and N = 1,200 (the one-sweep fused scoring, 19 batches, the last one partial):
    chunk 2i + 1 has the summary and entropy of chunk 2i, so every score occurs twice. The
    chosen set must be a top K of the oracle's group maxima; where twins straddle the
    threshold, the smaller chunk is chosen (the oracle's tie rule); rows whose K-th and
    (K+1)-th scores differ by more than 1e-3 match the oracle exactly."""
    B, Hq, Hkv, d, r, D, K, R, beta = 1, 8, 2, 128, 16, 96, 31, 200, 0.5
    G, L, T = Hq // Hkv, N * 64, N * 63
    print(f"[case] top-K ties N={N} K={K} Hq={Hq} Hkv={Hkv}", flush=True)
    rng = np.random.default_rng(2024)

    def bf16(shape, std=1.0):
        return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16)
    q, x = bf16((B, Hq, L, d)), bf16((B, L, D))
    A, Bm = bf16((D, r), 0.02), bf16((r, Hq * d), 0.02)
    s = rng.standard_normal((B, Hq, N // 2, d)).repeat(2, axis=2).astype(np.float32)
    H = (rng.random((B, Hq, N // 2)) * 4.0).repeat(2, axis=2).astype(np.float32)
    idx, zsel = lcr.route_score_topk(q.cuda(), x.cuda(), A.cuda(), Bm.cuda(), torch.from_numpy(s).cuda(),
                                     torch.from_numpy(H).cuda(), Hkv=Hkv, K=K, radius=R, beta=beta)
    torch.cuda.synchronize()
    queries = np.unique(np.concatenate([np.arange(0, 64), np.arange(T // 2, T // 2 + 64), np.arange(T - 64, T)]))
    f = lambda t: t.float().numpy().astype(np.float64)
    slots = O.slot_of(queries)
    qt = O.routing_query(f(q)[:, :, slots], f(x)[:, slots], f(A), f(Bm))
    zhat = O.group_max(O.route_scores(qt, s.astype(np.float64), H.astype(np.float64), beta, 1.0 / np.sqrt(d)), G)
    cand = O.candidate_mask(queries, R, N)
    ref_idx, margin = O.select_topk(zhat, cand, K)
    got = idx.cpu().numpy()[:, :, queries].astype(np.int64)
    straddle = 0
    for b in range(B):
        for g in range(Hkv):
            for j in range(len(queries)):
                row = got[b, g, j]
                assert np.all(np.diff(row) > 0) and row.min() >= 0, "ascending distinct chunk ids"
                chosen = np.zeros(N, bool)
                chosen[row] = True
                assert cand[j][row].all(), "only candidates"
                z = zhat[b, g, j]
                left = cand[j] & ~chosen
                assert z[chosen].min() >= z[left].max() - 1e-4, "a top K of the group maxima"
                for c in range(0, N, 2):   # twins straddling the threshold: the smaller id
                    if cand[j][c] and cand[j][c + 1] and chosen[c] != chosen[c + 1]:
                        straddle += 1
                        assert chosen[c], f"twin {c + 1} chosen over {c}"
                if margin[b, g, j] > 1e-3:
                    assert np.array_equal(row, ref_idx[b, g, j]), "selection differs from the oracle"
    print(f"    rows={B * Hkv * len(queries)} twins straddling the threshold: {straddle}", flush=True)
    assert straddle > 0


def _routed_plan_ws(cfg, K, nq):
    dims = lcr.make_dims(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d,
                         torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)
    return lcr.workspace_bytes(2, dims, 0, 0, K, nq, cfg.R)


def test_determinism_and_decode_split_matches_prefill():
    """The pooled prefill kernel (a producer wave and consumer waves synchronised through
    LDS counters) gives the same bits on two runs; the split decode plan on the tail
    queries agrees with it to the output tolerance. N = 128 chunks, 8/2 heads: 538
    blocks, so the whole-range call takes the pooled plan (no workspace); 20 tail
    queries take the split plan (one partial per run of entries)."""
    cfg = get_config("tiny_fp32", N=128, Hq=8, Hkv=2, d=128, r=32, D=256, K=8, R=128, dtype="bf16")
    print("[case] determinism of the pooled prefill plan", flush=True)
    assert _routed_plan_ws(cfg, cfg.K, cfg.T) == 0, "the whole-range call must take the pooled prefill plan"
    assert _routed_plan_ws(cfg, cfg.K, 20) > 0, "the tail call must take the split decode plan"
    inp = route_inputs(cfg)
    dev = {k: to_dev(v) for k, v in inp.items()}
    runs = [lcr.route_layer(dev["q"], dev["k"], dev["v"], dev["x"], dev["A"], dev["Bm"], K=cfg.K, radius=cfg.R,
                            scale=cfg.scale, want_lse=True) for _ in range(2)]
    torch.cuda.synchronize()
    a, b = runs
    for key in ["s", "H", "idx", "zsel", "o", "lse"]:
        assert torch.equal(a[key], b[key]), key
    # the routed attention alone, twice more on the first run's selection
    o1, l1 = lcr.routed_attention(dev["q"], dev["k"], dev["v"], a["idx"], a["zsel"], radius=cfg.R, scale=cfg.scale,
                                  want_lse=True)
    o2, l2 = lcr.routed_attention(dev["q"], dev["k"], dev["v"], a["idx"], a["zsel"], radius=cfg.R, scale=cfg.scale,
                                  want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1, a["o"])
    # 20 tail queries take the split plan; their rows must match the prefill run closely
    q0 = cfg.T - 20
    c, lc = lcr.routed_attention(dev["q"], dev["k"], dev["v"], a["idx"][:, :, q0:].contiguous(),
                                 a["zsel"][:, :, q0:].contiguous(), radius=cfg.R, scale=cfg.scale, q0=q0, nq=20,
                                 want_lse=True)
    torch.cuda.synchronize()
    sl = torch.from_numpy(O.slot_of(np.arange(q0, cfg.T))).cuda()
    assert max_err(f64(c[:, :, sl]), f64(a["o"][:, :, sl])) < OUT_TOL["bf16"]
    assert max_err(f64(lc), f64(a["lse"][:, :, q0:])) < LSE_TOL["bf16"]


@pytest.mark.parametrize("heads", [(28, 4, 128), (16, 2, 64), (4, 2, 128)], ids=lambda h: f"{h[0]}/{h[1]} d{h[2]}")
def test_routed_attention_chunk_logit_extremes(heads):
    """The pooled prefill kernel on given selections whose chunk logits force every
    branch of its online softmax, checked against the oracle: rows whose logits climb
    by 12 at each selected chunk (a rescale at every remote visit), fall by 12, lie far
    below the window (chunk weights near zero), or are ordinary; some rows select fewer
    chunks than K (-1 / -inf padding). Most remote visits have one active query of the
    tile, the path whose lane pairs share that query's scores. N = 128; GQA groups of 7,
    8 and 2 heads (idle head lanes in the tile), d = 128 and 64."""
    Hq, Hkv, d = heads
    cfg = get_config("tiny_fp32", N=128, Hq=Hq, Hkv=Hkv, d=d, r=32, D=256, K=8, R=64, dtype="bf16")
    print(f"[case] chunk logit extremes: N=128 Hq={Hq} Hkv={Hkv} d={d} K=8 R=64 bf16", flush=True)
    assert _routed_plan_ws(cfg, cfg.K, cfg.T) == 0, "the whole-range call must take the pooled prefill plan"
    inp = route_inputs(cfg)
    rng = np.random.default_rng(20261204)
    B, Hq, Hkv, G, K, T = cfg.B, cfg.Hq, cfg.Hkv, cfg.G, cfg.K, cfg.T
    idx = np.full((B, Hkv, T, K), -1, dtype=np.int32)
    zsel = np.full((B, Hq, T, K), -np.inf, dtype=np.float32)
    c = np.arange(cfg.N)
    for t in range(T):
        # remote chunks of query t: none of their content indices lies in its window
        cand = c[(63 * c + 62 < t - cfg.R) | (63 * c > t + cfg.R)]
        m = min(K, len(cand)) - (3 if t % 7 == 0 else 0)
        kk = np.arange(m)
        pattern = t % 4
        for g in range(Hkv):
            idx[0, g, t, :m] = np.sort(rng.choice(cand, size=m, replace=False))
            for hh in range(G):
                if pattern == 0:
                    z = -20.0 + 12.0 * kk
                elif pattern == 1:
                    z = 40.0 - 12.0 * kk
                elif pattern == 2:
                    z = np.full(m, -60.0)
                else:
                    z = rng.normal(0.0, 2.0, size=m)
                zsel[0, g * G + hh, t, :m] = z + 0.5 * hh
    dev = {k: to_dev(v) for k, v in inp.items() if k in ("q", "k", "v")}
    o, lse = lcr.routed_attention(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx).cuda(),
                                  torch.from_numpy(zsel).cuda(), radius=cfg.R, scale=cfg.scale, want_lse=True)
    torch.cuda.synchronize()
    queries = np.unique(np.concatenate([np.arange(0, 44), np.arange(4000, 4044), np.arange(T - 44, T),
                                        rng.choice(T, size=40, replace=False)]))
    f = _f(inp)
    o_ref, l_ref = O.routed_attention(f["q"][:, :, O.slot_of(queries)], f["k"], f["v"], idx[:, :, queries].astype(np.int64),
                                      zsel[:, :, queries].astype(np.float64), cfg.R, cfg.scale, queries)
    o_err = max_err(f64(o)[:, :, O.slot_of(queries)], o_ref)
    l_err = max_err(f64(lse)[:, :, queries], l_ref)
    print(f"    rows={len(queries)} o_err={o_err:.2e} lse_err={l_err:.2e}", flush=True)
    assert o_err < OUT_TOL["bf16"], f"output error {o_err:.3e}"
    assert l_err < LSE_TOL["bf16"], f"lse error {l_err:.3e}"


def test_tile_order_independence():
    """The tiled kernels (fused scoring, pooled routed attention) give the same bits when
    their blocks walk the tiles in reversed order: no block depends on another or on the
    order in which the hardware dispatches them. Same layer as the determinism test
    (N = 128, 8/2 heads: the fused scoring and the pooled prefill plan)."""
    cfg = get_config("tiny_fp32", N=128, Hq=8, Hkv=2, d=128, r=32, D=256, K=8, R=128, dtype="bf16")
    print("[case] tile order independence of the tiled prefill kernels", flush=True)
    assert _routed_plan_ws(cfg, cfg.K, cfg.T) == 0, "the whole-range call must take the pooled prefill plan"
    inp = route_inputs(cfg)
    dev = {k: to_dev(v) for k, v in inp.items()}
    run = lambda: lcr.route_layer(dev["q"], dev["k"], dev["v"], dev["x"], dev["A"], dev["Bm"], K=cfg.K,
                                  radius=cfg.R, scale=cfg.scale, want_lse=True)
    a = run()
    prev = lcr.set_tile_order(True)
    try:
        assert prev == 0
        b = run()
        torch.cuda.synchronize()
    finally:
        lcr.set_tile_order(False)
    for key in ["s", "H", "idx", "zsel", "o", "lse"]:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("d", [64, 128])
def test_route_layer_fp32_prefill_plan(d):
    """float32 inputs at a size whose routed attention takes the block-per-query-range
    plan (N = 128 chunks, 8/2 heads: 504 blocks of 32 queries, three bf16 operand planes
    per float32 value) rather than the split decode plan, which the tiny float32 cases
    take; sampled query blocks against the oracle at the float32 tolerance."""
    cfg = get_config("tiny_fp32", N=128, Hq=8, Hkv=2, d=d, r=16, D=96, K=8, R=128, beta=0.3, dtype="fp32")
    assert _routed_plan_ws(cfg, cfg.K, cfg.T) == 0, "float32 at this size must not take the split plan"
    queries = sample_query_blocks(cfg.T, n_blocks=4, block=64, seed=21)
    route_parity(cfg, queries=queries, label=f"fp32 prefill plan d={d}")


def _nan_or_equal(got, ref, what):
    """Per row (all trailing axes), either every value is NaN or the row equals ref bit for bit."""
    g = got.reshape(-1, got.shape[-1]) if got.dim() > 1 else got.reshape(-1, 1)
    r = ref.reshape(-1, ref.shape[-1]) if ref.dim() > 1 else ref.reshape(-1, 1)
    nan_rows = torch.isnan(g).all(dim=1)
    partial = torch.isnan(g).any(dim=1) & ~nan_rows
    assert not bool(partial.any()), f"{what}: rows with some NaN values"
    assert torch.equal(g[~nan_rows], r[~nan_rows]), f"{what}: a completed row differs from the normal run"
    return int(nan_rows.sum())


def test_wait_give_up_writes_nan_rows():
    """Failure handling of the pooled kernels, forced from the host: with a wait limit of one
    poll, waves give up on their LDS counters, stop, and write NaN to the rows they own; every
    kernel still exits. Rows of waves that finished are the normal run's bits. The default
    limit is restored before the test ends."""
    cfg = get_config("tiny_fp32", N=128, Hq=8, Hkv=2, d=128, r=32, D=256, K=8, R=128, dtype="bf16")
    print("[case] wait give-up: forward and backward with a one-poll wait limit", flush=True)
    assert _routed_plan_ws(cfg, cfg.K, cfg.T) == 0
    inp = route_inputs(cfg)
    dev = {k: to_dev(v) for k, v in inp.items()}
    ref = lcr.route_layer(dev["q"], dev["k"], dev["v"], dev["x"], dev["A"], dev["Bm"], K=cfg.K, radius=cfg.R,
                          scale=cfg.scale, want_lse=True)
    dO = torch.randn(dev["q"].shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    args = (dev["q"], dev["k"], dev["v"], ref["idx"], ref["zsel"], ref["o"], ref["lse"], dO)
    bref = lcr.routed_attention_backward(*args, radius=cfg.R, scale=cfg.scale)
    torch.cuda.synchronize()
    sl = torch.from_numpy(O.slot_of(np.arange(cfg.T))).cuda()
    assert not bool(torch.isnan(ref["o"][:, :, sl].float()).any()) and not bool(torch.isnan(bref[0]).any())
    prev = lcr.set_wait_limit(1)
    try:
        o, lse = lcr.routed_attention(dev["q"], dev["k"], dev["v"], ref["idx"], ref["zsel"], radius=cfg.R,
                                      scale=cfg.scale, want_lse=True)
        dq, _, _, dz = lcr.routed_attention_backward(*args, radius=cfg.R, scale=cfg.scale)
        torch.cuda.synchronize()
    finally:
        lcr.set_wait_limit(0)
    assert prev == 1 << 22
    n_o = _nan_or_equal(o[:, :, sl].float(), ref["o"][:, :, sl].float(), "o")
    n_l = _nan_or_equal(lse.unsqueeze(-1), ref["lse"].unsqueeze(-1), "lse")
    n_dq = _nan_or_equal(dq[:, :, sl], bref[0][:, :, sl], "dq")
    n_dz = _nan_or_equal(dz, bref[3], "dzsel")
    print(f"    NaN rows: o {n_o}, lse {n_l}, dq {n_dq}, dzsel {n_dz} of {cfg.Hq * cfg.T}", flush=True)
    assert n_o > 0 and n_o == n_l, "a give-up must show as NaN rows of o and lse alike"
    assert n_dq > 0 and n_dq == n_dz
    # the default limit is back: a normal call again
    o3 = lcr.routed_attention(dev["q"], dev["k"], dev["v"], ref["idx"], ref["zsel"], radius=cfg.R, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(o3, ref["o"])


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
    # one head per group (a single wave loads and computes: three-tile ring at d = 128),
    # radius wide enough for runs of tiles inside every row's window
    ("bf16 one head per group", dict(B=1, Hq=2, Hkv=2, L=1500, d=128, R=600, dtype="bf16")),
    ("bf16 d64 one head per group", dict(B=1, Hq=2, Hkv=2, L=900, d=64, R=300, dtype="bf16")),
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


def _random_swa_cases(n=10, seed=4242):
    """Seeded shapes across the SWA kernel's plans: 1 to 8 heads per group (one, two or four
    loading waves), d 64 / 128, any length and radius (partial tiles, radii past the
    sequence, radius 0), bf16 and float32."""
    rng = np.random.default_rng(seed)
    out = []
    for j in range(n):
        G = int(rng.choice([1, 2, 3, 4, 7, 8]))
        Hkv = int(rng.choice([1, 2]))
        L = int(rng.integers(1, 1600))
        mode = int(rng.integers(0, 3))
        R = 0 if mode == 0 else int(rng.integers(1, 200) if mode == 1 else rng.integers(L // 2 + 1, 2 * L + 2))
        d = int(rng.choice([64, 128]))
        dt = "fp32" if j % 4 == 3 else "bf16"
        out.append((f"random {j}", dict(B=int(rng.integers(1, 3)), Hq=G * Hkv, Hkv=Hkv, L=L, d=d, R=R, dtype=dt)))
    return out


@pytest.mark.parametrize("case", _random_swa_cases(), ids=lambda c: c[0])
def test_swa_random_shapes(case):
    test_swa(case)


def _random_route_cases(n=8, seed=5151):
    """Seeded whole-layer shapes: chunk counts from 2 to 48, GQA groups of 1 to 8 heads,
    d 64 / 128, K 0 to 16, radii from 0 past the sequence, partial query ranges, an
    entropy weight, bf16 and float32."""
    rng = np.random.default_rng(seed)
    out = []
    for j in range(n):
        N = int(rng.integers(2, 49))
        G = int(rng.choice([1, 2, 4, 7, 8]))
        Hkv = int(rng.choice([1, 2]))
        T = N * 63
        q0 = int(rng.integers(0, T // 2)) if j % 3 == 1 else 0
        nq = int(rng.integers(1, T - q0 + 1)) if j % 3 == 1 else None
        dt = "fp32" if j % 4 == 2 else "bf16"
        over = dict(N=N, Hq=G * Hkv, Hkv=Hkv, d=int(rng.choice([64, 128])), r=16, D=96,
                    K=int(rng.integers(0, 17)), R=[0, int(rng.integers(1, 300)), 4000][int(rng.integers(0, 3))],
                    beta=float(rng.choice([0.0, 0.5])), dtype=dt)
        out.append((f"random {j}", over, q0, nq))
    return out


@pytest.mark.parametrize("case", _random_route_cases(), ids=lambda c: c[0])
def test_route_layer_random_shapes(case):
    name, over, q0, nq = case
    cfg = get_config("tiny_fp32", **over)
    route_parity(cfg, q0=q0, nq=nq, label=f"{name} {over} q0={q0} nq={nq}")


def _device_route_layer_sampled(cfg, layer, label, n_blocks=4, seed=11):
    """A route layer with inputs drawn on the device; the oracle gets the same bits copied
    back (mask-query rows, sampled query and x rows, K, V) and checks sampled queries."""
    from lcr_inputs import stack_layer_torch
    print(f"[case] {label}: N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} K={cfg.K} R={cfg.R}", flush=True)
    t = stack_layer_torch(cfg, layer, "cuda", route=True)
    res = lcr.route_layer(t["q"], t["k"], t["v"], t["x"], t["A"], t["Bm"], K=cfg.K, radius=cfg.R, beta=cfg.beta,
                          scale=cfg.scale, want_lse=True)
    torch.cuda.synchronize()
    queries = sample_query_blocks(cfg.T, n_blocks=n_blocks, block=32, seed=seed)
    slots = torch.from_numpy(O.slot_of(queries)).cuda()
    q_rows = f64(t["q"][:, :, slots])
    q_mask = f64(t["q"].view(cfg.B, cfg.Hq, cfg.N, 64, cfg.d)[:, :, :, 63])
    x_rows = f64(t["x"][:, slots])
    k, v, A, Bm = f64(t["k"]), f64(t["v"]), f64(t["A"]), f64(t["Bm"])
    ref = O.route_layer_rows(q_rows, q_mask, k, v, x_rows, A, Bm, K=cfg.K, R=cfg.R, beta=cfg.beta, scale=cfg.scale,
                             queries=queries)
    tq = queries
    idx_gpu = res["idx"][:, :, torch.from_numpy(tq).cuda()].cpu().numpy().astype(np.int64)
    same = check_selection(idx_gpu, ref, cfg.K, label)
    # every sampled row is checked: rows whose selection differs from the oracle's (ungated
    # near-ties) get the oracle's attention recomputed with the GPU's chunks and its scores
    zref = O.gather_zsel(ref["z"], idx_gpu, cfg.G)
    fin = np.isfinite(zref)
    zg = f64(res["zsel"][:, :, torch.from_numpy(tq).cuda()])
    assert np.array_equal(fin, np.isfinite(zg)), "zsel padding"
    z_err = max_err(zg[fin], zref[fin])
    o_ref, lse_ref = ref["o"].copy(), ref["lse"].copy()
    diff_t = np.nonzero(~same.all(axis=(0, 1)))[0]
    if len(diff_t):
        o2, l2 = O.routed_attention(q_rows[:, :, diff_t], k, v, idx_gpu[:, :, diff_t], zref[:, :, diff_t], cfg.R,
                                    cfg.scale, queries[diff_t])
        o_ref[:, :, diff_t], lse_ref[:, :, diff_t] = o2, l2
    o_err = max_err(f64(res["o"][:, :, slots]), o_ref)
    l_err = max_err(f64(res["lse"][:, :, torch.from_numpy(tq).cuda()]), lse_ref)
    print(f"    rows={len(tq)} same={int(same.all(axis=(0, 1)).sum())} recomputed={len(diff_t)} o_err={o_err:.2e} "
          f"lse_err={l_err:.2e} z_err={z_err:.2e}", flush=True)
    assert o_err < OUT_TOL["bf16"] and l_err < LSE_TOL["bf16"]
    assert z_err < Z_TOL["bf16"] * max(1.0, np.abs(zref[fin]).max())


@pytest.mark.timeout(600)
def test_stack_64k_route_layer_sampled():
    """A route layer of the 64K stack (N = 1,024 chunks: the two-sweep fused scoring at its
    largest N, the routed kernel's chunk pool with 1,024 positions)."""
    _device_route_layer_sampled(get_config("stack_64k"), 3, "stack_64k route layer 3")


@pytest.mark.timeout(600)
def test_prefill_128k_route_layer_sampled():
    """A 128K prefill route layer (N = 2,048 chunks, 129,024 queries): the one-sweep fused
    scoring (selection merged batch by batch) and a smaller chunk pool in the routed kernel."""
    _device_route_layer_sampled(get_config("stack_64k", N=2048), 5, "prefill 128K route layer", seed=12)
