"""Backward of routed attention: HIP path against the fp64 oracle, through the C ABI.

Selections: random chunk scores ranked over each query's remote chunks by the
oracle's own candidate and top-K functions (any valid selection is a valid
input to the backward), or, in one case, the oracle route layer's selection.
Chunk logits are seeded normals. Both sides receive identical bits.

Tolerance: bf16 products with the probabilities and their gradients rounded to
bf16 (relative 2^-9 each) and float32 sums, so every gradient must lie within
2e-2 of the oracle's in max-abs error relative to max(1, max |oracle|).

Tiny cases are checked in full. The 16K prefill layer runs at full size in the
launch configuration the benchmark times; dq and dzsel are checked on sampled
query blocks, dk and dv on sampled chunks against the oracle run over every
query that reaches those chunks (its window queries and every query that
selected it).
"""
import numpy as np
import pytest
import torch

import learned_chunk_routed_amd as lcr
from lcr_inputs import as_f64, backward_draws, get_config, route_inputs, sample_query_blocks
from oracle import backward as OB
from oracle import route as O
from gpu_util import to_dev, f64

pytestmark = pytest.mark.gpu

BWD_TOL = 2e-2
SL, CT = 64, 63


def rel_err(a, b):
    b = np.asarray(b)
    if b.size == 0:
        return 0.0
    return float(np.max(np.abs(np.asarray(a) - b))) / max(1.0, float(np.max(np.abs(b))))


def selection(cfg, draws, q0, nq):
    """idx [B,Hkv,nq,K] int64 and zsel [B,Hq,nq,K] (float32 values, -inf padding)."""
    queries = np.arange(q0, q0 + nq)
    cand = O.candidate_mask(queries, cfg.R, cfg.N)
    idx, _ = O.select_topk(draws["score"].astype(np.float64), cand, cfg.K)
    fin = np.repeat(idx, cfg.G, axis=1) >= 0
    zsel = np.where(fin, draws["zsel"], -np.inf).astype(np.float32)
    return idx, zsel


def run_gpu(cfg, inp, dO_bits, idx, zsel, q0, nq):
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
    z_t = torch.from_numpy(np.ascontiguousarray(zsel)).cuda()
    o, lse = lcr.routed_attention(q, k, v, idx_t, z_t, radius=cfg.R, scale=cfg.scale, q0=q0, nq=nq,
                                  want_lse=True)
    dq, dk, dv, dz = lcr.routed_attention_backward(q, k, v, idx_t, z_t, o, lse, to_dev(dO_bits), radius=cfg.R,
                                                   scale=cfg.scale, q0=q0, nq=nq)
    torch.cuda.synchronize()
    return f64(dq), f64(dk), f64(dv), f64(dz)


TINY = {
    "d128 G4": dict(N=12, Hq=8, Hkv=2, d=128, K=3, R=40),
    "d64 G1 ragged partial range": dict(N=10, Hq=2, Hkv=2, d=64, K=2, R=20, q0=37, nq=301),
    "G8 fewer candidates than K": dict(N=8, Hq=8, Hkv=1, d=128, K=6, R=150),
    "window only K=0": dict(N=8, Hq=4, Hkv=1, d=64, K=0, R=70),
    "B2 G7": dict(B=2, N=9, Hq=14, Hkv=2, d=128, K=4, R=30),
    "radius 0": dict(N=6, Hq=4, Hkv=1, d=128, K=2, R=0),
}


@pytest.mark.parametrize("name", sorted(TINY))
def test_backward_tiny(name):
    kw = dict(TINY[name])
    q0 = kw.pop("q0", 0)
    nq = kw.pop("nq", None)
    cfg = get_config("prefill_16k", dtype="bf16", **kw)
    nq = cfg.T - q0 if nq is None else nq
    print(f"[case] backward {name}: B={cfg.B} N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} K={cfg.K} R={cfg.R} "
          f"q0={q0} nq={nq}", flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, q0, nq)
    idx, zsel = selection(cfg, dr, q0, nq)
    gq, gk, gv, gz = run_gpu(cfg, inp, dr["dO"], idx, zsel, q0, nq)
    queries = np.arange(q0, q0 + nq)
    sl = O.slot_of(queries)
    q, k, v = as_f64(inp["q"]), as_f64(inp["k"]), as_f64(inp["v"])
    dO = as_f64(dr["dO"])
    rq, rk, rv, rz = OB.routed_attention_backward(q[:, :, sl], k, v, idx, zsel.astype(np.float64), cfg.R,
                                                  cfg.scale, queries, dO[:, :, sl])
    errs = dict(dq=rel_err(gq[:, :, sl], rq), dk=rel_err(gk, rk), dv=rel_err(gv, rv),
                dzsel=rel_err(np.where(np.isfinite(zsel), gz, 0.0), rz))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e < BWD_TOL, f"{name}: {n} error {e:.3e}"
    # rows outside the queried set stay zero in the binding's dq; mask-slot rows of dk, dv are zero
    other = np.setdiff1d(np.arange(cfg.L), sl)
    assert np.all(gq[:, :, other] == 0)
    assert np.all(gk[:, :, SL - 1::SL] == 0) and np.all(gv[:, :, SL - 1::SL] == 0)
    if cfg.K:
        assert np.all(gz[~np.isfinite(zsel)] == 0), "padded selections get no gradient"


@pytest.mark.parametrize("name", sorted(TINY))
def test_backward_tiny_fp32(name):
    """float32 inputs take the plain float32 backward (vector ALUs, fixed order): every
    gradient within 1e-5 of the fp64 oracle (relative to its largest magnitude), two
    calls equal bit for bit, untouched rows zero."""
    kw = dict(TINY[name])
    q0 = kw.pop("q0", 0)
    nq = kw.pop("nq", None)
    cfg = get_config("prefill_16k", dtype="fp32", **kw)
    nq = cfg.T - q0 if nq is None else nq
    print(f"[case] float32 backward {name}: B={cfg.B} N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} K={cfg.K} "
          f"R={cfg.R} q0={q0} nq={nq}", flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, q0, nq)
    idx, zsel = selection(cfg, dr, q0, nq)
    gq, gk, gv, gz = run_gpu(cfg, inp, dr["dO"], idx, zsel, q0, nq)
    again = run_gpu(cfg, inp, dr["dO"], idx, zsel, q0, nq)
    for x, y, n in zip((gq, gk, gv, gz), again, ("dq", "dk", "dv", "dzsel")):
        assert np.array_equal(x, y), f"{n} differs between two identical calls"
    queries = np.arange(q0, q0 + nq)
    sl = O.slot_of(queries)
    q, k, v = as_f64(inp["q"]), as_f64(inp["k"]), as_f64(inp["v"])
    dO = as_f64(dr["dO"])
    rq, rk, rv, rz = OB.routed_attention_backward(q[:, :, sl], k, v, idx, zsel.astype(np.float64), cfg.R,
                                                  cfg.scale, queries, dO[:, :, sl])
    errs = dict(dq=rel_err(gq[:, :, sl], rq), dk=rel_err(gk, rk), dv=rel_err(gv, rv),
                dzsel=rel_err(np.where(np.isfinite(zsel), gz, 0.0), rz))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e < 1e-5, f"{name}: {n} error {e:.3e}"
    other = np.setdiff1d(np.arange(cfg.L), sl)
    assert np.all(gq[:, :, other] == 0)
    assert np.all(gk[:, :, SL - 1::SL] == 0) and np.all(gv[:, :, SL - 1::SL] == 0)
    if cfg.K:
        assert np.all(gz[~np.isfinite(zsel)] == 0), "padded selections get no gradient"


def test_backward_layer_selection():
    """The selection and chunk logits of the oracle route layer itself (a real top-K)."""
    cfg = get_config("prefill_16k", N=10, Hq=8, Hkv=2, d=128, K=3, R=30, beta=0.2)
    print("[case] backward with the oracle layer's own selection", flush=True)
    inp = route_inputs(cfg)
    f = {n: as_f64(inp[n]) for n in ("q", "k", "v", "x", "A", "Bm")}
    queries = np.arange(cfg.T)
    ref = O.route_layer(f["q"], f["k"], f["v"], f["x"], f["A"], f["Bm"], K=cfg.K, R=cfg.R, beta=cfg.beta,
                        scale=cfg.scale, queries=queries)
    zsel = ref["zsel"].astype(np.float32)
    dr = backward_draws(cfg, 0, cfg.T)
    gq, gk, gv, gz = run_gpu(cfg, inp, dr["dO"], ref["idx"], zsel, 0, cfg.T)
    sl = O.slot_of(queries)
    rq, rk, rv, rz = OB.routed_attention_backward(f["q"][:, :, sl], f["k"], f["v"], ref["idx"],
                                                  zsel.astype(np.float64), cfg.R, cfg.scale, queries,
                                                  as_f64(dr["dO"])[:, :, sl])
    errs = dict(dq=rel_err(gq[:, :, sl], rq), dk=rel_err(gk, rk), dv=rel_err(gv, rv),
                dzsel=rel_err(np.where(np.isfinite(zsel), gz, 0.0), rz))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e < BWD_TOL, f"{n} error {e:.3e}"


@pytest.mark.timeout(300)
def test_backward_prefill_16k_sampled():
    cfg = get_config("prefill_16k")
    q0, nq = 0, cfg.T
    print(f"[case] backward prefill_16k full size: N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} K={cfg.K} R={cfg.R}",
          flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, q0, nq)
    idx, zsel = selection(cfg, dr, q0, nq)
    gq, gk, gv, gz = run_gpu(cfg, inp, dr["dO"], idx, zsel, q0, nq)
    k, v = as_f64(inp["k"]), as_f64(inp["v"])
    G = cfg.G
    # dq and dzsel on sampled query blocks (all heads)
    queries = sample_query_blocks(cfg.T, n_blocks=4, block=32, seed=5)
    sl = O.slot_of(queries)
    qrows = as_f64(inp["q"][:, :, sl])
    dOrows = as_f64(dr["dO"][:, :, sl])
    rq, _, _, rz = OB.routed_attention_backward(qrows, k, v, idx[:, :, queries], zsel[:, :, queries].astype(
        np.float64), cfg.R, cfg.scale, queries, dOrows)
    e_q = rel_err(gq[:, :, sl], rq)
    zs = zsel[:, :, queries]
    e_z = rel_err(np.where(np.isfinite(zs), gz[:, :, queries], 0.0), rz)
    print(f"    sampled rows={len(queries)} dq={e_q:.2e} dzsel={e_z:.2e}", flush=True)
    assert e_q < BWD_TOL and e_z < BWD_TOL
    # dk and dv on sampled chunks: every query that reaches the chunk, one KV group at a time
    for g, c in ((0, 0), (2, cfg.N // 2 + 3)):
        lo, hi = max(0, c * CT - cfg.R), min(cfg.T - 1, c * CT + CT - 1 + cfg.R)
        sel_t = np.nonzero(np.any(idx[0, g] == c, axis=-1))[0]
        qs = np.union1d(np.arange(lo, hi + 1), sel_t)
        hs = slice(g * G, (g + 1) * G)
        slq = O.slot_of(qs)
        _, rk, rv, _ = OB.routed_attention_backward(
            as_f64(inp["q"][:, hs][:, :, slq]), k[:, g:g + 1], v[:, g:g + 1], idx[:, g:g + 1][:, :, qs],
            zsel[:, hs][:, :, qs].astype(np.float64), cfg.R, cfg.scale, qs, as_f64(dr["dO"][:, hs][:, :, slq]))
        rows = slice(c * SL, c * SL + SL)
        e_k = rel_err(gk[:, g, rows], rk[:, 0, rows])
        e_v = rel_err(gv[:, g, rows], rv[:, 0, rows])
        print(f"    group {g} chunk {c}: {len(qs)} queries ({len(sel_t)} selecting) dk={e_k:.2e} dv={e_v:.2e}",
              flush=True)
        assert e_k < BWD_TOL and e_v < BWD_TOL


def test_backward_decode_sized_tail():
    """32 tail queries of a 64-chunk sequence (the decode shape): one index tile, most
    chunks reached only through selections."""
    cfg = get_config("prefill_16k", N=64, K=8, R=256)
    q0, nq = cfg.T - 32, 32
    print(f"[case] backward decode-sized tail: N={cfg.N} K={cfg.K} q0={q0} nq={nq}", flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, q0, nq)
    idx, zsel = selection(cfg, dr, q0, nq)
    gq, gk, gv, gz = run_gpu(cfg, inp, dr["dO"], idx, zsel, q0, nq)
    queries = np.arange(q0, q0 + nq)
    sl = O.slot_of(queries)
    rq, rk, rv, rz = OB.routed_attention_backward(as_f64(inp["q"])[:, :, sl], as_f64(inp["k"]), as_f64(inp["v"]),
                                                  idx, zsel.astype(np.float64), cfg.R, cfg.scale, queries,
                                                  as_f64(dr["dO"])[:, :, sl])
    errs = dict(dq=rel_err(gq[:, :, sl], rq), dk=rel_err(gk, rk), dv=rel_err(gv, rv),
                dzsel=rel_err(np.where(np.isfinite(zsel), gz, 0.0), rz))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e < BWD_TOL, f"{n} error {e:.3e}"


def test_backward_reproducible_and_empty_range():
    """Two calls give identical bits (fixed summation order); nq = 0 writes zero dk, dv."""
    cfg = get_config("prefill_16k", N=40, Hq=8, Hkv=2, K=6, R=64)
    print("[case] backward reproducibility and nq = 0", flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, 0, cfg.T)
    idx, zsel = selection(cfg, dr, 0, cfg.T)
    a = run_gpu(cfg, inp, dr["dO"], idx, zsel, 0, cfg.T)
    b = run_gpu(cfg, inp, dr["dO"], idx, zsel, 0, cfg.T)
    for x, y, n in zip(a, b, ("dq", "dk", "dv", "dzsel")):
        assert np.array_equal(x, y), f"{n} differs between two identical calls"
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    e_idx = torch.zeros((1, cfg.Hkv, 0, cfg.K), dtype=torch.int32, device="cuda")
    e_z = torch.zeros((1, cfg.Hq, 0, cfg.K), dtype=torch.float32, device="cuda")
    e_l = torch.zeros((1, cfg.Hq, 0), dtype=torch.float32, device="cuda")
    dq, dk, dv, dz = lcr.routed_attention_backward(q, k, v, e_idx, e_z, torch.zeros_like(q), e_l,
                                                   torch.zeros_like(q), radius=cfg.R, scale=cfg.scale, q0=5, nq=0)
    torch.cuda.synchronize()
    assert dz.numel() == 0 and not dq.any() and not dk.any() and not dv.any()


def test_backward_tile_order_independence():
    """The pooled query side of the backward gives the same bits when its blocks walk the
    (KV group, query block) tiles in reversed order."""
    cfg = get_config("prefill_16k", N=40, Hq=8, Hkv=2, K=6, R=64)
    print("[case] backward tile order independence", flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, 0, cfg.T)
    idx, zsel = selection(cfg, dr, 0, cfg.T)
    a = run_gpu(cfg, inp, dr["dO"], idx, zsel, 0, cfg.T)
    lcr.set_tile_order(True)
    try:
        b = run_gpu(cfg, inp, dr["dO"], idx, zsel, 0, cfg.T)
    finally:
        lcr.set_tile_order(False)
    for x, y, n in zip(a, b, ("dq", "dk", "dv", "dzsel")):
        assert np.array_equal(x, y), f"{n} differs with the tiles in reversed order"


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_16k"])
def test_chunk_summary_backward(name):
    """Pooling backward: mask-slot rows of dq written, content rows of dk accumulated
    onto what is there (here a seeded non-zero start), against the oracle."""
    cfg = get_config(name)
    print(f"[case] chunk_summary_backward {name}", flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, 0, 1)
    q, k = to_dev(inp["q"]), to_dev(inp["k"])
    dk0 = np.random.default_rng(3).standard_normal(inp["k"].shape).astype(np.float32)
    dq, dk = lcr.chunk_summary_backward(q, k, to_dev(dr["ds"]), to_dev(dr["dH"]), scale=cfg.scale,
                                        dk=torch.from_numpy(dk0).cuda())
    torch.cuda.synchronize()
    f_q, f_k = as_f64(inp["q"]), as_f64(inp["k"])
    qm = f_q.reshape(cfg.B, cfg.Hq, cfg.N, SL, cfg.d)[:, :, :, SL - 1]
    rq, rk = OB.chunk_summary_backward(qm, f_k, cfg.scale, dr["ds"].astype(np.float64),
                                       dr["dH"].astype(np.float64))
    gq = f64(dq).reshape(cfg.B, cfg.Hq, cfg.N, SL, cfg.d)
    e_q = rel_err(gq[:, :, :, SL - 1], rq)
    e_k = rel_err(f64(dk) - dk0, rk)
    print(f"    dq={e_q:.2e} dk={e_k:.2e}", flush=True)
    assert e_q < 1e-5 and e_k < 1e-5
    assert not gq[:, :, :, :SL - 1].any(), "content rows of dq are not written"
    assert np.array_equal(f64(dk).reshape(cfg.B, cfg.Hkv, cfg.N, SL, cfg.d)[:, :, :, SL - 1],
                          dk0.reshape(cfg.B, cfg.Hkv, cfg.N, SL, cfg.d)[:, :, :, SL - 1]), "mask rows of dk untouched"


SCORE_CASES = {
    "tiny_fp32": ("tiny_fp32", {}, 0, None),
    "bf16 G7 ragged range": ("prefill_16k", dict(N=12, Hq=14, Hkv=2, d=64, r=16, D=96, K=3, R=20, beta=0.4), 50, 333),
    "bf16 B2 rank 128 entropy": ("prefill_32k_entropy", dict(N=10, Hq=8, Hkv=2, r=128, D=160, K=4, R=30), 0, None),
    "prefill_16k": ("prefill_16k", {}, 0, None),
}


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(SCORE_CASES))
def test_route_score_backward(name):
    """Scoring backward against the oracle: dq accumulated onto a seeded start at the
    queried rows only, dx at the queried rows, dA, dBm, ds, dH in full."""
    base, over, q0, nq = SCORE_CASES[name]
    cfg = get_config(base, **over)
    nq = cfg.T - q0 if nq is None else nq
    print(f"[case] route_score_backward {name}: B={cfg.B} N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} r={cfg.r} "
          f"D={cfg.D} K={cfg.K} beta={cfg.beta} q0={q0} nq={nq} dtype={cfg.dtype}", flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, q0, nq)
    idx, zsel = selection(cfg, dr, q0, nq)
    dz = np.where(np.isfinite(zsel), dr["zsel"], 0.0).astype(np.float32)
    s_ref, _ = O.chunk_summary(as_f64(inp["q"]), as_f64(inp["k"]), cfg.scale)
    s32 = s_ref.astype(np.float32)
    dq0 = np.random.default_rng(11).standard_normal(inp["q"].shape).astype(np.float32)
    out = lcr.route_score_backward(to_dev(inp["q"]), to_dev(inp["x"]), to_dev(inp["A"]), to_dev(inp["Bm"]),
                                   torch.from_numpy(s32).cuda(), torch.from_numpy(idx.astype(np.int32)).cuda(),
                                   torch.from_numpy(dz).cuda(), beta=cfg.beta, scale=cfg.scale, q0=q0, nq=nq,
                                   dq=torch.from_numpy(dq0).cuda())
    torch.cuda.synchronize()
    queries = np.arange(q0, q0 + nq)
    sl = O.slot_of(queries)
    rq, rx, rA, rB, rs, rH = OB.route_score_backward(as_f64(inp["q"])[:, :, sl], as_f64(inp["x"])[:, sl],
                                                     as_f64(inp["A"]), as_f64(inp["Bm"]), s32.astype(np.float64),
                                                     None, idx, dz.astype(np.float64), cfg.beta, cfg.scale)
    gq = f64(out["dq"])
    gx = f64(out["dx"])
    errs = dict(dq=rel_err(gq[:, :, sl] - dq0[:, :, sl], rq), dx=rel_err(gx[:, sl], rx), dA=rel_err(f64(out["dA"]), rA),
                dBm=rel_err(f64(out["dBm"]), rB), ds=rel_err(f64(out["ds"]), rs), dH=rel_err(f64(out["dH"]), rH))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e < 1e-4, f"{name}: {n} error {e:.3e}"
    other = np.setdiff1d(np.arange(cfg.L), sl)
    assert np.array_equal(gq[:, :, other], dq0[:, :, other]), "dq rows outside the queried set are untouched"
    assert not gx[:, other].any(), "dx rows outside the queried set stay zero"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_route_layer_backward_end_to_end(dtype):
    """The three backward calls chained (attention, scoring, pooling) give the whole
    layer's gradients with the oracle's selection held fixed: within the bf16
    tolerance for bf16 inputs, within 1e-5 for float32 inputs (every call then
    computes in float32)."""
    cfg = get_config("prefill_16k", N=10, Hq=8, Hkv=2, d=128, r=16, D=96, K=3, R=30, beta=0.3, dtype=dtype)
    print(f"[case] route layer backward end to end, {dtype}", flush=True)
    inp = route_inputs(cfg)
    f = {n: as_f64(inp[n]) for n in ("q", "k", "v", "x", "A", "Bm")}
    queries = np.arange(cfg.T)
    ref = O.route_layer(f["q"], f["k"], f["v"], f["x"], f["A"], f["Bm"], K=cfg.K, R=cfg.R, beta=cfg.beta,
                        scale=cfg.scale, queries=queries)
    dr = backward_draws(cfg, 0, cfg.T)
    dO_rows = as_f64(dr["dO"])[:, :, O.slot_of(queries)]
    want = OB.route_layer_backward(f["q"], f["k"], f["v"], f["x"], f["A"], f["Bm"], ref["idx"], dO_rows, R=cfg.R,
                                   beta=cfg.beta, scale=cfg.scale, queries=queries)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "x", "A", "Bm")}
    res = lcr.route_layer(d["q"], d["k"], d["v"], d["x"], d["A"], d["Bm"], K=cfg.K, radius=cfg.R, beta=cfg.beta,
                          scale=cfg.scale, want_lse=True)
    idx_t = torch.from_numpy(ref["idx"].astype(np.int32)).cuda()     # the oracle's selection, as in `want`
    zsel = torch.from_numpy(ref["zsel"].astype(np.float32)).cuda()
    o, lse = lcr.routed_attention(d["q"], d["k"], d["v"], idx_t, zsel, radius=cfg.R, scale=cfg.scale, want_lse=True)
    dq, dk, dv, dz = lcr.routed_attention_backward(d["q"], d["k"], d["v"], idx_t, zsel, o, lse, to_dev(dr["dO"]),
                                                   radius=cfg.R, scale=cfg.scale)
    sc = lcr.route_score_backward(d["q"], d["x"], d["A"], d["Bm"], res["s"], idx_t, dz, beta=cfg.beta,
                                  scale=cfg.scale, dq=dq)
    lcr.chunk_summary_backward(d["q"], d["k"], sc["ds"], sc["dH"], scale=cfg.scale, dq=dq, dk=dk)
    torch.cuda.synchronize()
    errs = dict(dq=rel_err(f64(dq), want["dq"]), dk=rel_err(f64(dk), want["dk"]), dv=rel_err(f64(dv), want["dv"]),
                dx=rel_err(f64(sc["dx"]), want["dx"]), dA=rel_err(f64(sc["dA"]), want["dA"]),
                dBm=rel_err(f64(sc["dBm"]), want["dBm"]))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    tol = BWD_TOL if dtype == "bf16" else 1e-5
    for n, e in errs.items():
        assert e < tol, f"{n} error {e:.3e}"


@pytest.mark.timeout(300)
def test_backward_decode_128k_tail():
    """The 128K decode shape (2,048 chunks, 32 tail queries): the chunk pool does not fit in
    LDS at this N, so the query side takes the per-wave chunk walk."""
    cfg = get_config("decode_128k")
    q0, nq = cfg.T - 32, 32
    print(f"[case] backward decode_128k tail: N={cfg.N} Hq={cfg.Hq} Hkv={cfg.Hkv} K={cfg.K} q0={q0} nq={nq}",
          flush=True)
    inp = route_inputs(cfg)
    dr = backward_draws(cfg, q0, nq)
    idx, zsel = selection(cfg, dr, q0, nq)
    gq, gk, gv, gz = run_gpu(cfg, inp, dr["dO"], idx, zsel, q0, nq)
    queries = np.arange(q0, q0 + nq)
    sl = O.slot_of(queries)
    rq, rk, rv, rz = OB.routed_attention_backward(as_f64(inp["q"][:, :, sl]), as_f64(inp["k"]), as_f64(inp["v"]),
                                                  idx, zsel.astype(np.float64), cfg.R, cfg.scale, queries,
                                                  as_f64(dr["dO"][:, :, sl]))
    errs = dict(dq=rel_err(gq[:, :, sl], rq), dk=rel_err(gk, rk), dv=rel_err(gv, rv),
                dzsel=rel_err(np.where(np.isfinite(zsel), gz, 0.0), rz))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e < BWD_TOL, f"{n} error {e:.3e}"


@pytest.mark.timeout(300)
def test_route_layer_backward_binding_entropy_32k_sampled():
    """route_layer_backward (the three calls chained) on the 32K entropy workload (batch 2,
    beta = 0.5, shared per-chunk key offsets). Inputs of the backward that the forward would
    provide come from the oracle (summaries; a selection ranked by the oracle over seeded
    scores; seeded chunk logits); o and lse come from the GPU forward on those inputs and are
    used on the GPU side only. Checked on sampled query blocks: dzsel, and the dq rows
    (attention part plus scoring part, the oracle's per-row sums)."""
    cfg = get_config("prefill_32k_entropy")
    print(f"[case] route_layer_backward prefill_32k_entropy: B={cfg.B} N={cfg.N} beta={cfg.beta}", flush=True)
    inp = route_inputs(cfg)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "x", "A", "Bm")}
    s_ref, _ = O.chunk_summary(as_f64(inp["q"]), as_f64(inp["k"]), cfg.scale)
    s32 = s_ref.astype(np.float32)
    dr = backward_draws(cfg, 0, cfg.T)
    idx, zsel = selection(cfg, dr, 0, cfg.T)
    idx_t = torch.from_numpy(idx.astype(np.int32)).cuda()
    z_t = torch.from_numpy(np.ascontiguousarray(zsel)).cuda()
    o, lse = lcr.routed_attention(d["q"], d["k"], d["v"], idx_t, z_t, radius=cfg.R, scale=cfg.scale, want_lse=True)
    fwd = dict(s=torch.from_numpy(s32).cuda(), idx=idx_t, zsel=z_t, o=o, lse=lse)
    g = lcr.route_layer_backward(d["q"], d["k"], d["v"], d["x"], d["A"], d["Bm"], fwd, to_dev(dr["dO"]),
                                 radius=cfg.R, beta=cfg.beta, scale=cfg.scale)
    torch.cuda.synchronize()
    queries = sample_query_blocks(cfg.T, n_blocks=3, block=16, seed=9)
    sl = O.slot_of(queries)
    qrows = as_f64(inp["q"][:, :, sl])
    rq_a, _, _, rz = OB.routed_attention_backward(qrows, as_f64(inp["k"]), as_f64(inp["v"]), idx[:, :, queries],
                                                  zsel[:, :, queries].astype(np.float64), cfg.R, cfg.scale,
                                                  queries, as_f64(dr["dO"][:, :, sl]))
    rq_s = OB.route_score_backward(qrows, as_f64(inp["x"][:, sl]), as_f64(inp["A"]), as_f64(inp["Bm"]),
                                   s32.astype(np.float64), None, idx[:, :, queries], rz, cfg.beta, cfg.scale)[0]
    fin = np.isfinite(zsel[:, :, queries])
    errs = dict(dzsel=rel_err(np.where(fin, f64(g["dzsel"])[:, :, queries], 0.0), rz),
                dq=rel_err(f64(g["dq"])[:, :, sl], rq_a + rq_s))
    print("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e < BWD_TOL, f"{n} error {e:.3e}"
