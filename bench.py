"""Benchmark of the route-layer hot path on one MI355X.

A step is one route layer over the 16K-prefill workload (1 x 256 chunks x 64
slots, 28 query / 4 KV heads, d = 128, rank-64 residual from hidden 3584,
K = 32, window radius 256, beta = 0; bf16 inputs ~ N(0,1), residual factors ~
N(0, 0.02)): chunk summaries, routing query + scores + GQA max + top-K, routed
attention, with every input resident in HBM before timing starts.

Printed JSON line (one, rank 0):
  value        content queries per second over the timed steps
  roofline     the dominant kernel's algorithmic rate against its roofline,
               timed live with HIP events on the stream it runs on
  cpu_baseline the fp64 oracle on a bounded sample of the same workload,
               extrapolated to the whole layer
  decode_128k  ms per decode step (32 tail queries, 2048 chunks), HBM roofline;
               summary_ms: a whole summary pass against the refresh of the one
               chunk whose keys a decode step rewrites
  swa_64k      ms per sliding-window layer (65,536 slots, radius 1280)
  dense_16k    ms per dense bidirectional attention layer (16,384 slots, every
               slot attends to every slot: the sliding window with R >= L);
               dense_64k and dense_128k the same at 65,536 and 131,072 slots
  prefill_32k_entropy  ms per 32K route layer with the entropy term (batch 2, beta 0.5)
  prefill_128k ms per 128K prefill route layer (2,048 chunks), with the scoring call and the
               routed attention timed on their own
  stack_64k    ms per 28-layer attention forward at 64K (7 route layers, 21 SWA layers)
  backward_16k ms of the route layer's backward on the 16K-prefill workload:
               attention (dq, dk, dv, dzsel, with its MFMA roofline), scoring
               (dq, dx, dA, dBm, ds, dH) and pooling (dq mask rows, dk)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--no-decode] [--no-swa] [--only {prefill,decode,swa,dense,backward,entropy,prefill128k,stack,copy}]
(--only copy runs a plain 1 GiB device copy, used to calibrate byte counters.)
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-attn ms/decode step at 128K & prefill queries/s; % HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "learned_chunk_routed_amd", "csrc", "attention.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def stored_traffic(kernel_tag, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel source (the summary records the source hash)."""
    path = os.path.join(PROFILE_DIR, f"{kernel_tag}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source sha256\[:16\]: `([0-9a-f]+)`", text)
    m_bytes = re.search(r"hbm bytes per launch: `([0-9.eE+]+)`", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash(KERNEL_SRC):
        return None
    return float(m_bytes.group(1))


# ----------------------------------------------------------------------------- algorithmic work

def prefill_flops(cfg, idx_counts):
    """Dense-contraction flops of the routed attention (window + chosen chunks):
    4*d per (head, query, window key) and 4*d*63 per (head, query, chosen chunk)."""
    i = np.arange(cfg.T)
    win = np.minimum(cfg.T - 1, i + cfg.R) - np.maximum(0, i - cfg.R) + 1
    local = 4.0 * cfg.d * cfg.Hq * cfg.B * float(win.sum())
    chunks = 4.0 * cfg.d * 63 * cfg.G * float(idx_counts)
    return local, chunks


def decode_bytes(cfg, idx_np):
    """Unique bytes the decode step must touch: all summaries and entropies, the union
    of chosen chunks' content K/V per KV group, the tail window's K/V, q/x rows, residual
    factors, outputs and selections."""
    d, N, Hq, Hkv = cfg.d, cfg.N, cfg.Hq, cfg.Hkv
    summ = Hq * N * d * 4 + Hq * N * 4
    union = sum(len(np.unique(idx_np[0, g][idx_np[0, g] >= 0])) for g in range(Hkv))
    chunks = union * 63 * d * 2 * 2
    lo = max(0, cfg.q0 - cfg.R)
    hi = cfg.T - 1
    window = Hkv * (hi - lo + 1) * d * 2 * 2
    small = cfg.nq * (Hq * d * 2 + cfg.D * 2) + cfg.D * cfg.r * 2 + cfg.r * Hq * d * 2 \
        + cfg.nq * Hq * d * 2 + cfg.nq * Hkv * cfg.K * 4 + cfg.nq * Hq * cfg.K * 4
    return summ + chunks + window + small, union


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(cfg, inp, n_sample=1024):
    """The oracle as it stands on a bounded sample: the summaries of every chunk (a
    fixed cost of the layer) plus routing and attention for n_sample consecutive
    queries; extrapolated to all T queries."""
    from threadpoolctl import threadpool_info
    from lcr_inputs import as_f64
    from oracle import route as O

    t0 = time.perf_counter()
    f = {k: as_f64(v) for k, v in inp.items()}
    t_conv = time.perf_counter() - t0
    B, Hq, L, d = f["q"].shape
    N = L // 64
    t0 = time.perf_counter()
    q_mask = f["q"].reshape(B, Hq, N, 64, d)[:, :, :, 63, :]
    s, H = O.chunk_summary_from_mask(q_mask, f["k"], cfg.scale)
    t_sum = time.perf_counter() - t0
    queries = np.arange(cfg.T // 2, cfg.T // 2 + n_sample)
    sl = O.slot_of(queries)
    t0 = time.perf_counter()
    qt = O.routing_query(f["q"][:, :, sl], f["x"][:, sl], f["A"], f["Bm"])
    z = O.route_scores(qt, s, H, cfg.beta, cfg.scale)
    zhat = O.group_max(z, cfg.G)
    cand = O.candidate_mask(queries, cfg.R, cfg.N)
    idx, _ = O.select_topk(zhat, cand, cfg.K)
    zsel = O.gather_zsel(z, idx, cfg.G)
    O.routed_attention(f["q"][:, :, sl], f["k"], f["v"], idx, zsel, cfg.R, cfg.scale, queries)
    t_q = time.perf_counter() - t0
    t_full = t_sum + t_q * cfg.T / n_sample
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": round(cfg.T * cfg.B / t_full, 3),
        "unit": "queries/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"summaries of all {N} chunks x {Hq} heads ({t_sum:.2f} s) + routing and attention for "
                   f"{n_sample} consecutive queries ({t_q:.2f} s), extrapolated x{cfg.T / n_sample:.0f}; "
                   f"input upcast {t_conv:.2f} s not counted"),
    }


# ----------------------------------------------------------------------------- GPU timings

def bench_prefill(args, torch, lcr):
    from lcr_inputs import get_config, route_inputs
    cfg = get_config("prefill_16k")
    log(f"[bench] prefill_16k: generating inputs")
    inp = route_inputs(cfg)
    d = {k: to_dev(v, torch) for k, v in inp.items()}
    B, Hq, Hkv, N, dd = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    dev = "cuda"
    s = torch.empty((B, Hq, N, dd), dtype=torch.float32, device=dev)
    H = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, cfg.T, cfg.K), dtype=torch.int32, device=dev)
    zsel = torch.empty((B, Hq, cfg.T, cfg.K), dtype=torch.float32, device=dev)
    out = torch.zeros_like(d["q"])
    dims = lcr.make_dims(B, Hq, Hkv, N, dd, torch.bfloat16)
    ws_score = torch.empty(max(1, lcr.workspace_bytes(1, dims, cfg.D, cfg.r, cfg.K, cfg.T)), dtype=torch.uint8,
                           device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(times=None):
        if times is not None:
            ev[0].record()
        lcr.chunk_summary(d["q"], d["k"], cfg.scale, s=s, H=H)
        if times is not None:
            ev[1].record()
        lcr.route_score_topk(d["q"], d["x"], d["A"], d["Bm"], s, H, Hkv=Hkv, K=cfg.K, radius=cfg.R,
                             beta=cfg.beta, scale=cfg.scale, idx=idx, zsel=zsel, ws=ws_score)
        if times is not None:
            ev[2].record()
        lcr.routed_attention(d["q"], d["k"], d["v"], idx, zsel, radius=cfg.R, scale=cfg.scale, out=out)
        if times is not None:
            ev[3].record()

    log(f"[bench] prefill_16k: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: whole steps, no per-op events (clean wall time)
    log(f"[bench] prefill_16k: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-op durations with HIP events on the launch stream, same number of steps
    per_op = []
    for _ in range(args.steps):
        step(times=True)
        torch.cuda.synchronize()
        per_op.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
    per_op = np.array(per_op)
    med = np.median(per_op, axis=0)
    counts = int((idx >= 0).sum().item())
    local, chunks = prefill_flops(cfg, counts)
    attn_ms = float(per_op[:, 2].mean())
    achieved = (local + chunks) / (attn_ms * 1e-3) / 1e12
    traffic = stored_traffic("routed_attention", "prefill_16k")
    return cfg, inp, {
        "wall_s": wall,
        "ms_per_step": wall / args.steps * 1e3,
        "op_ms_median": {"chunk_summary": round(float(med[0]), 4), "route_score_topk": round(float(med[1]), 4),
                         "routed_attention": round(float(med[2]), 4)},
        "roofline": {"bound": "mfma", "kernel": "routed_prefill_kernel", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_gflop_per_launch": round((local + chunks) / 1e9, 2),
                     "launch_ms_mean": round(attn_ms, 4)},
    }


def bench_decode(args, torch, lcr):
    from lcr_inputs import get_config, decode_cache, decode_step
    cfg = get_config("decode_128k")
    log("[bench] decode_128k: generating cache")
    cache = decode_cache(cfg)
    B, Hq, Hkv, N, dd, L = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.L
    dev = "cuda"
    k, v = to_dev(cache["k"], torch), to_dev(cache["v"], torch)
    q = torch.zeros((B, Hq, L, dd), dtype=torch.bfloat16, device=dev)
    q.view(B, Hq, N, 64, dd)[:, :, :, 63] = to_dev(cache["q_mask"], torch)
    x = torch.zeros((B, L, cfg.D), dtype=torch.bfloat16, device=dev)
    A, Bm = to_dev(cache["A"], torch), to_dev(cache["Bm"], torch)
    i_tail = np.arange(cfg.q0, cfg.T)
    slots = torch.from_numpy((i_tail // 63) * 64 + i_tail % 63).to(dev)
    s, H = lcr.chunk_summary(q, k, cfg.scale)          # once per cache, untimed
    # the summaries a decode loop keeps current: a whole pass against a refresh of the
    # one chunk whose keys a step rewrites (the last one here); and the pass of the
    # mean-summary ablation
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    lcr.chunk_summary(q, k, cfg.scale, s=s, H=H, chunks=(N - 1, 1))
    sm, Hm = lcr.chunk_summary_mean(k, Hq)
    torch.cuda.synchronize()
    sev[0].record()
    for _ in range(5):
        lcr.chunk_summary(q, k, cfg.scale, s=s, H=H)
    sev[1].record()
    for _ in range(20):
        lcr.chunk_summary(q, k, cfg.scale, s=s, H=H, chunks=(N - 1, 1))
    sev[2].record()
    for _ in range(5):
        lcr.chunk_summary_mean(k, Hq, s=sm, H=Hm)
    sev[3].record()
    torch.cuda.synchronize()
    summary_ms = {"whole": round(sev[0].elapsed_time(sev[1]) / 5, 4),
                  "one_chunk_refresh": round(sev[1].elapsed_time(sev[2]) / 20, 4),
                  "mean_whole": round(sev[2].elapsed_time(sev[3]) / 5, 4)}
    steps_in = [decode_step(cfg, j) for j in range(cfg.steps)]
    q_tail = [to_dev(st["q_tail"], torch) for st in steps_in]
    x_tail = [to_dev(st["x_tail"], torch) for st in steps_in]
    idx = torch.empty((B, Hkv, cfg.nq, cfg.K), dtype=torch.int32, device=dev)
    zsel = torch.empty((B, Hq, cfg.nq, cfg.K), dtype=torch.float32, device=dev)
    out = torch.zeros_like(q)
    dims = lcr.make_dims(B, Hq, Hkv, N, dd, torch.bfloat16)
    ws_s = torch.empty(max(1, lcr.workspace_bytes(1, dims, cfg.D, cfg.r, cfg.K, cfg.nq)), dtype=torch.uint8,
                       device=dev)
    ws_a = torch.empty(max(1, lcr.workspace_bytes(2, dims, 0, 0, cfg.K, cfg.nq, cfg.R)), dtype=torch.uint8,
                       device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(j, timed):
        q[:, :, slots] = q_tail[j]
        x[:, slots] = x_tail[j]
        if timed:
            ev0.record()
        lcr.route_score_topk(q, x, A, Bm, s, H, Hkv=Hkv, K=cfg.K, radius=cfg.R, beta=cfg.beta, scale=cfg.scale,
                             q0=cfg.q0, nq=cfg.nq, idx=idx, zsel=zsel, ws=ws_s)
        lcr.routed_attention(q, k, v, idx, zsel, radius=cfg.R, scale=cfg.scale, q0=cfg.q0, nq=cfg.nq, out=out,
                             ws=ws_a)
        if timed:
            ev1.record()

    log("[bench] decode_128k: warmup")
    for j in range(min(5, cfg.steps)):
        run(j, False)
    torch.cuda.synchronize()
    # eager: the two library calls issued from Python each step (host launch cost included)
    eager_ms = []
    for j in range(cfg.steps):
        run(j, True)
        torch.cuda.synchronize()
        eager_ms.append(ev0.elapsed_time(ev1))
    # graph: the same two calls captured once in a HIP graph and replayed per step, as a
    # serving loop runs a decode step; the step's fresh q and x rows are copied in first
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lcr.route_score_topk(q, x, A, Bm, s, H, Hkv=Hkv, K=cfg.K, radius=cfg.R, beta=cfg.beta, scale=cfg.scale,
                             q0=cfg.q0, nq=cfg.nq, idx=idx, zsel=zsel, ws=ws_s)
        lcr.routed_attention(q, k, v, idx, zsel, radius=cfg.R, scale=cfg.scale, q0=cfg.q0, nq=cfg.nq, out=out,
                             ws=ws_a)
    torch.cuda.synchronize()
    log("[bench] decode_128k: graph replays")
    ms, nbytes = [], []
    for j in range(cfg.steps):
        q[:, :, slots] = q_tail[j]
        x[:, slots] = x_tail[j]
        ev0.record()
        graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        ms.append(ev0.elapsed_time(ev1))
        b, _ = decode_bytes(cfg, idx.cpu().numpy())
        nbytes.append(b)
    # cold: the Infinity Cache is scrubbed before each step by writing a 512 MB buffer (untimed)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for j in range(16):
        q[:, :, slots] = q_tail[j]
        x[:, slots] = x_tail[j]
        scrub.fill_(j & 255)
        torch.cuda.synchronize()
        ev0.record()
        graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        cold.append(ev0.elapsed_time(ev1))
    del scrub
    ms, eager_ms = np.array(ms), np.array(eager_ms)
    med = float(np.median(ms))
    gbs = float(np.median(np.array(nbytes))) / (med * 1e-3) / 1e9
    return {"ms_per_step_median": round(med, 4), "ms_min": round(float(ms.min()), 4),
            "ms_max": round(float(ms.max()), 4), "steps": int(cfg.steps),
            "eager_ms_per_step_median": round(float(np.median(eager_ms)), 4),
            "cold_ms_per_step_median": round(float(np.median(np.array(cold))), 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_mb_per_step": round(float(np.median(nbytes)) / 1e6, 2)},
            "summary_ms": summary_ms,
            "note": "route_score_topk + routed_attention per step on cached K/V, replayed from a HIP graph "
                    "(eager_ms_per_step_median: the same calls issued from Python; cold_ms_per_step_median: 16 "
                    "steps each after a 512 MB write that scrubs the Infinity Cache); summaries precomputed"}


def bench_swa(args, torch, lcr):
    from lcr_inputs import get_config, stack_layer_torch
    cfg = get_config("stack_64k")
    t = stack_layer_torch(cfg, 0, "cuda", route=False)
    out = torch.empty_like(t["q"])
    for _ in range(2):
        lcr.swa_attention(t["q"], t["k"], t["v"], radius=cfg.swa_radius, scale=cfg.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 5
    e0.record()
    for _ in range(n):
        lcr.swa_attention(t["q"], t["k"], t["v"], radius=cfg.swa_radius, scale=cfg.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    u = np.arange(cfg.L)
    keys = float((np.minimum(cfg.L - 1, u + cfg.swa_radius) - np.maximum(0, u - cfg.swa_radius) + 1).sum())
    flops = 4.0 * cfg.d * cfg.Hq * keys
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms_per_layer": round(ms, 4), "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                                     "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def bench_dense(args, torch, lcr, L=16384):
    """Dense bidirectional attention over L slots (28 query / 4 KV heads, d = 128,
    bf16 ~ N(0,1), seeded): the swa entry point with a radius covering the sequence."""
    B, Hq, Hkv, d = 1, 28, 4, 128
    g = torch.Generator(device="cuda").manual_seed(L)
    q = torch.randn((B, Hq, L, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    scale = 1.0 / np.sqrt(d)
    for _ in range(2):
        lcr.swa_attention(q, k, v, radius=L, scale=scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 5 if L <= 16384 else 2
    e0.record()
    for _ in range(n):
        lcr.swa_attention(q, k, v, radius=L, scale=scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 4.0 * d * Hq * B * float(L) * float(L)
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms_per_layer": round(ms, 4), "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                                     "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def _route_layer_runner(cfg, d, torch, lcr, bufs=None):
    """Preallocated buffers and one call sequence for a whole route layer (summaries,
    scoring + top-K, routed attention); returns (step, idx, bufs): step(ev) records ev[0]
    before and ev[1] after the routed attention when ev is given. Pass the bufs of an
    earlier runner of the same shape to share them (layers that run one after another)."""
    B, Hq, Hkv, N, dd = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d
    dev = "cuda"
    if bufs is None:
        dims = lcr.make_dims(B, Hq, Hkv, N, dd, torch.bfloat16)
        bufs = dict(
            s=torch.empty((B, Hq, N, dd), dtype=torch.float32, device=dev),
            H=torch.empty((B, Hq, N), dtype=torch.float32, device=dev),
            idx=torch.empty((B, Hkv, cfg.T, cfg.K), dtype=torch.int32, device=dev),
            zsel=torch.empty((B, Hq, cfg.T, cfg.K), dtype=torch.float32, device=dev),
            out=torch.zeros_like(d["q"]),
            ws_s=torch.empty(max(1, lcr.workspace_bytes(1, dims, cfg.D, cfg.r, cfg.K, cfg.T)), dtype=torch.uint8,
                             device=dev),
            ws_a=torch.empty(max(1, lcr.workspace_bytes(2, dims, 0, 0, cfg.K, cfg.T, cfg.R)), dtype=torch.uint8,
                             device=dev))
    b = bufs

    def step(ev=None):
        lcr.chunk_summary(d["q"], d["k"], cfg.scale, s=b["s"], H=b["H"])
        lcr.route_score_topk(d["q"], d["x"], d["A"], d["Bm"], b["s"], b["H"], Hkv=Hkv, K=cfg.K, radius=cfg.R,
                             beta=cfg.beta, scale=cfg.scale, idx=b["idx"], zsel=b["zsel"], ws=b["ws_s"])
        if ev is not None:
            ev[0].record()
        lcr.routed_attention(d["q"], d["k"], d["v"], b["idx"], b["zsel"], radius=cfg.R, scale=cfg.scale,
                             out=b["out"], ws=b["ws_a"])
        if ev is not None:
            ev[1].record()
    return step, b["idx"], bufs


def bench_entropy(args, torch, lcr):
    """The 32K route layer with the entropy term: batch 2, N = 512 chunks, beta = 0.5, keys
    with a shared per-chunk offset N(0, 0.3). Whole layers timed with HIP events (2 warmup,
    5 timed); the routed attention's own launches timed beside them for its roofline."""
    from lcr_inputs import get_config, route_inputs
    cfg = get_config("prefill_32k_entropy")
    log("[bench] prefill_32k_entropy: generating inputs")
    d = {k: to_dev(v, torch) for k, v in route_inputs(cfg).items()}
    step, idx, _ = _route_layer_runner(cfg, d, torch, lcr)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n = 5
    e[0].record()
    for _ in range(n):
        step()
    e[1].record()
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / n
    ra = []
    for _ in range(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        step(ev)
        torch.cuda.synchronize()
        ra.append(ev[0].elapsed_time(ev[1]))
    attn_ms = float(np.mean(ra))
    local, chunks = prefill_flops(cfg, int((idx >= 0).sum().item()))
    tf = (local + chunks) / (attn_ms * 1e-3) / 1e12
    return {"ms_per_layer": round(ms, 4), "queries_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
            "routed_attention_ms": round(attn_ms, 4),
            "roofline": {"bound": "mfma", "kernel": "routed_prefill_kernel", "achieved": round(tf, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def bench_prefill_128k(args, torch, lcr):
    """A 128K prefill route layer: N = 2,048 chunks (131,072 slots, 129,024 content queries),
    28/4 heads, d = 128, rank 64 from hidden 3584, K = 32, window radius 256, beta = 0, inputs
    drawn on the device. Whole layers timed with HIP events (1 warmup, 3 timed), then the
    scoring call and the routed attention timed on their own."""
    from lcr_inputs import get_config, stack_layer_torch
    cfg = get_config("stack_64k", N=2048)
    log("[bench] prefill_128k: generating inputs on the device")
    d = stack_layer_torch(cfg, 0, "cuda", route=True)
    step, idx, b = _route_layer_runner(cfg, d, torch, lcr)
    step()
    torch.cuda.synchronize()
    n = 3
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for _ in range(n):
        step()
    e[1].record()
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / n

    def timed(fn):
        out = []
        for _ in range(n):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            out.append(ev[0].elapsed_time(ev[1]))
        return float(np.mean(out))
    score_ms = timed(lambda: lcr.route_score_topk(d["q"], d["x"], d["A"], d["Bm"], b["s"], b["H"], Hkv=cfg.Hkv,
                                                  K=cfg.K, radius=cfg.R, beta=cfg.beta, scale=cfg.scale,
                                                  idx=b["idx"], zsel=b["zsel"], ws=b["ws_s"]))
    attn_ms = timed(lambda: lcr.routed_attention(d["q"], d["k"], d["v"], b["idx"], b["zsel"], radius=cfg.R,
                                                 scale=cfg.scale, out=b["out"], ws=b["ws_a"]))
    local, chunks = prefill_flops(cfg, int((idx >= 0).sum().item()))
    tf = (local + chunks) / (attn_ms * 1e-3) / 1e12
    del d, b
    return {"ms_per_layer": round(ms, 3), "queries_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
            "route_score_topk_ms": round(score_ms, 3), "routed_attention_ms": round(attn_ms, 3),
            "roofline": {"bound": "mfma", "kernel": "routed_prefill_kernel", "achieved": round(tf, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def bench_stack(args, torch, lcr):
    """The 28-layer attention forward at 64K: route layers at l % 4 == 3 (7 of them), bidirectional
    SWA with radius 1280 over all 65,536 slots in the other 21, each layer with its own inputs
    (drawn on the device beforehand, about 20 GB). One warmup forward, then 2 timed; per-kind
    layer times from HIP events in a further forward."""
    from lcr_inputs import get_config, stack_layer_torch
    cfg = get_config("stack_64k")
    log("[bench] stack_64k: generating 28 layers of inputs on the device")
    layers = [stack_layer_torch(cfg, l, "cuda", route=(l % cfg.route_every == cfg.route_every - 1))
              for l in range(cfg.layers)]
    runners = []
    swa_out = torch.empty_like(layers[0]["q"])
    bufs = None   # the route layers run one after another: one set of buffers and workspaces
    for l, t in enumerate(layers):
        if "x" in t:
            step, idx, bufs = _route_layer_runner(cfg, t, torch, lcr, bufs)
            runners.append(("route", step))
        else:
            runners.append(("swa", t))

    def forward(evs=None):
        for l, (kind, r) in enumerate(runners):
            if evs is not None:
                evs[l][0].record()
            if kind == "route":
                r()
            else:
                lcr.swa_attention(r["q"], r["k"], r["v"], radius=cfg.swa_radius, scale=cfg.scale, out=swa_out)
            if evs is not None:
                evs[l][1].record()
    forward()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for _ in range(2):
        forward()
    e[1].record()
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / 2
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in runners]
    forward(evs)
    torch.cuda.synchronize()
    lm = [ev[0].elapsed_time(ev[1]) for ev in evs]
    route_ms = [m for m, (k, _) in zip(lm, runners) if k == "route"]
    swa_ms = [m for m, (k, _) in zip(lm, runners) if k == "swa"]
    # algorithmic attention flops: routed window + chunks per route layer (the chosen-chunk count of
    # the last route layer, whose selection the shared buffers hold; every row chooses K chunks
    # except at the sequence ends), 4 d per (head, slot, key) for SWA
    lo, ch = prefill_flops(cfg, int((bufs["idx"] >= 0).sum().item()))
    flops = len(route_ms) * (lo + ch)
    u = np.arange(cfg.L)
    keys = float((np.minimum(cfg.L - 1, u + cfg.swa_radius) - np.maximum(0, u - cfg.swa_radius) + 1).sum())
    flops += len(swa_ms) * 4.0 * cfg.d * cfg.Hq * keys
    tf = flops / (ms * 1e-3) / 1e12
    del layers, runners, bufs
    return {"ms_per_forward": round(ms, 3), "route_layer_ms_mean": round(float(np.mean(route_ms)), 3),
            "swa_layer_ms_mean": round(float(np.mean(swa_ms)), 3), "route_layers": len(route_ms),
            "swa_layers": len(swa_ms),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_tflop_per_forward": round(flops / 1e12, 2)}}


def bench_backward(args, torch, lcr):
    """Backward of the route layer over the 16K-prefill workload: the forward's own
    selection, chunk logits, summaries, output and log-normaliser (computed once,
    untimed) and a seeded N(0,1) bf16 upstream gradient. Times the attention backward
    (dq, dk, dv, dzsel), the scoring backward (dq, dx, dA, dBm, ds, dH) and the pooling
    backward (dq at the mask rows, dk) separately, each averaged over 5 calls."""
    from lcr_inputs import get_config, route_inputs
    cfg = get_config("prefill_16k")
    inp = route_inputs(cfg)
    d = {k: to_dev(v, torch) for k, v in inp.items()}
    res = lcr.route_layer(d["q"], d["k"], d["v"], d["x"], d["A"], d["Bm"], K=cfg.K, radius=cfg.R, beta=cfg.beta,
                          scale=cfg.scale, want_lse=True)
    g = torch.Generator(device="cuda").manual_seed(7)
    dO = torch.randn(d["q"].shape, generator=g, device="cuda").to(torch.bfloat16)
    dims = lcr.make_dims(cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, torch.bfloat16)
    ws_a = torch.empty(lcr.workspace_bytes(4, dims, 0, 0, cfg.K, cfg.T, cfg.R), dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(lcr.workspace_bytes(5, dims, cfg.D, cfg.r, cfg.K, cfg.T, 0), dtype=torch.uint8, device="cuda")
    st = {}

    def attn():
        st["a"] = lcr.routed_attention_backward(d["q"], d["k"], d["v"], res["idx"], res["zsel"], res["o"],
                                                res["lse"], dO, radius=cfg.R, scale=cfg.scale, ws=ws_a)

    def score():
        st["s"] = lcr.route_score_backward(d["q"], d["x"], d["A"], d["Bm"], res["s"], res["idx"], st["a"][3],
                                           beta=cfg.beta, scale=cfg.scale, dq=st["a"][0], ws=ws_s)

    def pool():
        lcr.chunk_summary_backward(d["q"], d["k"], st["s"]["ds"], st["s"]["dH"], scale=cfg.scale, dq=st["a"][0],
                                   dk=st["a"][1])

    ms = {}
    for name, fn in (("attention", attn), ("scoring", score), ("pooling", pool)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / 5
    local, chunks = prefill_flops(cfg, int((res["idx"] >= 0).sum().item()))
    # per (head, query, key): S, dP and dQ on the query side (6d), S, dP, dV and dK on the key side (8d)
    flops = (local + chunks) * 14.0 / 4.0
    tf = flops / (ms["attention"] * 1e-3) / 1e12
    return {"ms_attention": round(ms["attention"], 4), "ms_scoring": round(ms["scoring"], 4),
            "ms_pooling": round(ms["pooling"], 4), "ms_layer": round(sum(ms.values()), 4),
            "attention_algorithmic_gflop": round(flops / 1e9, 1),
            "roofline": {"bound": "mfma", "kernels": "attention backward call", "achieved": round(tf, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-swa", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "swa", "dense", "backward", "entropy", "prefill128k",
                                       "stack", "copy"],
                    default=None)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the route layer runs on a single MI355X here; "
              "multi-GPU sharding is described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import learned_chunk_routed_amd as lcr
    lcr.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.only == "decode":
        print(json.dumps({"decode_128k": bench_decode(args, torch, lcr)}), flush=True)
        return
    if args.only == "swa":
        print(json.dumps({"swa_64k": bench_swa(args, torch, lcr)}), flush=True)
        return
    if args.only == "dense":
        print(json.dumps({f"dense_{L // 1024}k": bench_dense(args, torch, lcr, L) for L in (16384, 65536, 131072)}),
              flush=True)
        return
    if args.only == "entropy":
        print(json.dumps({"prefill_32k_entropy": bench_entropy(args, torch, lcr)}), flush=True)
        return
    if args.only == "prefill128k":
        print(json.dumps({"prefill_128k": bench_prefill_128k(args, torch, lcr)}), flush=True)
        return
    if args.only == "stack":
        print(json.dumps({"stack_64k": bench_stack(args, torch, lcr)}), flush=True)
        return
    if args.only == "backward":
        print(json.dumps({"backward_16k": bench_backward(args, torch, lcr)}), flush=True)
        return
    if args.only == "copy":
        # Plain device copy of a known size: calibrates the HBM byte counters.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return

    cfg, inp, pre = bench_prefill(args, torch, lcr)
    value = cfg.T * cfg.B * args.steps / pre["wall_s"]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V/x, residual factors N(0,0.02))",
        "config": {"workload": "prefill_16k route layer: B=1, N=256 chunks x 64 slots (16,128 content "
                               "queries), Hq=28, Hkv=4, d=128, r=64, D=3584, K=32, R=256, beta=0",
                   "global_batch": cfg.B, "seq_len": cfg.L, "parallelism": "single GPU"},
        "op_ms_median": pre["op_ms_median"],
        "roofline": pre["roofline"],
    }
    if args.only is None and not args.no_decode:
        line["decode_128k"] = bench_decode(args, torch, lcr)
    if args.only is None and not args.no_swa:
        line["swa_64k"] = bench_swa(args, torch, lcr)
        for L in (16384, 65536, 131072):
            line[f"dense_{L // 1024}k"] = bench_dense(args, torch, lcr, L)
    if args.only is None:
        line["backward_16k"] = bench_backward(args, torch, lcr)
        line["prefill_32k_entropy"] = bench_entropy(args, torch, lcr)
        line["prefill_128k"] = bench_prefill_128k(args, torch, lcr)
        line["stack_64k"] = bench_stack(args, torch, lcr)
    if args.only is None and not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
