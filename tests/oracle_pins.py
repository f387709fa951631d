"""Pins for the fp64 oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees. They
are run by test_oracle_pins.py and, with mistakes planted in the oracle, by
test_oracle_mutations.py (every planted mistake must make at least one pin fail).

Kinds of pin used here: closed forms (uniform pooling, identical keys, ideal
chunk logits), invariants (convexity, translation, permutation of remote
chunks, mask-slot independence, constant entropy shift), brute force over all
K-subsets and over explicit index sets, and library routines (torch's
scaled_dot_product_attention in float64 with explicit boolean masks).

All oracle calls go through the module object ``O`` so that planted mistakes
are seen.
"""
import itertools
import math

import numpy as np
import torch

from oracle import route as O
from oracle import backward as OB

SL, CT = 64, 63


# ----------------------------------------------------------------------------- helpers

def rng(seed):
    return np.random.default_rng([20251, seed])


def case(seed=0, B=1, N=10, Hq=4, Hkv=2, d=16, r=4, D=24, K=3, R=20, beta=0.3):
    g = rng(seed)
    L = N * SL
    c = dict(B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, r=r, D=D, K=K, R=R, beta=beta, L=L, T=N * CT,
             G=Hq // Hkv, scale=1.0 / math.sqrt(d))
    c["q"] = g.standard_normal((B, Hq, L, d))
    c["k"] = g.standard_normal((B, Hkv, L, d))
    c["v"] = g.standard_normal((B, Hkv, L, d))
    c["x"] = g.standard_normal((B, L, D))
    c["A"] = 0.2 * g.standard_normal((D, r))
    c["Bm"] = 0.2 * g.standard_normal((r, Hq * d))
    return c


def run_layer(c, queries, **over):
    kw = dict(K=c["K"], R=c["R"], beta=c["beta"], scale=c["scale"], queries=queries)
    kw.update(over)
    return O.route_layer(c["q"], c["k"], c["v"], c["x"], c["A"], c["Bm"], **kw)


def sdpa(q, k, v, mask, scale):
    """torch reference attention in float64; q [M,d], k,v [n,d], mask bool [M,n]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    return o[0, 0].numpy()


def content_slots(T):
    i = np.arange(T)
    return (i // CT) * SL + i % CT


def close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------- pooling (step 1)

def pin_pooling_convex_and_entropy_bounds():
    c = case(1)
    s, H = O.chunk_summary(c["q"], c["k"], c["scale"])
    kc = c["k"].reshape(c["B"], c["Hkv"], c["N"], SL, c["d"])[:, :, :, :CT]
    kc = np.repeat(kc, c["G"], axis=1)
    assert np.all(s >= kc.min(axis=3) - 1e-12) and np.all(s <= kc.max(axis=3) + 1e-12), \
        "summary outside the convex hull of its chunk's content keys"
    assert np.all(H >= -1e-12) and np.all(H <= math.log(CT) + 1e-12), "entropy outside [0, ln 63]"


def pin_pooling_uniform_when_mask_query_is_zero():
    c = case(2)
    q = c["q"].copy()
    q.reshape(c["B"], c["Hq"], c["N"], SL, c["d"])[:, :, :, SL - 1] = 0.0
    s, H = O.chunk_summary(q, c["k"], c["scale"])
    kc = c["k"].reshape(c["B"], c["Hkv"], c["N"], SL, c["d"])[:, :, :, :CT]
    close(s, np.repeat(kc.mean(axis=3), c["G"], axis=1), 1e-12, "mean summary")
    close(H, np.full_like(H, math.log(CT)), 1e-12, "uniform entropy ln 63")


def pin_mean_summary_is_pooling_with_zero_mask_queries():
    """The mean-summary ablation equals mask-query pooling with every mask query zero
    (the softmax of equal logits is uniform): two independent routes to one result."""
    c = case(21, Hq=6, Hkv=2)
    q = c["q"].copy()
    q.reshape(c["B"], c["Hq"], c["N"], SL, c["d"])[:, :, :, SL - 1] = 0.0
    s_pool, H_pool = O.chunk_summary(q, c["k"], c["scale"])
    s_mean, H_mean = O.chunk_summary_mean(c["k"], c["Hq"])
    close(s_mean, s_pool, 1e-12, "mean summary against uniform pooling")
    close(H_mean, H_pool, 1e-12, "entropy of uniform pooling")
    kc = c["k"].reshape(c["B"], c["Hkv"], c["N"], SL, c["d"])
    assert not np.allclose(s_mean[:, 0], kc[:, 0, :, SL - 1]), "the mask slot's key is not averaged"


def pin_pooling_concentrates_on_aligned_key():
    """Mask query = lambda * k_j* with a wide logit gap => the pooling is one-hot on j*."""
    c = case(3, d=32)
    B, Hq, Hkv, N, d, G = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["G"]
    q = c["q"].copy()
    qv = q.reshape(B, Hq, N, SL, d)
    kc = c["k"].reshape(B, Hkv, N, SL, d)[:, :, :, :CT]
    want = np.empty((B, Hq, N, d))
    for h in range(Hq):
        for n in range(N):
            kk = kc[0, h // G, n]
            gram = kk @ kk.T
            offmax = np.max(np.where(np.eye(CT, dtype=bool), -np.inf, gram), axis=1)
            gaps = np.diag(gram) - offmax
            jstar = int(np.argmax(gaps))
            assert gaps[jstar] > 0
            qv[0, h, n, SL - 1] = (80.0 / (c["scale"] * gaps[jstar])) * kk[jstar]
            want[0, h, n] = kk[jstar]
    s, H = O.chunk_summary(q, c["k"], c["scale"])
    close(s, want, 1e-9, "summary of a sharply aligned mask query")
    assert np.all(H < 1e-9), "entropy of a one-hot pooling"


def pin_pooling_is_per_query_head():
    """Heads of one KV group pool with their own mask queries: a zero mask query gives the
    mean key while its group neighbour, aligned sharply with key j*, gets k_j*."""
    c = case(31, d=32, Hq=4, Hkv=2)
    B, Hq, Hkv, N, d, G = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["G"]
    q = c["q"].copy()
    qv = q.reshape(B, Hq, N, SL, d)
    kc = c["k"].reshape(B, Hkv, N, SL, d)[:, :, :, :CT]
    for g in range(Hkv):
        for n in range(N):
            kk = kc[0, g, n]
            gram = kk @ kk.T
            gaps = np.diag(gram) - np.max(np.where(np.eye(CT, dtype=bool), -np.inf, gram), axis=1)
            j = int(np.argmax(gaps))
            qv[0, g * G, n, SL - 1] = (80.0 / (c["scale"] * gaps[j])) * kk[j]
            qv[0, g * G + 1, n, SL - 1] = 0.0
    s, H = O.chunk_summary(q, c["k"], c["scale"])
    for g in range(Hkv):
        close(s[0, g * G + 1], kc[0, g].mean(axis=1), 1e-12, "zero mask query pools uniformly")
        close(H[0, g * G + 1], np.full(N, math.log(CT)), 1e-12, "uniform entropy")
        assert np.all(H[0, g * G] < 1e-9), "aligned head pools one key"


def pin_pooling_translation():
    c = case(4)
    s0, H0 = O.chunk_summary(c["q"], c["k"], c["scale"])
    k = c["k"].copy()
    w = rng(44).standard_normal(c["d"])
    cc = 3
    k[:, :, cc * SL: cc * SL + CT] += w          # content keys of chunk 3 only
    s1, H1 = O.chunk_summary(c["q"], k, c["scale"])
    close(s1[:, :, cc], s0[:, :, cc] + w, 1e-12, "translated summary")
    close(H1, H0, 1e-12, "entropy under translation")
    other = [n for n in range(c["N"]) if n != cc]
    close(s1[:, :, other], s0[:, :, other], 0.0, "other chunks untouched")


def pin_mask_slot_keys_are_not_keys():
    c = case(5)
    queries = np.arange(0, c["T"], 5)
    r0 = run_layer(c, queries)
    c2 = dict(c)
    k, v = c["k"].copy(), c["v"].copy()
    ms = np.arange(c["N"]) * SL + SL - 1
    k[:, :, ms] += 7.0 * rng(55).standard_normal(k[:, :, ms].shape)
    v[:, :, ms] += 7.0 * rng(56).standard_normal(v[:, :, ms].shape)
    c2["k"], c2["v"] = k, v
    r1 = run_layer(c2, queries)
    close(r1["s"], r0["s"], 1e-12, "summaries ignore mask-slot keys")
    close(r1["o"], r0["o"], 1e-12, "route output ignores mask-slot keys/values")


# ----------------------------------------------------------------------------- residual (step 2)

def pin_residual_zero_factor():
    c = case(6)
    sl = content_slots(c["T"])[:50]
    qt = O.routing_query(c["q"][:, :, sl], c["x"][:, sl], np.zeros_like(c["A"]), c["Bm"])
    close(qt, c["q"][:, :, sl], 0.0, "A = 0 gives the plain query")
    qt = O.routing_query(c["q"][:, :, sl], c["x"][:, sl], c["A"], np.zeros_like(c["Bm"]))
    close(qt, c["q"][:, :, sl], 0.0, "B = 0 gives the plain query")


def pin_residual_rank_and_loops():
    c = case(7, r=3)
    sl = content_slots(c["T"])[:200]
    qr = c["q"][:, :, sl]
    qt = O.routing_query(qr, c["x"][:, sl], c["A"], c["Bm"])
    res = (qt - qr)[0].transpose(1, 0, 2).reshape(len(sl), -1)     # [n, Hq*d]
    sv = np.linalg.svd(res, compute_uv=False)
    assert sv[c["r"]] < 1e-10 * sv[0], "residual has rank above r"
    # explicit loops on a few entries: head h, dim e of query t
    for (t, h, e) in [(0, 0, 0), (17, 3, 5), (199, 1, 15), (50, 2, 9)]:
        acc = 0.0
        for j in range(c["r"]):
            xa = sum(c["x"][0, sl[t], m] * c["A"][m, j] for m in range(c["D"]))
            acc += xa * c["Bm"][j, h * c["d"] + e]
        close(qt[0, h, t, e], qr[0, h, t, e] + acc, 1e-12, "residual entry by loops")


# ----------------------------------------------------------------------------- candidates, scores, top-K

def pin_candidates_by_explicit_sets():
    for (N, R) in [(10, 20), (8, 0), (6, 62), (6, 63), (5, 400)]:
        T = N * CT
        qs = np.arange(T)
        cand = O.candidate_mask(qs, R, N)
        for i in range(0, T, 7):
            lo, hi = O.window_bounds(i, R, T)
            win = set(range(lo, hi + 1))
            assert win == {u for u in range(T) if abs(u - i) <= R}, "window set"
            for n in range(N):
                chunk = set(range(n * CT, n * CT + CT))
                assert cand[i, n] == (len(chunk & win) == 0), f"candidate rule i={i} c={n} R={R}"


def pin_topk_brute_force():
    for seed in range(3):
        c = case(10 + seed, N=9, K=3, R=30, beta=0.4)
        queries = np.arange(0, c["T"], 11)
        r = run_layer(c, queries)
        zhat, cand = r["zhat"], r["cand"]
        for b in range(c["B"]):
            for g in range(c["Hkv"]):
                for t in range(len(queries)):
                    cs = np.nonzero(cand[t])[0]
                    m = min(c["K"], len(cs))
                    best = max(itertools.combinations(cs, m), key=lambda S: sum(zhat[b, g, t, list(S)]))
                    got = r["idx"][b, g, t]
                    assert list(got[:m]) == sorted(best) and np.all(got[m:] == -1), "top-K set"


def pin_topk_margin_by_explicit_sort():
    """The selection margin of every row against an explicit sort of that row's
    candidate group scores: the K-th best minus the (K+1)-th best, +inf when the row
    has at most K candidates. Equivalently, the lowest chosen score minus the highest
    score left out, which ties the margin to the chosen set itself. (The GPU tests
    use this margin to decide which rows must match bit for bit.)"""
    cases = [(9, 3, 30, 0.4), (7, 4, 70, 0.0), (12, 1, 10, 0.9), (6, 5, 40, 0.2)]
    n_inf = n_fin = 0
    for seed, (N, K, R, beta) in enumerate(cases):
        c = case(40 + seed, N=N, K=K, R=R, beta=beta)
        queries = np.arange(0, c["T"], 5)
        r = run_layer(c, queries)
        for b in range(c["B"]):
            for g in range(c["Hkv"]):
                for t in range(len(queries)):
                    cs = [cc for cc in range(N) if r["cand"][t, cc]]
                    vals = sorted((float(r["zhat"][b, g, t, cc]) for cc in cs), reverse=True)
                    got = float(r["margin"][b, g, t])
                    if len(vals) <= K:
                        assert got == math.inf, "margin must be +inf with at most K candidates"
                        n_inf += 1
                        continue
                    n_fin += 1
                    assert abs(got - (vals[K - 1] - vals[K])) <= 1e-12, "margin = K-th minus (K+1)-th score"
                    chosen = [int(x) for x in r["idx"][b, g, t] if x >= 0]
                    left = [cc for cc in cs if cc not in chosen]
                    lo_in = min(float(r["zhat"][b, g, t, cc]) for cc in chosen)
                    hi_out = max(float(r["zhat"][b, g, t, cc]) for cc in left)
                    assert abs(got - (lo_in - hi_out)) <= 1e-12, "margin = lowest chosen minus highest left out"
    assert n_inf > 0 and n_fin > 0, "the cases must cover both kinds of row"


def pin_topk_ties_and_padding():
    c = case(12, N=7, K=4, R=70, beta=0.0)
    c["q"][:] = 0.0
    c["A"][:] = 0.0
    queries = np.arange(0, c["T"], 9)
    r = run_layer(c, queries)
    for t, i in enumerate(queries):
        cs = np.nonzero(r["cand"][t])[0]
        m = min(c["K"], len(cs))
        want = list(cs[:m]) + [-1] * (c["K"] - m)
        assert list(r["idx"][0, 0, t]) == want, "exact ties go to smaller chunk indices; -1 padding"
        assert np.all(np.isneginf(r["zsel"][0, :, t, m:])), "-inf padding of zsel"


def pin_entropy_sign_and_shift():
    c = case(13, N=10, K=3, R=20, beta=0.7)
    c["q"][:] = 0.0
    c["q"].reshape(c["B"], c["Hq"], c["N"], SL, c["d"])[:, :, :, SL - 1] = \
        rng(131).standard_normal((c["B"], c["Hq"], c["N"], c["d"])) * 3.0
    c["A"][:] = 0.0
    queries = np.arange(0, c["T"], 13)
    r = run_layer(c, queries)
    Hmin = r["H"].reshape(c["B"], c["Hkv"], c["G"], c["N"]).min(axis=2)     # zhat = -beta min_h H
    for g in range(c["Hkv"]):
        for t in range(len(queries)):
            cs = np.nonzero(r["cand"][t])[0]
            order = cs[np.argsort(Hmin[0, g, cs], kind="stable")]
            assert list(r["idx"][0, g, t]) == sorted(order[: c["K"]]), "lowest-entropy chunks win"
    # a constant added to every entropy leaves the selection unchanged
    c2 = case(14, beta=0.5)
    q2 = np.arange(0, c2["T"], 6)
    rr = run_layer(c2, q2)
    z = O.route_scores(rr["qt"], rr["s"], rr["H"] + 3.25, 0.5, c2["scale"])
    idx2, _ = O.select_topk(O.group_max(z, c2["G"]), rr["cand"], c2["K"])
    assert np.array_equal(idx2, rr["idx"]), "constant entropy shift changes selection"
    z0 = O.route_scores(rr["qt"], rr["s"], rr["H"] * 0 + 100.0, 0.0, c2["scale"])
    close(z0, O.route_scores(rr["qt"], rr["s"], rr["H"], 0.0, c2["scale"]), 0.0, "beta=0 ignores H")


def pin_scores_closed_form_identical_keys():
    """All content keys of chunk n equal w_n => s_n = w_n, H = ln 63, z = scale q~.w_n - beta ln 63."""
    c = case(15, N=10, K=3, R=20, beta=0.3)
    B, Hq, Hkv, N, d = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"]
    W = rng(151).standard_normal((B, Hkv, N, d))
    kv = c["k"].reshape(B, Hkv, N, SL, d)
    kv[:, :, :, :CT] = W[:, :, :, None, :]
    queries = np.arange(0, c["T"], 17)
    r = run_layer(c, queries)
    Wh = np.repeat(W, c["G"], axis=1)
    close(r["s"], Wh, 1e-12, "summary of identical keys")
    close(r["H"], np.full_like(r["H"], math.log(CT)), 1e-12, "entropy of identical keys")
    qt = r["qt"]
    for (h, t, n) in [(0, 0, 5), (3, 4, 9), (2, 7, 0), (1, 11, 6)]:
        want = c["scale"] * float(np.dot(qt[0, h, t], W[0, h // c["G"], n])) - c["beta"] * math.log(CT)
        close(r["z"][0, h, t, n], want, 1e-12, "closed-form score")
        kk = list(r["idx"][0, h // c["G"], t])
        if n in kk:
            close(r["zsel"][0, h, t, kk.index(n)], want, 1e-12, "zsel is the head's own score")


def pin_group_max_dominant_head():
    """One head loves chunk n* (+), the others hate it (-): the group maximum selects it."""
    c = case(16, N=10, K=1, R=20, beta=0.0, Hq=4, Hkv=1, d=8)
    B, Hq, N, d, G = c["B"], c["Hq"], c["N"], c["d"], c["G"]
    e = np.eye(d)
    kv = c["k"].reshape(B, 1, N, SL, d)
    kv[:, :, :, :CT] = 0.0
    nstar = 8
    kv[:, :, nstar, :CT] = e[0]
    c["A"][:] = 0.0
    queries = np.arange(0, 5 * CT, 29)           # queries in the first chunks; chunk 8 is remote
    sl = O.slot_of(queries)
    c["q"][:, :, sl] = 0.0
    c["q"][:, :, sl, 0] = -10.0
    c["q"][:, 2, sl, 0] = 10.0                   # head 2 of the group loves chunk n*
    r = run_layer(c, queries)
    assert np.all(r["idx"][0, 0, :, 0] == nstar), "group maximum must select the chunk one head loves"
    zs = r["zsel"][0, :, :, 0]
    assert np.all(zs[2] > 0) and np.all(np.delete(zs, 2, axis=0) < 0), "per-head zsel"


# ----------------------------------------------------------------------------- attention (steps 6-8)

def _flat_weights(c, r, queries):
    """Independent formulation: explicit weights over all T content keys, per (head, query)."""
    B, Hq, Hkv, N, d, G, T, R, sc = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"], c["G"], c["T"], c["R"], c["scale"]
    cs = content_slots(T)
    out_o = np.zeros((B, Hq, len(queries), d))
    out_l = np.zeros((B, Hq, len(queries)))
    for t, i in enumerate(queries):
        for h in range(Hq):
            g = h // G
            qv = c["q"][0, h, O.slot_of(i)]
            logit = np.full(T, -np.inf)
            for u in range(T):
                if abs(u - i) <= R:
                    logit[u] = sc * qv @ c["k"][0, g, cs[u]]
            for kk, n in enumerate(r["idx"][0, g, t]):
                if n < 0:
                    continue
                us = np.arange(n * CT, n * CT + CT)
                ell = sc * c["k"][0, g, cs[us]] @ qv
                lse_c = np.log(np.sum(np.exp(ell - ell.max()))) + ell.max()
                logit[us] = r["zsel"][0, h, t, kk] + ell - lse_c
            m = logit[np.isfinite(logit)].max()
            w = np.exp(logit - m)
            Z = w.sum()
            out_o[0, h, t] = (w / Z) @ c["v"][0, g, cs]
            out_l[0, h, t] = m + np.log(Z)
    return out_o, out_l


def pin_weights_formulation_and_convexity():
    c = case(20, N=8, K=3, R=25, beta=0.2)
    queries = np.array([0, 1, 62, 63, 100, 251, 300, 503])
    r = run_layer(c, queries)
    o2, l2 = _flat_weights(c, r, queries)
    close(r["o"], o2, 1e-12, "two-level softmax equals its flattened weights")
    close(r["lse"], l2, 1e-12, "log partition")
    # convexity: o within the per-coordinate range of the V rows it can see
    cs = content_slots(c["T"])
    for t, i in enumerate(queries):
        for g in range(c["Hkv"]):
            lo, hi = O.window_bounds(i, c["R"], c["T"])
            rows = list(cs[lo: hi + 1])
            for n in r["idx"][0, g, t]:
                if n >= 0:
                    rows += list(cs[n * CT: n * CT + CT])
            V = c["v"][0, g, rows]
            oo = r["o"][0, g * c["G"]:(g + 1) * c["G"], t]
            assert np.all(oo >= V.min(0) - 1e-12) and np.all(oo <= V.max(0) + 1e-12), "convex combination"
    Pu, Pc, _ = O.partition(rng(21).standard_normal((3, 9)), rng(22).standard_normal((3, 4)))
    close(Pu.sum(1) + Pc.sum(1), np.ones(3), 1e-14, "partition weights sum to one")


def pin_ideal_chunk_logit_is_flat_attention():
    """zsel = log-sum-exp of the chunk's own logits => flat softmax over window + chosen chunks."""
    c = case(23, N=9, K=3, R=30, beta=0.1)
    queries = np.array([5, 70, 200, 311, 450, 566])
    r = run_layer(c, queries)
    cs = content_slots(c["T"])
    zsel = r["zsel"].copy()
    for t, i in enumerate(queries):
        for h in range(c["Hq"]):
            g = h // c["G"]
            qv = c["q"][0, h, O.slot_of(i)]
            for kk, n in enumerate(r["idx"][0, g, t]):
                if n >= 0:
                    ell = c["scale"] * c["k"][0, g, cs[n * CT:(n + 1) * CT]] @ qv
                    zsel[0, h, t, kk] = np.log(np.sum(np.exp(ell - ell.max()))) + ell.max()
    o, _ = O.routed_attention(c["q"][:, :, O.slot_of(queries)], c["k"], c["v"], r["idx"], zsel,
                              c["R"], c["scale"], queries)
    for t, i in enumerate(queries):
        for h in range(c["Hq"]):
            g = h // c["G"]
            mask = np.zeros(c["T"], dtype=bool)
            lo, hi = O.window_bounds(i, c["R"], c["T"])
            mask[lo: hi + 1] = True
            for n in r["idx"][0, g, t]:
                if n >= 0:
                    mask[n * CT:(n + 1) * CT] = True
            want = sdpa(c["q"][0, h, O.slot_of(i)][None], c["k"][0, g, cs], c["v"][0, g, cs],
                        mask[None], c["scale"])[0]
            close(o[0, h, t], want, 1e-12, "flat attention over window and chosen chunks")


def pin_k0_is_window_attention():
    c = case(24, N=8, K=0, R=40)
    queries = np.arange(0, c["T"], 23)
    r = run_layer(c, queries)
    cs = content_slots(c["T"])
    ii = np.arange(c["T"])
    for t, i in enumerate(queries):
        for h in range(c["Hq"]):
            g = h // c["G"]
            mask = (np.abs(ii - i) <= c["R"])[None]
            want = sdpa(c["q"][0, h, O.slot_of(i)][None], c["k"][0, g, cs], c["v"][0, g, cs], mask, c["scale"])[0]
            close(r["o"][0, h, t], want, 1e-12, "K=0 is windowed attention")


def pin_wide_window_is_dense_attention():
    c = case(25, N=6, K=3, R=6 * CT)
    queries = np.arange(0, c["T"], 19)
    r = run_layer(c, queries)
    assert not r["cand"].any() and np.all(r["idx"] == -1), "no remote chunk when the window covers all"
    cs = content_slots(c["T"])
    for h in range(c["Hq"]):
        g = h // c["G"]
        want = sdpa(c["q"][0, h, O.slot_of(queries)], c["k"][0, g, cs], c["v"][0, g, cs],
                    np.ones((len(queries), c["T"]), dtype=bool), c["scale"])
        close(r["o"][0, h], want, 1e-12, "dense bidirectional attention over content tokens")


def pin_identical_chunk_keys_average_values():
    """Identical keys inside a chunk => the second softmax is uniform => u_bar = mean of content V."""
    g = rng(26)
    kc = np.repeat(g.standard_normal((2, 1, 8)), CT, axis=1)
    vc = g.standard_normal((2, CT, 8))
    ub = O.chunk_attention(g.standard_normal((3, 8)), kc, vc, 0.35)
    close(ub, np.broadcast_to(vc.mean(axis=1), ub.shape), 1e-12, "uniform intra-chunk weights")


def pin_remote_chunk_permutation():
    """Moving whole remote chunks (all 64 slots) permutes the selection and leaves outputs unchanged."""
    c = case(27, N=12, K=3, R=40, beta=0.4)
    queries = np.arange(0, 2 * CT - 40, 3)        # windows stay inside chunks 0..2
    r0 = run_layer(c, queries)
    perm = np.arange(c["N"])
    perm[4:] = 4 + rng(271).permutation(c["N"] - 4)     # new position p holds old chunk perm[p]
    inv = np.argsort(perm)
    def mv(a, axis):
        sh = list(a.shape)
        sh[axis:axis + 1] = [c["N"], SL]
        return np.take(a.reshape(sh), perm, axis=axis).reshape(a.shape)
    c2 = dict(c)
    c2["q"], c2["k"], c2["v"], c2["x"] = mv(c["q"], 2), mv(c["k"], 2), mv(c["v"], 2), mv(c["x"], 1)
    r1 = run_layer(c2, queries)
    close(r1["o"], r0["o"], 1e-12, "output under a permutation of remote chunks")
    mapped = np.where(r0["idx"] >= 0, inv[np.maximum(r0["idx"], 0)], -1)
    assert np.array_equal(np.sort(mapped, axis=-1), np.sort(r1["idx"], axis=-1)), "selection maps"


def pin_gqa_shared_support():
    """Every head of a KV group reads exactly the group's chosen remote chunks: perturbing the
    values of a remote chunk moves a head's output iff the chunk is in its group's set."""
    c = case(28, N=9, K=2, R=20, Hq=6, Hkv=2)
    queries = np.array([3, 150, 400])
    r = run_layer(c, queries)
    assert r["idx"].shape == (1, 2, 3, 2), "one selection per KV group"
    qr = c["q"][:, :, O.slot_of(queries)]
    base, _ = O.routed_attention(qr, c["k"], c["v"], r["idx"], r["zsel"], c["R"], c["scale"], queries)
    for n in range(c["N"]):
        v = c["v"].copy()
        v[:, :, n * SL: n * SL + CT] += 1.0
        o, _ = O.routed_attention(qr, c["k"], v, r["idx"], r["zsel"], c["R"], c["scale"], queries)
        for t, i in enumerate(queries):
            if not r["cand"][t, n]:
                continue
            for h in range(c["Hq"]):
                moved = np.max(np.abs(o[0, h, t] - base[0, h, t])) > 1e-9
                assert moved == (n in set(r["idx"][0, h // c["G"], t])), "head support = group set"


# ----------------------------------------------------------------------------- SWA

def pin_swa_against_library():
    g = rng(30)
    B, Hq, Hkv, L, d = 1, 4, 2, 200, 16
    q, k, v = (g.standard_normal((B, H, L, d)) for H in (Hq, Hkv, Hkv))
    sc = 0.25
    t = np.arange(L)
    for R in (0, 1, 17, 64, L - 1, 5 * L):
        rows = np.arange(0, L, 3)
        o, lse = O.swa_attention(q, k, v, R, sc, rows)
        for h in range(Hq):
            mask = np.abs(rows[:, None] - t[None, :]) <= R
            close(o[0, h], sdpa(q[0, h, rows], k[0, h // 2], v[0, h // 2], mask, sc), 1e-12, f"SWA R={R}")
            logits = sc * q[0, h, rows] @ k[0, h // 2].T
            logits[~mask] = -np.inf
            ref = torch.logsumexp(torch.from_numpy(logits), dim=-1).numpy()
            close(lse[0, h], ref, 1e-12, "SWA log partition")
        if R == 0:
            close(o, np.repeat(v, 2, axis=1)[:, :, rows], 1e-12, "radius 0 returns v")


# ----------------------------------------------------------------------------- backward (membership fixed)

def _fd(f, args, name, w, eps=1e-6):
    """Central difference of scalar f along direction w of argument `name`."""
    up = dict(args)
    dn = dict(args)
    up[name] = args[name] + eps * w
    dn[name] = args[name] - eps * w
    return (f(**up) - f(**dn)) / (2 * eps)


def _check_fd(f, args, grads, what, ndir=3, seed=0, tol=1e-6):
    """Directional derivatives of f along random directions against <grad, w>."""
    g = rng(100 + seed)
    for name, gr in grads.items():
        for _ in range(ndir):
            w = g.standard_normal(args[name].shape)
            num = _fd(f, args, name, w)
            ana = float(np.sum(gr * w))
            assert abs(num - ana) <= tol * max(1.0, abs(num)), \
                f"{what}: d/d{name} finite difference {num:.9e} vs gradient {ana:.9e}"


def _bwd_case(seed, K, R, queries, N=6):
    c = case(seed, N=N, Hq=4, Hkv=2, d=8, K=K, R=R)
    r = run_layer(c, queries)
    g = rng(seed + 1)
    zsel = np.where(r["idx"].repeat(c["G"], axis=1) >= 0, g.standard_normal(r["zsel"].shape), -np.inf)
    dO = g.standard_normal(r["o"].shape)
    return c, r, zsel, dO


def pin_attention_backward_finite_differences():
    for K, R in ((2, 12), (4, 100)):                       # R=100 leaves rows with fewer than K candidates
        queries = np.array([0, 3, 64, 150, 290, 377])
        c, r, zsel, dO = _bwd_case(40 + K, K, R, queries)
        qr = c["q"][:, :, O.slot_of(queries)]
        args = dict(qr=qr, k=c["k"], v=c["v"], zs=np.where(np.isfinite(zsel), zsel, 0.0))
        fin = np.isfinite(zsel)

        def f(qr, k, v, zs):
            o, _ = O.routed_attention(qr, k, v, r["idx"], np.where(fin, zs, -np.inf), R, c["scale"], queries)
            return float(np.sum(o * dO))

        dq, dk, dv, dz = OB.routed_attention_backward(qr, c["k"], c["v"], r["idx"], zsel, R, c["scale"],
                                                      queries, dO)
        if K == 4:
            assert not fin.all(), "case must hold padded selections"
        assert np.all(dz[~fin] == 0), "no gradient for padded selections"
        _check_fd(f, args, dict(qr=dq, k=dk, v=dv, zs=dz), f"routed attention backward K={K} R={R}", seed=K)


def _torch_attention_grads(qrows, kc, vc, mask, dO, scale):
    """float64 torch autograd of masked attention; qrows [n,d], kc, vc [T,d], mask [n,T]."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)).requires_grad_(True) for a in (qrows, kc, vc))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    (o[0, 0] * torch.from_numpy(dO)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_attention_backward_window_only_is_library_autograd():
    c = case(44, N=7, Hq=4, Hkv=2, d=8, K=0, R=37)
    queries = np.arange(0, c["T"], 11)
    r = run_layer(c, queries)
    dO = rng(45).standard_normal(r["o"].shape)
    dq, dk, dv, _ = OB.routed_attention_backward(c["q"][:, :, O.slot_of(queries)], c["k"], c["v"], r["idx"],
                                                 r["zsel"], c["R"], c["scale"], queries, dO)
    cs = content_slots(c["T"])
    mask = np.abs(queries[:, None] - np.arange(c["T"])[None, :]) <= c["R"]
    wk, wv = np.zeros_like(dk), np.zeros_like(dv)
    for h in range(c["Hq"]):
        g = h // c["G"]
        gq, gk, gv = _torch_attention_grads(c["q"][0, h, O.slot_of(queries)], c["k"][0, g, cs], c["v"][0, g, cs],
                                            mask, dO[0, h], c["scale"])
        close(dq[0, h], gq, 1e-12, "window-only dq")
        wk[0, g, cs] += gk
        wv[0, g, cs] += gv
    close(dk, wk, 1e-12, "window-only dk")
    close(dv, wv, 1e-12, "window-only dv")


def pin_attention_backward_lse_chunk_logits_is_flat_autograd():
    """With zsel = log-sum-exp of the chunk's own logits (a function of q), the total
    gradient is that of flat attention over the window and the chosen chunks: the
    attention backward plus dzsel times the gradient of log-sum-exp (scale * pi k
    for q, scale * pi q for k)."""
    c = case(46, N=9, Hq=4, Hkv=2, d=8, K=3, R=30)
    queries = np.array([5, 70, 200, 311, 450, 566])
    r = run_layer(c, queries)
    sc = c["scale"]
    cs = content_slots(c["T"])
    qr = c["q"][:, :, O.slot_of(queries)]
    zsel = r["zsel"].copy()
    pis = {}
    for t in range(len(queries)):
        for h in range(c["Hq"]):
            g = h // c["G"]
            for kk, n in enumerate(r["idx"][0, g, t]):
                if n >= 0:
                    ell = sc * c["k"][0, g, cs[n * CT:(n + 1) * CT]] @ qr[0, h, t]
                    zsel[0, h, t, kk] = np.log(np.sum(np.exp(ell - ell.max()))) + ell.max()
                    pis[(h, t, kk)] = np.exp(ell - zsel[0, h, t, kk])
    dO = rng(47).standard_normal(r["o"].shape)
    dq, dk, dv, dz = OB.routed_attention_backward(qr, c["k"], c["v"], r["idx"], zsel, c["R"], sc, queries, dO)
    for (h, t, kk), pi in pis.items():
        g = h // c["G"]
        rows = cs[r["idx"][0, g, t, kk] * CT + np.arange(CT)]
        dq[0, h, t] += dz[0, h, t, kk] * sc * pi @ c["k"][0, g, rows]
        dk[0, g, rows] += dz[0, h, t, kk] * sc * pi[:, None] * qr[0, h, t][None, :]
    wk, wv = np.zeros_like(dk), np.zeros_like(dv)
    for h in range(c["Hq"]):
        g = h // c["G"]
        mask = np.zeros((len(queries), c["T"]), dtype=bool)
        for t, i in enumerate(queries):
            lo, hi = O.window_bounds(i, c["R"], c["T"])
            mask[t, lo: hi + 1] = True
            for n in r["idx"][0, g, t]:
                if n >= 0:
                    mask[t, n * CT:(n + 1) * CT] = True
        gq, gk, gv = _torch_attention_grads(qr[0, h], c["k"][0, g, cs], c["v"][0, g, cs], mask, dO[0, h], sc)
        close(dq[0, h], gq, 1e-12, "flat-equivalent dq")
        wk[0, g, cs] += gk
        wv[0, g, cs] += gv
    close(dk, wk, 1e-12, "flat-equivalent dk")
    close(dv, wv, 1e-12, "flat-equivalent dv")


def pin_score_backward_finite_differences():
    queries = np.array([0, 40, 130, 260, 377])
    c, r, _, _ = _bwd_case(48, 3, 20, queries)
    g = rng(49)
    s = g.standard_normal((1, c["Hq"], c["N"], c["d"]))
    H = np.abs(g.standard_normal((1, c["Hq"], c["N"])))
    sl = O.slot_of(queries)
    fin = r["idx"].repeat(c["G"], axis=1) >= 0
    dzsel = np.where(fin, g.standard_normal(r["zsel"].shape), 0.0)
    args = dict(qr=c["q"][:, :, sl], xr=c["x"][:, sl], A=c["A"], Bm=c["Bm"], s=s, H=H)

    def f(qr, xr, A, Bm, s, H):
        z = O.route_scores(O.routing_query(qr, xr, A, Bm), s, H, c["beta"], c["scale"])
        zs = O.gather_zsel(z, r["idx"], c["G"])
        return float(np.sum(np.where(fin, zs, 0.0) * dzsel))

    dq, dx, dA, dBm, ds, dH = OB.route_score_backward(args["qr"], args["xr"], c["A"], c["Bm"], s, H, r["idx"],
                                                      dzsel, c["beta"], c["scale"])
    _check_fd(f, args, dict(qr=dq, xr=dx, A=dA, Bm=dBm, s=ds, H=dH), "route score backward", seed=7)


def pin_summary_backward_finite_differences():
    c = case(50, N=5, Hq=4, Hkv=2, d=8)
    g = rng(51)
    qm = c["q"].reshape(1, c["Hq"], c["N"], SL, c["d"])[:, :, :, SL - 1]
    ds = g.standard_normal((1, c["Hq"], c["N"], c["d"]))
    dH = g.standard_normal((1, c["Hq"], c["N"]))
    args = dict(qm=qm, k=c["k"])

    def f(qm, k):
        s, H = O.chunk_summary_from_mask(qm, k, c["scale"])
        return float(np.sum(s * ds) + np.sum(H * dH))

    dq, dk = OB.chunk_summary_backward(qm, c["k"], c["scale"], ds, dH)
    _check_fd(f, args, dict(qm=dq, k=dk), "chunk summary backward", seed=8)
    assert np.all(dk.reshape(1, c["Hkv"], c["N"], SL, c["d"])[:, :, :, SL - 1] == 0), "mask-slot keys get nothing"


def pin_summary_backward_uniform_point():
    """Zero mask query: uniform weights. Entropy is at its maximum (no gradient from dH);
    the summary's gradient is scale * Cov(k) ds for the query and ds/63 for each key."""
    c = case(52, N=4, Hq=2, Hkv=1, d=8)
    g = rng(53)
    qm = np.zeros((1, c["Hq"], c["N"], c["d"]))
    ds = g.standard_normal((1, c["Hq"], c["N"], c["d"]))
    dH = g.standard_normal((1, c["Hq"], c["N"]))
    dq_h, dk_h = OB.chunk_summary_backward(qm, c["k"], c["scale"], np.zeros_like(ds), dH)
    close(dq_h, 0.0, 1e-13, "entropy is stationary at uniform weights")
    close(dk_h, 0.0, 1e-13, "entropy gradient on keys at a zero query")
    dq, dk = OB.chunk_summary_backward(qm, c["k"], c["scale"], ds, np.zeros_like(dH))
    kc = c["k"].reshape(1, 1, c["N"], SL, c["d"])[0, 0, :, :CT]
    for n in range(c["N"]):
        cov = np.cov(kc[n].T, bias=True)
        for h in range(c["Hq"]):
            close(dq[0, h, n], c["scale"] * cov @ ds[0, h, n], 1e-13, "covariance closed form")
        close(dk.reshape(1, 1, c["N"], SL, c["d"])[0, 0, n, :CT],
              np.repeat(ds[0, :, n].sum(0)[None] / CT, CT, axis=0), 1e-13, "uniform key gradient")


def pin_layer_backward_finite_differences():
    queries = np.array([2, 66, 190, 301, 377])
    c, r, _, dO = _bwd_case(54, 3, 15, queries)
    idx = r["idx"]
    sl = O.slot_of(queries)
    G, N, sc = c["G"], c["N"], c["scale"]

    def f(q, k, v, x, A, Bm):
        qm = q.reshape(1, c["Hq"], N, SL, c["d"])[:, :, :, SL - 1]
        s, H = O.chunk_summary_from_mask(qm, k, sc)
        z = O.route_scores(O.routing_query(q[:, :, sl], x[:, sl], A, Bm), s, H, c["beta"], sc)
        o, _ = O.routed_attention(q[:, :, sl], k, v, idx, O.gather_zsel(z, idx, G), c["R"], sc, queries)
        return float(np.sum(o * dO))

    args = dict(q=c["q"], k=c["k"], v=c["v"], x=c["x"], A=c["A"], Bm=c["Bm"])
    gr = OB.route_layer_backward(c["q"], c["k"], c["v"], c["x"], c["A"], c["Bm"], idx, dO, R=c["R"],
                                 beta=c["beta"], scale=sc, queries=queries)
    _check_fd(f, args, dict(q=gr["dq"], k=gr["dk"], v=gr["dv"], x=gr["dx"], A=gr["dA"], Bm=gr["dBm"]),
              "route layer backward", seed=9)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
