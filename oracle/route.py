"""Route-layer attention and bidirectional sliding-window attention in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests, the smoke
check and the benchmark's CPU-baseline leg, never by the product path.

Notation. A sequence of N chunks has L = 64 N slots. Chunk c holds content
tokens in slots 64c .. 64c+62 and its routing mask in slot 64c+63 ("Prefilling-
dLLM v2", Abstract and Figure 3 caption; "The 172x Speedup Has an Evidence
Budget", section "How learned routing controls what the model can read": 63
content tokens plus one appended routing position per 64-slot chunk). Content
index i (0 <= i < T = 63 N) lives in slot sigma(i) = 64 floor(i/63) + (i mod 63).
Query head h uses KV head g(h) = floor(h / G), G = Hq / Hkv.

Readings of points the pages leave open are listed next to the code that takes
them; each is repeated in the design notes of the repository.
"""
import numpy as np

SLOTS = 64
CONTENT = 63


# ----------------------------------------------------------------------------- indexing

def slot_of(i):
    """Slot of content index i: 64 * (i // 63) + i % 63."""
    i = np.asarray(i, dtype=np.int64)
    return (i // CONTENT) * SLOTS + (i % CONTENT)


def group_of(h, G):
    """KV head used by query head h: contiguous GQA groups (Figure 3 caption: a GQA group)."""
    return h // G


# ----------------------------------------------------------------------------- primitives

def softmax(x, axis=-1):
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(x - m)
    return e / e.sum(axis=axis, keepdims=True)


def entropy(p, axis=-1):
    """Shannon entropy with the natural log; a zero weight contributes zero."""
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return -t.sum(axis=axis)


def logsumexp(x, axis=-1):
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return (m + np.log(np.exp(x - m).sum(axis=axis, keepdims=True))).squeeze(axis)


# ----------------------------------------------------------------------------- step 1: summaries

def chunk_summary_from_mask(q_mask, k, scale):
    """Summary keys and pooling entropies from the mask-slot queries.

    "Prefilling-dLLM v2", Figure 3 caption: the routing mask's query pools its
    chunk's content keys with a softmax inside the chunk, and the weighted sum is
    the summary key s_c. "The 172x Speedup...", same section: the entropy of these
    pooling weights is the second ranking signal.

    Readings: every logit uses scale = 1/sqrt(d); the summary is per query head
    (head h's mask query pools KV head g(h)'s keys); the 63 content keys are
    pooled, the mask slot's own key is not; entropy is Shannon, natural log.

    q_mask [B,Hq,N,d] (the query at slot 64c+63), k [B,Hkv,L,d]
    -> s [B,Hq,N,d], H [B,Hq,N].
    """
    B, Hq, N, d = q_mask.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    kc = k.reshape(B, Hkv, N, SLOTS, d)[:, :, :, :CONTENT, :]
    s = np.empty((B, Hq, N, d))
    H = np.empty((B, Hq, N))
    for h in range(Hq):
        g = group_of(h, G)
        logits = scale * np.einsum("bnd,bnjd->bnj", q_mask[:, h], kc[:, g])
        alpha = softmax(logits, axis=-1)
        s[:, h] = np.einsum("bnj,bnjd->bnd", alpha, kc[:, g])
        H[:, h] = entropy(alpha, axis=-1)
    return s, H


def chunk_summary(q, k, scale):
    """Summaries from the full query tensor q [B,Hq,L,d]: its mask-slot rows are used."""
    B, Hq, L, d = q.shape
    N = L // SLOTS
    q_mask = q.reshape(B, Hq, N, SLOTS, d)[:, :, :, SLOTS - 1, :]
    return chunk_summary_from_mask(q_mask, k, scale)


def chunk_summary_mean(k, Hq):
    """Mean summaries: "Prefilling-dLLM v2", Table 6 (row "Mean summary") and its
    discussion, where attention-weighted summaries are replaced by mean pooling.

    Readings: the 63 content keys are averaged (the mask slot's key is not); the
    summary is repeated for every query head of the group; the pooling weights are
    uniform, so the entropy is ln 63 for every chunk.

    k [B,Hkv,L,d] -> s [B,Hq,N,d], H [B,Hq,N].
    """
    B, Hkv, L, d = k.shape
    N, G = L // SLOTS, Hq // Hkv
    kc = k.reshape(B, Hkv, N, SLOTS, d)[:, :, :, :CONTENT, :]
    s = np.repeat(kc.mean(axis=3), G, axis=1)
    H = np.full((B, Hq, N), np.log(CONTENT))
    return s, H


# ----------------------------------------------------------------------------- step 2: routing query

def routing_query(q_rows, x_rows, A, Bm):
    """Residual-augmented routing query q~ = q + (x A) B, split per head.

    "Prefilling-dLLM v2", Figure 3 caption: a content query adds a low-rank
    residual before scoring the summaries; "The 172x Speedup...": rank 64, it
    adapts queries for routing without replacing the query projection.

    Reading: x A B with A [D,r] and B [r, Hq*d], no extra scale; columns
    h*d..(h+1)*d of x A B belong to head h.

    q_rows [B,Hq,n,d] (plain queries at the query slots), x_rows [B,n,D]
    -> q~ [B,Hq,n,d].
    """
    B, Hq, n, d = q_rows.shape
    res = (x_rows @ A) @ Bm
    return q_rows + res.reshape(B, n, Hq, d).transpose(0, 2, 1, 3)


# ----------------------------------------------------------------------------- step 3: window, candidates

def window_bounds(i, R, T):
    """Bidirectional local window of content index i: [max(0,i-R), min(T-1,i+R)].

    "Prefilling-dLLM v2", Table 3: the local window is a bidirectional radius
    (256 on route layers). Reading: content-index space, |u - i| <= R, clipped at
    the sequence ends.
    """
    return max(0, int(i) - R), min(T - 1, int(i) + R)


def candidate_mask(queries, R, N):
    """Remote chunks of each query: no content index of the chunk lies in its window.

    "Prefilling-dLLM v2", Table 3: the remote budget is gathered beyond the local
    window. Reading: a chunk is a candidate only if none of its content tokens is
    in the window, so the two key sets never overlap.

    queries [n] content indices -> bool [n, N].
    """
    queries = np.asarray(queries, dtype=np.int64)
    c = np.arange(N, dtype=np.int64)
    first = CONTENT * c
    last = first + CONTENT - 1
    i = queries[:, None]
    return (last[None, :] < i - R) | (first[None, :] > i + R)


# ----------------------------------------------------------------------------- steps 4-5: scores, top-K

def route_scores(qt, s, H, beta, scale):
    """z[b,h,i,c] = scale * q~[b,h,i] . s[b,h,c] - beta * H[b,h,c].

    "Prefilling-dLLM v2", Figure 3 caption (the residual-augmented query scores
    the summaries); "The 172x Speedup...": similarity to the summary and the
    pooling entropy rank the chunks. Reading: similarity minus beta times entropy.
    """
    return scale * np.einsum("bhnd,bhcd->bhnc", qt, s) - beta * H[:, :, None, :]


def group_max(z, G):
    """Maximum over the G query heads of each KV group ("Prefilling-dLLM v2", Figure 3 caption)."""
    B, Hq, n, N = z.shape
    return z.reshape(B, Hq // G, G, n, N).max(axis=2)


def select_topk(zhat, cand, K):
    """Top-K remote chunks per (batch, KV group, query), shared by the group's heads.

    "Prefilling-dLLM v2", Figure 3 caption. Readings: ties go to the smaller chunk
    index; the chosen chunks are stored in ascending order; with fewer than K
    candidates all are chosen and the list is padded with -1.

    zhat [B,Hkv,n,N], cand bool [n,N] -> idx int64 [B,Hkv,n,K], margin [B,Hkv,n]
    (K-th minus (K+1)-th best score; +inf when at most K candidates).
    """
    B, Hkv, n, N = zhat.shape
    key = np.where(cand[None, None], -zhat, np.inf)
    order = np.argsort(key, axis=-1, kind="stable")          # best first, ties by index
    ncand = cand.sum(axis=-1)                                  # [n]
    idx = np.full((B, Hkv, n, K), -1, dtype=np.int64)
    margin = np.full((B, Hkv, n), np.inf)
    if K == 0:
        return idx, margin
    take = order[..., :K]
    vals = np.take_along_axis(zhat, order, axis=-1)
    for j in range(n):
        m = min(K, int(ncand[j]))
        if m > 0:
            idx[:, :, j, :m] = np.sort(take[:, :, j, :m], axis=-1)
        if ncand[j] > K:
            margin[:, :, j] = vals[:, :, j, K - 1] - vals[:, :, j, K]
    return idx, margin


def gather_zsel(z, idx, G):
    """zsel[b,h,i,k] = z[b,h,i,idx[b,g(h),i,k]]; -inf where idx is -1."""
    B, Hq, n, N = z.shape
    idx_h = np.repeat(idx, G, axis=1)
    safe = np.where(idx_h >= 0, idx_h, 0)
    out = np.take_along_axis(z, safe, axis=-1)
    return np.where(idx_h >= 0, out, -np.inf)


# ----------------------------------------------------------------------------- steps 6-8: attention

def chunk_attention(qh, kc, vc, scale):
    """Second softmax inside each selected chunk.

    "Prefilling-dLLM v2", Figure 3 caption: a second softmax spreads each
    chunk's mass over its content tokens. Reading: over the 63 content keys with
    the plain query. qh [G,d]; kc, vc [nsel,63,d] -> u_bar [G,nsel,d].
    """
    ell = scale * np.einsum("hd,cjd->hcj", qh, kc)
    pi = softmax(ell, axis=-1)
    return np.einsum("hcj,cjd->hcd", pi, vc)


def partition(a, zc):
    """One softmax over local-window logits a [G,W] and chunk logits zc [G,nsel].

    "Prefilling-dLLM v2", Figure 3 caption: the selected chunk scores and the
    local window's log-sum-exp share one partition. Returns P_u [G,W], P_c
    [G,nsel], lse [G].
    """
    allv = np.concatenate([a, zc], axis=1)
    M = np.max(allv, axis=1, keepdims=True)
    e = np.exp(allv - M)
    Z = e.sum(axis=1, keepdims=True)
    P = e / Z
    return P[:, : a.shape[1]], P[:, a.shape[1]:], (M + np.log(Z))[:, 0]


def routed_attention(q_rows, k, v, idx, zsel, R, scale, queries):
    """Route-layer output for the given content queries.

    o = sum_u P_u v_u + sum_c P_c u_bar_c with local logits a_u = scale * q . k_u
    over the window and chunk logits zsel (the head's own score, residual and
    entropy included).

    q_rows [B,Hq,n,d] plain queries at sigma(queries); k, v [B,Hkv,L,d];
    idx [B,Hkv,n,K] (ascending, -1 padded); zsel [B,Hq,n,K]
    -> o [B,Hq,n,d], lse [B,Hq,n].
    """
    B, Hq, n, d = q_rows.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    N = k.shape[2] // SLOTS
    T = N * CONTENT
    jj = np.arange(CONTENT)
    o = np.empty((B, Hq, n, d))
    lse = np.empty((B, Hq, n))
    for b in range(B):
        for t, i in enumerate(np.asarray(queries)):
            lo, hi = window_bounds(i, R, T)
            ws = slot_of(np.arange(lo, hi + 1))
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                qh = q_rows[b, hs, t]                               # [G,d]
                a = scale * qh @ k[b, g, ws].T                      # [G,W]
                sel = idx[b, g, t]
                sel = sel[sel >= 0]
                zc = zsel[b, hs, t, : len(sel)]                     # [G,nsel]
                cs = sel[:, None] * SLOTS + jj[None, :]             # [nsel,63]
                ubar = chunk_attention(qh, k[b, g, cs], v[b, g, cs], scale)
                Pu, Pc, lz = partition(a, zc)
                o[b, hs, t] = Pu @ v[b, g, ws] + np.einsum("hc,hcd->hd", Pc, ubar)
                lse[b, hs, t] = lz
    return o, lse


def route_layer_rows(q_rows, q_mask, k, v, x_rows, A, Bm, *, K, R, beta, scale, queries):
    """Whole route layer for the given content queries (steps 1-8 in order).

    q_rows [B,Hq,n,d] queries at sigma(queries); q_mask [B,Hq,N,d] mask-slot
    queries; x_rows [B,n,D]. Returns a dict with every intermediate.
    """
    B, Hq, n, d = q_rows.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    N = k.shape[2] // SLOTS
    s, H = chunk_summary_from_mask(q_mask, k, scale)
    qt = routing_query(q_rows, x_rows, A, Bm)
    z = route_scores(qt, s, H, beta, scale)
    zhat = group_max(z, G)
    cand = candidate_mask(queries, R, N)
    idx, margin = select_topk(zhat, cand, K)
    zsel = gather_zsel(z, idx, G)
    o, lse = routed_attention(q_rows, k, v, idx, zsel, R, scale, queries)
    return dict(s=s, H=H, qt=qt, z=z, zhat=zhat, cand=cand, idx=idx, margin=margin,
                zsel=zsel, o=o, lse=lse)


def route_layer(q, k, v, x, A, Bm, *, K, R, beta, scale, queries):
    """Whole route layer from full tensors q [B,Hq,L,d], x [B,L,D]."""
    B, Hq, L, d = q.shape
    N = L // SLOTS
    slots = slot_of(queries)
    q_mask = q.reshape(B, Hq, N, SLOTS, d)[:, :, :, SLOTS - 1, :]
    return route_layer_rows(q[:, :, slots], q_mask, k, v, x[:, slots], A, Bm,
                            K=K, R=R, beta=beta, scale=scale, queries=queries)


# ----------------------------------------------------------------------------- companion: SWA

def swa_attention(q, k, v, R, scale, rows=None):
    """Bidirectional sliding-window attention over slots |u - t| <= R.

    "Prefilling-dLLM v2", Abstract and Table 3: the layers that do not route use
    a bidirectional sliding window (radius 1280). Reading: slot space, every slot
    (content or mask) is an ordinary token, clipped at the ends.

    q [B,Hq,L,d], k, v [B,Hkv,L,d]; rows: slots to compute (default all)
    -> o [B,Hq,n,d], lse [B,Hq,n].
    """
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = np.arange(L) if rows is None else np.asarray(rows)
    o = np.empty((B, Hq, len(rows), d))
    lse = np.empty((B, Hq, len(rows)))
    for b in range(B):
        for t, u in enumerate(rows):
            lo, hi = max(0, int(u) - R), min(L - 1, int(u) + R)
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                a = scale * q[b, hs, u] @ k[b, g, lo: hi + 1].T
                o[b, hs, t] = softmax(a, axis=-1) @ v[b, g, lo: hi + 1]
                lse[b, hs, t] = logsumexp(a, axis=-1)
    return o, lse
