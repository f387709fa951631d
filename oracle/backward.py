"""Gradients of the route layer in float64, with chunk membership held fixed.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests and the
benchmark's CPU-baseline leg, never by the product path.

"The 172x Speedup Has an Evidence Budget" (section "How learned routing controls
what the model can read"): which chunks are chosen is not differentiable; the
router is trained through the masses the selected chunks receive. So idx is a
constant here, and gradients reach the router only through the selected chunk
logits zsel, which depend on the routing query and on the summaries.

Each function applies the chain rule to the forward of oracle.route step by
step, in the forward's order reversed. The one identity used throughout is the
softmax backward: for p = softmax(x) and an upstream gradient g on p,
dL/dx = p * (g - <p, g>).

Pins: tests/oracle_pins.py checks every function here against central finite
differences of the forward oracle, and the window-only case against torch's
float64 attention autograd.
"""
import numpy as np

from .route import SLOTS, CONTENT, slot_of, softmax, window_bounds, partition


def _softmax_backward(p, g, axis=-1):
    """dL/dx for p = softmax(x, axis) given g = dL/dp."""
    return p * (g - np.sum(p * g, axis=axis, keepdims=True))


# ----------------------------------------------------------------------------- steps 6-8: attention

def routed_attention_backward(q_rows, k, v, idx, zsel, R, scale, queries, do_rows):
    """Gradients of routed_attention for an upstream gradient do_rows on o.

    Forward ("Prefilling-dLLM v2", Figure 3 caption): one partition P over the
    window logits a_u = scale q.k_u and the selected chunk logits z_c; inside a
    chunk, pi = softmax(scale q.k_cj) over its 63 content keys and u_bar_c =
    sum_j pi_j v_cj; o = sum_u P_u v_u + sum_c P_c u_bar_c.

    q_rows [B,Hq,n,d]; k, v [B,Hkv,L,d]; idx [B,Hkv,n,K]; zsel [B,Hq,n,K];
    do_rows [B,Hq,n,d] -> dq_rows [B,Hq,n,d], dk, dv [B,Hkv,L,d],
    dzsel [B,Hq,n,K] (zero where idx is -1).
    """
    B, Hq, n, d = q_rows.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    N = k.shape[2] // SLOTS
    T = N * CONTENT
    jj = np.arange(CONTENT)
    dq = np.zeros((B, Hq, n, d))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dz = np.zeros(zsel.shape)
    for b in range(B):
        for t, i in enumerate(np.asarray(queries)):
            lo, hi = window_bounds(i, R, T)
            ws = slot_of(np.arange(lo, hi + 1))
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                qh = q_rows[b, hs, t]                                   # [G,d]
                dO = do_rows[b, hs, t]                                  # [G,d]
                kw, vw = k[b, g, ws], v[b, g, ws]                       # [W,d]
                sel = idx[b, g, t]
                sel = sel[sel >= 0]
                m = len(sel)
                cs = sel[:, None] * SLOTS + jj[None, :]                 # [m,63]
                kc, vc = k[b, g, cs], v[b, g, cs]                       # [m,63,d]
                # forward, kept for the backward (chunk-major arrays [m,G,...])
                a = scale * qh @ kw.T                                   # [G,W]
                zc = zsel[b, hs, t, :m]                                 # [G,m]
                Pu, Pc, _ = partition(a, zc)
                pi = softmax(scale * (qh @ kc.transpose(0, 2, 1)), axis=-1)   # [m,G,63]
                ubar = pi @ vc                                          # [m,G,d]
                # o = Pu vw + sum_c Pc ubar_c
                gPu = dO @ vw.T                                         # dL/dPu  [G,W]
                gPc = np.sum(dO[None] * ubar, axis=-1).T                # dL/dPc  [G,m]
                gubar = Pc.T[:, :, None] * dO[None]                     # dL/dubar [m,G,d]
                dv[b, g, ws] += Pu.T @ dO
                # partition: one softmax over [a, zc]
                gx = _softmax_backward(np.concatenate([Pu, Pc], axis=1),
                                       np.concatenate([gPu, gPc], axis=1))
                da, dzc = gx[:, : a.shape[1]], gx[:, a.shape[1]:]
                dz[b, hs, t, :m] = dzc
                dq[b, hs, t] += scale * da @ kw
                dk[b, g, ws] += scale * da.T @ qh
                # chunk attention: ubar = pi vc, pi = softmax(scale q kc^T)
                dv[b, g, cs] += pi.transpose(0, 2, 1) @ gubar
                gpi = gubar @ vc.transpose(0, 2, 1)                     # [m,G,63]
                dl = _softmax_backward(pi, gpi)
                dq[b, hs, t] += scale * np.sum(dl @ kc, axis=0)
                dk[b, g, cs] += scale * dl.transpose(0, 2, 1) @ qh
    return dq, dk, dv, dz


# ----------------------------------------------------------------------------- steps 2, 4, 5: scoring

def route_score_backward(q_rows, x_rows, A, Bm, s, H, idx, dzsel, beta, scale):
    """Gradients of zsel = gather(scale q~.s - beta H) with q~ = q + (x A) Bm.

    "Prefilling-dLLM v2", Figure 3 caption (residual-augmented query scoring the
    summaries); "The 172x Speedup...": similarity and pooling entropy rank the
    chunks. The gather by the fixed idx routes each dzsel entry to the score of
    one (head, chunk); the group maximum and the top-K choice only decide idx.

    q_rows [B,Hq,n,d], x_rows [B,n,D], A [D,r], Bm [r,Hq*d], s [B,Hq,N,d],
    H [B,Hq,N], idx [B,Hkv,n,K], dzsel [B,Hq,n,K]
    -> dq_rows [B,Hq,n,d], dx_rows [B,n,D], dA [D,r], dBm [r,Hq*d],
       ds [B,Hq,N,d], dH [B,Hq,N].
    """
    B, Hq, n, d = q_rows.shape
    Hkv = idx.shape[1]
    G = Hq // Hkv
    N = s.shape[2]
    u = x_rows @ A                                                      # [B,n,r]
    qt = q_rows + (u @ Bm).reshape(B, n, Hq, d).transpose(0, 2, 1, 3)
    # scatter dzsel onto the full score grid dz [B,Hq,n,N] (entries with idx -1 are dropped)
    dzfull = np.zeros((B, Hq, n, N))
    idx_h = np.repeat(idx, G, axis=1)
    bb, hh, tt, kk = np.nonzero(idx_h >= 0)
    np.add.at(dzfull, (bb, hh, tt, idx_h[bb, hh, tt, kk]), dzsel[bb, hh, tt, kk])
    # z = scale q~ . s - beta H
    dqt = scale * (dzfull @ s)                                          # [B,Hq,n,d]
    ds = scale * (np.swapaxes(dzfull, -1, -2) @ qt)                     # [B,Hq,N,d]
    dH = -beta * dzfull.sum(axis=2)
    # q~ = q + u Bm (head h takes columns h*d .. h*d+d-1)
    dres = dqt.transpose(0, 2, 1, 3).reshape(B, n, Hq * d)            # [B,n,Hq*d]
    r = A.shape[1]
    dBm = u.reshape(B * n, r).T @ dres.reshape(B * n, Hq * d)
    du = dres @ Bm.T                                                    # [B,n,r]
    dA = x_rows.reshape(B * n, -1).T @ du.reshape(B * n, r)
    dx = du @ A.T
    return dqt, dx, dA, dBm, ds, dH


# ----------------------------------------------------------------------------- step 1: summaries

def chunk_summary_backward(q_mask, k, scale, ds, dH):
    """Gradients of the mask-query pooling (chunk_summary_from_mask).

    "Prefilling-dLLM v2", Figure 3 caption: alpha = softmax over the chunk's 63
    content keys of scale q_mask.k_j, s = sum_j alpha_j k_j; "The 172x
    Speedup...": H = -sum_j alpha_j ln alpha_j.

    q_mask [B,Hq,N,d], k [B,Hkv,L,d], ds [B,Hq,N,d], dH [B,Hq,N]
    -> dq_mask [B,Hq,N,d], dk [B,Hkv,L,d] (content rows only; mask rows zero).
    """
    B, Hq, N, d = q_mask.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    kc = k.reshape(B, Hkv, N, SLOTS, d)[:, :, :, :CONTENT, :]
    dq = np.zeros(q_mask.shape)
    dkc = np.zeros(kc.shape)
    for h in range(Hq):
        g = h // G
        lam = scale * np.einsum("bnd,bnjd->bnj", q_mask[:, h], kc[:, g])
        alpha = softmax(lam, axis=-1)                                   # [B,N,63]
        with np.errstate(divide="ignore"):
            logal = np.where(alpha > 0, np.log(np.where(alpha > 0, alpha, 1.0)), 0.0)
        # s = sum alpha k  ->  dL/dalpha_j = ds . k_j ;  H = -sum alpha ln alpha -> -(ln alpha_j + 1) dH
        galpha = np.einsum("bnd,bnjd->bnj", ds[:, h], kc[:, g]) - (logal + 1.0) * dH[:, h, :, None]
        dlam = _softmax_backward(alpha, galpha)
        dq[:, h] = scale * np.einsum("bnj,bnjd->bnd", dlam, kc[:, g])
        dkc[:, g] += alpha[..., None] * ds[:, h][:, :, None, :]
        dkc[:, g] += scale * dlam[..., None] * q_mask[:, h][:, :, None, :]
    dk = np.zeros(k.shape)
    dk.reshape(B, Hkv, N, SLOTS, d)[:, :, :, :CONTENT, :] = dkc
    return dq, dk


# ----------------------------------------------------------------------------- whole layer

def route_layer_backward(q, k, v, x, A, Bm, idx, dO_rows, *, R, beta, scale, queries):
    """Gradients of the route layer for queries `queries` with idx held fixed.

    q [B,Hq,L,d], k, v [B,Hkv,L,d], x [B,L,D]; idx [B,Hkv,n,K] (the forward's
    choice); dO_rows [B,Hq,n,d] upstream gradient on o at slot(queries).
    Returns dict dq [B,Hq,L,d] (query rows from attention and scoring, mask rows
    from the summaries), dk, dv, dx [B,L,D], dA, dBm, and the intermediates
    dzsel, ds, dH.
    """
    from .route import chunk_summary_from_mask, routing_query, route_scores, gather_zsel
    B, Hq, L, d = q.shape
    N = L // SLOTS
    G = Hq // k.shape[1]
    slots = slot_of(queries)
    q_rows, x_rows = q[:, :, slots], x[:, slots]
    q_mask = q.reshape(B, Hq, N, SLOTS, d)[:, :, :, SLOTS - 1, :]
    s, H = chunk_summary_from_mask(q_mask, k, scale)
    z = route_scores(routing_query(q_rows, x_rows, A, Bm), s, H, beta, scale)
    zsel = gather_zsel(z, idx, G)
    dq_a, dk, dv, dzsel = routed_attention_backward(q_rows, k, v, idx, zsel, R, scale, queries, dO_rows)
    dq_s, dx_rows, dA, dBm, ds, dH = route_score_backward(q_rows, x_rows, A, Bm, s, H, idx, dzsel, beta, scale)
    dq_m, dk_m = chunk_summary_backward(q_mask, k, scale, ds, dH)
    dq = np.zeros(q.shape)
    dq[:, :, slots] += dq_a + dq_s
    dq.reshape(B, Hq, N, SLOTS, d)[:, :, :, SLOTS - 1, :] += dq_m
    dx = np.zeros(x.shape)
    dx[:, slots] += dx_rows
    return dict(dq=dq, dk=dk + dk_m, dv=dv, dx=dx, dA=dA, dBm=dBm, dzsel=dzsel, ds=ds, dH=dH)
