"""Python binding of the C ABI: argument marshalling only.

Every step of the route layer runs in the HIP kernels of liblcr.so; this module
checks tensors (device, dtype, contiguity, shapes), allocates outputs and
workspace through PyTorch and passes raw device pointers plus the current HIP
stream. There is no CPU or PyTorch fallback: a missing library raises.

Shapes follow include/lcr.h: q [B,Hq,L,d], k and v [B,Hkv,L,d] with L = 64*N,
x [B,L,D], A [D,r], Bm [r,Hq*d]; content query i lives in slot
64*(i//63) + i%63.
"""
import math

import torch

from . import _lib
from ._lib import Dims, check

SLOTS, CONTENT = 64, 63

_DTYPES = {torch.bfloat16: _lib.LCR_BF16, torch.float32: _lib.LCR_F32}


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check(t, name, device, dtype=None, shape=None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda and t.device == device, f"{name} must be on {device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def make_dims(B, Hq, Hkv, N, d, dtype) -> Dims:
    _need(dtype in _DTYPES, f"unsupported dtype {dtype}")
    return Dims(B, Hq, Hkv, N, d, _DTYPES[dtype])


def _dims_from(q, Hkv):
    _need(q.dim() == 4, "q must be [B,Hq,L,d]")
    B, Hq, L, d = q.shape
    _need(L % SLOTS == 0, f"L={L} must be a multiple of {SLOTS}")
    return make_dims(B, Hq, Hkv, L // SLOTS, d, q.dtype)


def default_scale(d):
    return 1.0 / math.sqrt(d)


def workspace_bytes(op, dims: Dims, D=0, r=0, K=0, nq=0, radius=0) -> int:
    return int(_lib.load().lcr_workspace_bytes(op, dims, D, r, K, radius, nq))


def set_wait_limit(polls: int) -> int:
    """Polls before a wait on an LDS counter inside the pooled kernels gives up
    (polls < 1 restores the default); a wave that gives up writes NaN rows.
    Process-wide; returns the previous setting."""
    return int(_lib.load().lcr_set_wait_limit(int(polls)))


def set_tile_order(reversed: bool) -> int:
    """Walk the tiles of the tiled kernels in reversed order (a test hook: outputs are
    bit for bit the same either way). Process-wide; returns the previous setting."""
    return int(_lib.load().lcr_set_tile_order(1 if reversed else 0))


def _workspace(nbytes, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def chunk_summary(q, k, scale=None, s=None, H=None, chunks=None):
    """Summary keys s [B,Hq,N,d] and pooling entropies H [B,Hq,N], float32.

    chunks=(c0, nc) refreshes only chunks c0 .. c0 + nc - 1 of the given s and H in
    place (after their keys changed); the other rows are left as they are."""
    lib = _lib.load()
    dev = q.device
    dims = _dims_from(q, k.shape[1])
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (dims.B, dims.Hkv, dims.N * SLOTS, dims.d))
    scale = default_scale(dims.d) if scale is None else float(scale)
    if chunks is not None and (s is None or H is None):
        raise ValueError("a refresh of some chunks updates existing s and H: pass both")
    if s is None:
        s = torch.empty((dims.B, dims.Hq, dims.N, dims.d), dtype=torch.float32, device=dev)
    if H is None:
        H = torch.empty((dims.B, dims.Hq, dims.N), dtype=torch.float32, device=dev)
    _check(s, "s", dev, torch.float32, (dims.B, dims.Hq, dims.N, dims.d))
    _check(H, "H", dev, torch.float32, (dims.B, dims.Hq, dims.N))
    if chunks is None:
        check(lib.lcr_chunk_summary(dims, q.data_ptr(), k.data_ptr(), scale, s.data_ptr(), H.data_ptr(),
                                    _stream(dev)), "lcr_chunk_summary")
    else:
        c0, nc = (int(c) for c in chunks)
        check(lib.lcr_chunk_summary_range(dims, q.data_ptr(), k.data_ptr(), scale, c0, nc, s.data_ptr(),
                                          H.data_ptr(), _stream(dev)), "lcr_chunk_summary_range")
    return s, H


def chunk_summary_mean(k, Hq, s=None, H=None):
    """Mean summaries (uniform pooling): s [B,Hq,N,d] = the mean content key of each chunk
    for every head of its group, H [B,Hq,N] = ln 63; float32."""
    lib = _lib.load()
    dev = k.device
    B, Hkv, L, d = k.shape
    N = L // SLOTS
    dims = make_dims(B, Hq, Hkv, N, d, k.dtype)
    _check(k, "k", dev, k.dtype, (B, Hkv, N * SLOTS, d))
    if s is None:
        s = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    if H is None:
        H = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    _check(s, "s", dev, torch.float32, (B, Hq, N, d))
    _check(H, "H", dev, torch.float32, (B, Hq, N))
    check(lib.lcr_chunk_summary_mean(dims, k.data_ptr(), s.data_ptr(), H.data_ptr(), _stream(dev)),
          "lcr_chunk_summary_mean")
    return s, H


def route_score_topk(q, x, A, Bm, s, H, *, Hkv, K, radius, beta=0.0, scale=None, q0=0, nq=None,
                     idx=None, zsel=None, ws=None):
    """Chosen remote chunks idx [B,Hkv,nq,K] (int32, ascending, -1 padded) and the
    per-head scores of the chosen chunks zsel [B,Hq,nq,K] (float32)."""
    lib = _lib.load()
    dev = q.device
    dims = _dims_from(q, Hkv)
    B, Hq, N, d = dims.B, dims.Hq, dims.N, dims.d
    T = N * CONTENT
    nq = T - q0 if nq is None else nq
    _check(q, "q", dev)
    _need(x.dim() == 3 and x.shape[:2] == (B, N * SLOTS), "x must be [B,L,D]")
    D = x.shape[2]
    _need(A.dim() == 2 and A.shape[0] == D, "A must be [D,r]")
    r = A.shape[1]
    _check(x, "x", dev, q.dtype)
    _check(A, "A", dev, q.dtype)
    _check(Bm, "Bm", dev, q.dtype, (r, Hq * d))
    _check(s, "s", dev, torch.float32, (B, Hq, N, d))
    _check(H, "H", dev, torch.float32, (B, Hq, N))
    scale = default_scale(d) if scale is None else float(scale)
    if idx is None:
        idx = torch.empty((B, Hkv, nq, K), dtype=torch.int32, device=dev)
    if zsel is None:
        zsel = torch.empty((B, Hq, nq, K), dtype=torch.float32, device=dev)
    _check(idx, "idx", dev, torch.int32, (B, Hkv, nq, K))
    _check(zsel, "zsel", dev, torch.float32, (B, Hq, nq, K))
    nbytes = workspace_bytes(_lib.OP_ROUTE_SCORE_TOPK, dims, D, r, K, nq)
    w = _workspace(nbytes, dev, ws)
    check(lib.lcr_route_score_topk(dims, q.data_ptr(), x.data_ptr(), A.data_ptr(), Bm.data_ptr(), D, r,
                                   s.data_ptr(), H.data_ptr(), float(beta), scale, K, radius, q0, nq,
                                   idx.data_ptr(), zsel.data_ptr(), None if w is None else w.data_ptr(),
                                   nbytes, _stream(dev)), "lcr_route_score_topk")
    return idx, zsel


def routed_attention(q, k, v, idx, zsel, *, radius, scale=None, q0=0, nq=None, out=None, lse=None,
                     want_lse=False, ws=None):
    """Route-layer output o [B,Hq,L,d] (rows of the queried content positions written;
    other rows of a freshly allocated `out` are zero) and optionally lse [B,Hq,nq]."""
    lib = _lib.load()
    dev = q.device
    dims = _dims_from(q, k.shape[1])
    B, Hq, Hkv, N, d = dims.B, dims.Hq, dims.Hkv, dims.N, dims.d
    T = N * CONTENT
    nq = T - q0 if nq is None else nq
    K = idx.shape[-1]
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (B, Hkv, N * SLOTS, d))
    _check(v, "v", dev, q.dtype, (B, Hkv, N * SLOTS, d))
    _check(idx, "idx", dev, torch.int32, (B, Hkv, nq, K))
    _check(zsel, "zsel", dev, torch.float32, (B, Hq, nq, K))
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.zeros_like(q)
    _check(out, "out", dev, q.dtype, tuple(q.shape))
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, nq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", dev, torch.float32, (B, Hq, nq))
    nbytes = workspace_bytes(_lib.OP_ROUTED_ATTENTION, dims, 0, 0, K, nq, radius)
    w = _workspace(nbytes, dev, ws)
    check(lib.lcr_routed_attention(dims, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                   zsel.data_ptr(), K, radius, scale, q0, nq, out.data_ptr(),
                                   None if lse is None else lse.data_ptr(), None if w is None else w.data_ptr(),
                                   nbytes, _stream(dev)), "lcr_routed_attention")
    return (out, lse) if (want_lse or lse is not None) else out


def routed_attention_backward(q, k, v, idx, zsel, o, lse, dO, *, radius, scale=None, q0=0, nq=None, ws=None):
    """Gradients of routed_attention with the chosen chunks fixed (bf16 inputs).

    o and lse are the forward's outputs; dO [B,Hq,L,d] bf16 (rows of the queried
    positions are read). Returns dq [B,Hq,L,d] (queried rows written, other rows
    zero), dk, dv [B,Hkv,L,d] and dzsel [B,Hq,nq,K], all float32."""
    lib = _lib.load()
    dev = q.device
    dims = _dims_from(q, k.shape[1])
    B, Hq, Hkv, N, d = dims.B, dims.Hq, dims.Hkv, dims.N, dims.d
    T = N * CONTENT
    nq = T - q0 if nq is None else nq
    K = idx.shape[-1]
    _need(q.dtype in (torch.bfloat16, torch.float32), "routed_attention_backward takes bfloat16 or float32 q, k, v, o, dO")
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (B, Hkv, N * SLOTS, d))
    _check(v, "v", dev, q.dtype, (B, Hkv, N * SLOTS, d))
    _check(o, "o", dev, q.dtype, tuple(q.shape))
    _check(dO, "dO", dev, q.dtype, tuple(q.shape))
    _check(idx, "idx", dev, torch.int32, (B, Hkv, nq, K))
    _check(zsel, "zsel", dev, torch.float32, (B, Hq, nq, K))
    _check(lse, "lse", dev, torch.float32, (B, Hq, nq))
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    dz = torch.empty((B, Hq, nq, K), dtype=torch.float32, device=dev)
    nbytes = workspace_bytes(_lib.OP_ROUTED_ATTENTION_BACKWARD, dims, 0, 0, K, nq, radius)
    w = _workspace(nbytes, dev, ws)
    check(lib.lcr_routed_attention_backward(dims, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                            zsel.data_ptr(), K, radius, scale, q0, nq, o.data_ptr(),
                                            lse.data_ptr(), dO.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                            dv.data_ptr(), dz.data_ptr() if K > 0 else None,
                                            None if w is None else w.data_ptr(), nbytes, _stream(dev)),
          "lcr_routed_attention_backward")
    return dq, dk, dv, dz


def route_score_backward(q, x, A, Bm, s, idx, dzsel, *, beta=0.0, scale=None, q0=0, nq=None, dq=None, ws=None):
    """Gradients of route_score_topk's chunk logits with the selection idx fixed.

    dzsel [B,Hq,nq,K] float32 is the upstream gradient (e.g. from
    routed_attention_backward). dq [B,Hq,L,d] float32 is accumulated into at the
    queried rows (allocated as zeros when not given). Returns a dict with dq,
    dx [B,L,D] (queried rows), dA [D,r], dBm [r,Hq*d], ds [B,Hq,N,d], dH [B,Hq,N],
    all float32."""
    lib = _lib.load()
    dev = q.device
    Hkv = idx.shape[1]
    dims = _dims_from(q, Hkv)
    B, Hq, N, d = dims.B, dims.Hq, dims.N, dims.d
    T = N * CONTENT
    nq = T - q0 if nq is None else nq
    K = idx.shape[-1]
    D, r = A.shape
    _check(q, "q", dev)
    _check(x, "x", dev, q.dtype, (B, N * SLOTS, D))
    _check(A, "A", dev, q.dtype, (D, r))
    _check(Bm, "Bm", dev, q.dtype, (r, Hq * d))
    _check(s, "s", dev, torch.float32, (B, Hq, N, d))
    _check(idx, "idx", dev, torch.int32, (B, Hkv, nq, K))
    _check(dzsel, "dzsel", dev, torch.float32, (B, Hq, nq, K))
    scale = default_scale(d) if scale is None else float(scale)
    if dq is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    _check(dq, "dq", dev, torch.float32, tuple(q.shape))
    out = dict(dq=dq, dx=torch.zeros((B, N * SLOTS, D), dtype=torch.float32, device=dev),
               dA=torch.empty((D, r), dtype=torch.float32, device=dev),
               dBm=torch.empty((r, Hq * d), dtype=torch.float32, device=dev),
               ds=torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev),
               dH=torch.empty((B, Hq, N), dtype=torch.float32, device=dev))
    nbytes = workspace_bytes(_lib.OP_ROUTE_SCORE_BACKWARD, dims, D, r, K, nq, 0)
    w = _workspace(nbytes, dev, ws)
    check(lib.lcr_route_score_backward(dims, q.data_ptr(), x.data_ptr(), A.data_ptr(), Bm.data_ptr(), D, r,
                                       s.data_ptr(), float(beta), scale, K, q0, nq,
                                       idx.data_ptr() if K > 0 else None, dzsel.data_ptr() if K > 0 else None,
                                       dq.data_ptr(), out["dx"].data_ptr(), out["dA"].data_ptr(),
                                       out["dBm"].data_ptr(), out["ds"].data_ptr(), out["dH"].data_ptr(),
                                       None if w is None else w.data_ptr(), nbytes, _stream(dev)),
          "lcr_route_score_backward")
    return out


def chunk_summary_backward(q, k, ds, dH, scale=None, dq=None, dk=None):
    """Gradients of chunk_summary for upstream ds [B,Hq,N,d], dH [B,Hq,N] (float32).
    Writes the mask-slot rows of dq and adds into the content rows of dk (both float32,
    allocated as zeros when not given); returns (dq, dk)."""
    lib = _lib.load()
    dev = q.device
    dims = _dims_from(q, k.shape[1])
    B, Hq, Hkv, N, d = dims.B, dims.Hq, dims.Hkv, dims.N, dims.d
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (B, Hkv, N * SLOTS, d))
    _check(ds, "ds", dev, torch.float32, (B, Hq, N, d))
    _check(dH, "dH", dev, torch.float32, (B, Hq, N))
    scale = default_scale(d) if scale is None else float(scale)
    if dq is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
    _check(dq, "dq", dev, torch.float32, tuple(q.shape))
    _check(dk, "dk", dev, torch.float32, tuple(k.shape))
    check(lib.lcr_chunk_summary_backward(dims, q.data_ptr(), k.data_ptr(), scale, ds.data_ptr(), dH.data_ptr(),
                                         dq.data_ptr(), dk.data_ptr(), _stream(dev)), "lcr_chunk_summary_backward")
    return dq, dk


def route_layer_backward(q, k, v, x, A, Bm, fwd, dO, *, radius, beta=0.0, scale=None, q0=0, nq=None):
    """Gradients of the whole route layer with the forward's selection held fixed.

    fwd is the dict route_layer returned (with want_lse=True: s, idx, zsel, o, lse);
    dO [B,Hq,L,d] (q's dtype) is the upstream gradient on o. Chains the attention, scoring
    and pooling backward calls; returns a dict with dq [B,Hq,L,d] (query rows from
    attention and scoring, mask rows from the pooling), dk, dv, dx, dA, dBm, and the
    intermediates dzsel, ds, dH (all float32)."""
    _need(fwd.get("lse") is not None, "route_layer_backward needs the forward's lse (route_layer(..., want_lse=True))")
    dq, dk, dv, dz = routed_attention_backward(q, k, v, fwd["idx"], fwd["zsel"], fwd["o"], fwd["lse"], dO,
                                               radius=radius, scale=scale, q0=q0, nq=nq)
    sc = route_score_backward(q, x, A, Bm, fwd["s"], fwd["idx"], dz, beta=beta, scale=scale, q0=q0, nq=nq, dq=dq)
    chunk_summary_backward(q, k, sc["ds"], sc["dH"], scale=scale, dq=dq, dk=dk)
    return dict(dq=dq, dk=dk, dv=dv, dx=sc["dx"], dA=sc["dA"], dBm=sc["dBm"], dzsel=dz, ds=sc["ds"], dH=sc["dH"])


def swa_attention(q, k, v, *, radius, scale=None, out=None, lse=None, want_lse=False):
    """Bidirectional sliding-window attention over slots |u - t| <= radius: o [B,Hq,L,d]."""
    lib = _lib.load()
    dev = q.device
    _need(q.dim() == 4 and k.dim() == 4, "q, k, v must be [B,H,L,d]")
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    _need(q.dtype in _DTYPES, f"unsupported dtype {q.dtype}")
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (B, Hkv, L, d))
    _check(v, "v", dev, q.dtype, (B, Hkv, L, d))
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dev, q.dtype, tuple(q.shape))
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", dev, torch.float32, (B, Hq, L))
    check(lib.lcr_swa_attention(B, Hq, Hkv, L, d, _DTYPES[q.dtype], q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                radius, scale, out.data_ptr(), None if lse is None else lse.data_ptr(),
                                _stream(dev)), "lcr_swa_attention")
    return (out, lse) if (want_lse or lse is not None) else out


def route_layer(q, k, v, x, A, Bm, *, K, radius, beta=0.0, scale=None, q0=0, nq=None, out=None,
                want_lse=False, s=None, H=None):
    """Whole route layer: summaries (unless s and H are given), scoring + top-K,
    routed attention. Returns a dict with s, H, idx, zsel, o (and lse)."""
    if s is None or H is None:
        s, H = chunk_summary(q, k, scale)
    idx, zsel = route_score_topk(q, x, A, Bm, s, H, Hkv=k.shape[1], K=K, radius=radius, beta=beta,
                                 scale=scale, q0=q0, nq=nq)
    res = routed_attention(q, k, v, idx, zsel, radius=radius, scale=scale, q0=q0, nq=nq, out=out,
                           want_lse=want_lse)
    o, lse = res if isinstance(res, tuple) else (res, None)
    return dict(s=s, H=H, idx=idx, zsel=zsel, o=o, lse=lse)
