"""lcr_routed_attention_noalloc (callers that cannot allocate) against
lcr_routed_attention, through the C ABI: two calls in a row, the second on a
smaller input, each equal bit for bit to the workspace call on the same inputs
(the same kernels run with their partials in the library's static scratch
instead of a caller workspace). A plan whose workspace exceeds the scratch is
rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import learned_chunk_routed_amd as lcr
from learned_chunk_routed_amd import _lib

pytestmark = pytest.mark.gpu

SL, CT = 64, 63


def _inputs(B, Hq, Hkv, N, d, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    L = N * SL
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).cuda()
    return dict(q=mk(B, Hq, L, d), k=mk(B, Hkv, L, d), v=mk(B, Hkv, L, d), x=mk(B, L, 64),
                A=(0.02 * torch.randn(64, 16, generator=g)).to(torch.bfloat16).cuda(),
                Bm=(0.02 * torch.randn(16, Hq * d, generator=g)).to(torch.bfloat16).cuda())


def _noalloc(t, idx, zsel, K, R, scale, q0, nq, out, lse):
    lib = _lib.load()
    B, Hq, L, d = t["q"].shape
    dims = lcr.make_dims(B, Hq, t["k"].shape[1], L // SL, d, t["q"].dtype)
    return lib.lcr_routed_attention_noalloc(
        dims, t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), idx.data_ptr(), zsel.data_ptr(), K, R,
        ctypes.c_float(scale), q0, nq, out.data_ptr(), lse.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _case(t, K, R, q0, nq, label):
    B, Hq, L, d = t["q"].shape
    Hkv, N = t["k"].shape[1], L // SL
    scale = 1.0 / np.sqrt(d)
    dims = lcr.make_dims(B, Hq, Hkv, N, d, t["q"].dtype)
    ws = lcr.workspace_bytes(2, dims, 0, 0, K, nq, R)
    print(f"[case] noalloc {label}: B={B} Hq={Hq} Hkv={Hkv} N={N} K={K} R={R} q0={q0} nq={nq} workspace={ws}",
          flush=True)
    assert 0 < ws <= _lib.LCR_NOALLOC_SCRATCH_BYTES, "the case must use the static scratch"
    s, H = lcr.chunk_summary(t["q"], t["k"], scale)
    idx, zsel = lcr.route_score_topk(t["q"], t["x"], t["A"], t["Bm"], s, H, Hkv=Hkv, K=K, radius=R, scale=scale,
                                     q0=q0, nq=nq)
    ref, ref_lse = lcr.routed_attention(t["q"], t["k"], t["v"], idx, zsel, radius=R, scale=scale, q0=q0, nq=nq,
                                        want_lse=True)
    out = torch.zeros_like(t["q"])
    lse = torch.empty((B, Hq, nq), dtype=torch.float32, device="cuda")
    rc = _noalloc(t, idx, zsel, K, R, scale, q0, nq, out, lse)
    torch.cuda.synchronize()
    assert rc == _lib.LCR_OK, _lib.status_string(rc)
    assert torch.equal(out, ref), f"{label}: output differs from the workspace call"
    assert torch.equal(lse, ref_lse), f"{label}: lse differs from the workspace call"
    assert bool(torch.isfinite(lse).all())
    return ws


def test_noalloc_matches_workspace_call_twice():
    t = _inputs(1, 28, 4, 256, 128, seed=3)
    T = 256 * CT
    big = _case(t, 32, 256, T - 32, 32, "decode block of 32 queries")
    small = _case(t, 16, 128, T - 600, 6, "6 queries, smaller K and radius")
    assert small < big
