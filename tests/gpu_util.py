"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing the HIP results with the fp64 oracle under the parity bar:
 - top-K sets bit-exact wherever the oracle's K-th/(K+1)-th margin exceeds 1e-3;
   elsewhere the GPU set must be a valid top-K within that margin;
 - outputs within 2e-2 max-abs for bf16 inputs, 1e-5 for float32 inputs.
"""
import numpy as np
import torch

from lcr_inputs import as_f64
from oracle import route as O

GATE = 1e-3
OUT_TOL = {"bf16": 2e-2, "fp32": 1e-5}
LSE_TOL = {"bf16": 2e-3, "fp32": 1e-5}
Z_TOL = {"bf16": 5e-5, "fp32": 2e-5}


def to_dev(a: np.ndarray, device="cuda"):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_selection(idx_gpu, ref, K, label):
    """idx_gpu [B,Hkv,n,K] int; ref: oracle dict (idx, margin, zhat, cand) for the same rows.
    Returns a boolean mask [B,Hkv,n] of rows whose sets equal the oracle's."""
    idx_o = ref["idx"]
    same = np.all(idx_gpu == idx_o, axis=-1)
    gated = ref["margin"] > GATE
    bad = gated & ~same
    assert not bad.any(), (f"{label}: {int(bad.sum())} of {int(gated.sum())} gated rows differ, e.g. "
                           f"{np.argwhere(bad)[:3].tolist()}")
    # every differing (ungated) row must still be a valid top-K
    for (b, g, t) in np.argwhere(~same):
        sel = idx_gpu[b, g, t]
        chosen = sel[sel >= 0]
        cands = np.nonzero(ref["cand"][t])[0]
        m = min(K, len(cands))
        assert len(chosen) == m and np.all(np.diff(chosen) > 0), f"{label}: malformed row {(b, g, t)}"
        assert np.all(np.isin(chosen, cands)), f"{label}: non-candidate chosen at {(b, g, t)}"
        zh = ref["zhat"][b, g, t]
        kth = np.sort(zh[cands])[::-1][m - 1]
        assert zh[chosen].min() >= kth - GATE, f"{label}: row {(b, g, t)} is not a top-K within the margin"
    return same


def oracle_attention_for(q_rows, k, v, idx, zsel, R, scale, queries):
    return O.routed_attention(q_rows, k, v, idx.astype(np.int64), zsel, R, scale, queries)


def max_err(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
