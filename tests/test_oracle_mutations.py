"""Planted mistakes in the oracle must each make at least one pin fail (CPU only).

Each mutation replaces one function of the oracle module with a plausible wrong
version (a dropped term, a wrong sign, a wrong index or radius, a transposed
split, a wrong reduction). The pins of oracle_pins.py are then run; the test
passes only if at least one of them fails under the mutation.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import backward as OB
from oracle import route as O

SL, CT = 64, 63
_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}
_orig_b = {name: getattr(OB, name) for name in dir(OB) if not name.startswith("__")}


def _scores_entropy_plus(qt, s, H, beta, scale):
    return scale * np.einsum("bhnd,bhcd->bhnc", qt, s) + beta * H[:, :, None, :]


def _scores_no_entropy(qt, s, H, beta, scale):
    return scale * np.einsum("bhnd,bhcd->bhnc", qt, s)


def _scores_no_scale(qt, s, H, beta, scale):
    return np.einsum("bhnd,bhcd->bhnc", qt, s) - beta * H[:, :, None, :]


def _residual_dropped(q_rows, x_rows, A, Bm):
    return q_rows.copy()


def _residual_head_split(q_rows, x_rows, A, Bm):
    B, Hq, n, d = q_rows.shape
    res = (x_rows @ A) @ Bm
    return q_rows + res.reshape(B, n, d, Hq).transpose(0, 3, 1, 2)


def _window_short(i, R, T):
    return max(0, int(i) - R + 1), min(T - 1, int(i) + R - 1)


def _cand_own_chunk_only(queries, R, N):
    q = np.asarray(queries)
    return np.arange(N)[None, :] != (q // CT)[:, None]


def _cand_partial_overlap(queries, R, N):
    i = np.asarray(queries)[:, None]
    first = CT * np.arange(N)[None, :]
    return (first < i - R) | (first > i + R)


def _slot_identity(i):
    return np.asarray(i, dtype=np.int64)


def _zsel_group_max(z, idx, G):
    zh = np.repeat(O.group_max(z, G), G, axis=1)
    return _orig["gather_zsel"](zh, idx, G)


def _topk_larger_index_wins(zhat, cand, K):
    flipped = zhat[..., ::-1]
    idx, margin = _orig["select_topk"](flipped, cand[:, ::-1], K)
    N = zhat.shape[-1]
    idx = np.where(idx >= 0, N - 1 - idx, -1)
    idx = np.where(idx >= 0, idx, np.iinfo(np.int64).max)
    idx = np.sort(idx, axis=-1)
    return np.where(idx == np.iinfo(np.int64).max, -1, idx), margin


def _topk_one_short(zhat, cand, K):
    idx, margin = _orig["select_topk"](zhat, cand, max(K - 1, 0))
    pad = np.full(idx.shape[:-1] + (K - idx.shape[-1],), -1, dtype=idx.dtype)
    return np.concatenate([idx, pad], axis=-1), margin


def _margin_next_pair(zhat, cand, K):
    idx, margin = _orig["select_topk"](zhat, cand, K)
    _, m2 = _orig["select_topk"](zhat, cand, K + 1)
    return idx, np.where(np.isfinite(margin), m2, margin)


def _margin_scaled(zhat, cand, K):
    idx, margin = _orig["select_topk"](zhat, cand, K)
    return idx, margin * 1e6


def _margin_zero_when_few(zhat, cand, K):
    idx, margin = _orig["select_topk"](zhat, cand, K)
    return idx, np.where(np.isfinite(margin), margin, 0.0)


def _group_mean(z, G):
    B, Hq, n, N = z.shape
    return z.reshape(B, Hq // G, G, n, N).mean(axis=2)


def _group_first_head(z, G):
    B, Hq, n, N = z.shape
    return z.reshape(B, Hq // G, G, n, N)[:, :, 0]


def _summary_all_slots(q_mask, k, scale):
    B, Hq, N, d = q_mask.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    kc = k.reshape(B, Hkv, N, SL, d)
    s = np.empty((B, Hq, N, d))
    H = np.empty((B, Hq, N))
    for h in range(Hq):
        a = O.softmax(scale * np.einsum("bnd,bnjd->bnj", q_mask[:, h], kc[:, h // G]), axis=-1)
        s[:, h] = np.einsum("bnj,bnjd->bnd", a, kc[:, h // G])
        H[:, h] = O.entropy(a, axis=-1)
    return s, H


def _summary_first_head_query(q_mask, k, scale):
    B, Hq, N, d = q_mask.shape
    G = Hq // k.shape[1]
    qm = np.repeat(q_mask[:, ::G], G, axis=1)
    return _orig["chunk_summary_from_mask"](qm, k, scale)


def _entropy_log2(p, axis=-1):
    return _orig["entropy"](p, axis=axis) / np.log(2.0)


def _chunk_attention_uniform(qh, kc, vc, scale):
    return np.broadcast_to(vc.mean(axis=1)[None], (qh.shape[0],) + vc.mean(axis=1).shape).copy()


def _partition_separate(a, zc):
    Pu, _, lse = _orig["partition"](a, np.full_like(zc, -np.inf)) if zc.shape[1] else _orig["partition"](a, zc)
    if zc.shape[1] == 0:
        return Pu, zc * 0, lse
    Pc = np.exp(zc - zc.max(1, keepdims=True))
    Pc /= Pc.sum(1, keepdims=True)
    return Pu / 2, Pc / 2, lse


def _partition_no_window(a, zc):
    if zc.shape[1] == 0:
        return _orig["partition"](a, zc)
    Pu, Pc, lse = _orig["partition"](np.full_like(a, -np.inf), zc)
    return Pu * 0, Pc, lse


def _swa_exclusive(q, k, v, R, scale, rows=None):
    return _orig["swa_attention"](q, k, v, max(R - 1, 0), scale, rows) if R > 0 else \
        _orig["swa_attention"](q, k, v, R, scale, rows)


def _swa_wrong_group(q, k, v, R, scale, rows=None):
    Hq, Hkv = q.shape[1], k.shape[1]
    kk = np.stack([k[:, h % Hkv] for h in range(Hq)], axis=1)
    vv = np.stack([v[:, h % Hkv] for h in range(Hq)], axis=1)
    return _orig["swa_attention"](q, kk, vv, R, scale, rows)


MUTATIONS = {
    "entropy sign flipped": ("route_scores", _scores_entropy_plus),
    "entropy term dropped": ("route_scores", _scores_no_entropy),
    "score scale dropped": ("route_scores", _scores_no_scale),
    "residual dropped": ("routing_query", _residual_dropped),
    "residual split over heads transposed": ("routing_query", _residual_head_split),
    "window radius one short": ("window_bounds", _window_short),
    "only the own chunk excluded from candidates": ("candidate_mask", _cand_own_chunk_only),
    "partially overlapping chunks allowed": ("candidate_mask", _cand_partial_overlap),
    "slot map without mask slots": ("slot_of", _slot_identity),
    "chunk logit uses the group maximum": ("gather_zsel", _zsel_group_max),
    "ties go to the larger index": ("select_topk", _topk_larger_index_wins),
    "one chunk short": ("select_topk", _topk_one_short),
    "margin taken one rank too deep": ("select_topk", _margin_next_pair),
    "margin scaled": ("select_topk", _margin_scaled),
    "margin zero instead of +inf with few candidates": ("select_topk", _margin_zero_when_few),
    "group mean instead of maximum": ("group_max", _group_mean),
    "group uses its first head only": ("group_max", _group_first_head),
    "pooling includes the mask slot": ("chunk_summary_from_mask", _summary_all_slots),
    "summary per KV head from the first head": ("chunk_summary_from_mask", _summary_first_head_query),
    "entropy in bits": ("entropy", _entropy_log2),
    "intra-chunk softmax replaced by a mean": ("chunk_attention", _chunk_attention_uniform),
    "window and chunks normalised separately": ("partition", _partition_separate),
    "window dropped from the partition": ("partition", _partition_no_window),
    "SWA radius exclusive": ("swa_attention", _swa_exclusive),
    "SWA heads mapped to the wrong KV head": ("swa_attention", _swa_wrong_group),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # an assertion or a crash both count as detection
            caught.append(f"{pin.__name__}: {type(e).__name__}")
            break
    assert caught, f"no pin detects the planted mistake: {name}"


# ----------------------------------------------------------------------------- backward mutations (module OB)

def _softmax_bwd_no_mean(p, g, axis=-1):
    return p * g


def _summary_bwd_entropy_sign(q_mask, k, scale, ds, dH):
    return _orig_b["chunk_summary_backward"](q_mask, k, scale, ds, -dH)


def _summary_bwd_no_key_pooling_term(q_mask, k, scale, ds, dH):
    dq, dk = _orig_b["chunk_summary_backward"](q_mask, k, scale, ds, dH)
    dq0, dk0 = _orig_b["chunk_summary_backward"](q_mask, k, scale, ds * 0, dH)
    return dq, dk0 + 0.5 * (dk - dk0)


def _score_bwd_residual_dropped(*a):
    dqt, dx, dA, dBm, ds, dH = _orig_b["route_score_backward"](*a)
    return dqt, dx * 0, dA * 0, dBm * 0, ds, dH


def _score_bwd_entropy_sign(*a):
    dqt, dx, dA, dBm, ds, dH = _orig_b["route_score_backward"](*a)
    return dqt, dx, dA, dBm, ds, -dH


def _attn_bwd_no_dzsel(*a):
    dq, dk, dv, dz = _orig_b["routed_attention_backward"](*a)
    return dq, dk, dv, dz * 0


def _bwd_softmax_wrong_axis(x, axis=-1):
    return _orig["softmax"](x, axis=0 if x.ndim > 1 and x.shape[0] > 1 else axis)


BWD_MUTATIONS = {
    "softmax backward without its mean term": ("_softmax_backward", _softmax_bwd_no_mean),
    "pooling entropy gradient sign flipped": ("chunk_summary_backward", _summary_bwd_entropy_sign),
    "pooling key gradient halved": ("chunk_summary_backward", _summary_bwd_no_key_pooling_term),
    "no gradient into the low-rank residual": ("route_score_backward", _score_bwd_residual_dropped),
    "scoring entropy gradient sign flipped": ("route_score_backward", _score_bwd_entropy_sign),
    "no gradient into the chunk logits": ("routed_attention_backward", _attn_bwd_no_dzsel),
    "backward recomputes the intra-chunk softmax over the wrong axis": ("softmax", _bwd_softmax_wrong_axis),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_backward_mutation_is_caught(name, monkeypatch):
    attr, fn = BWD_MUTATIONS[name]
    monkeypatch.setattr(OB, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
            break
    assert caught, f"no pin detects the planted mistake: {name}"
