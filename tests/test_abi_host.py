"""The C ABI on the host: the library loads, exports every declared entry point, and
rejects invalid arguments with the documented status codes before any launch
(CPU only: no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

from learned_chunk_routed_amd import _lib
from learned_chunk_routed_amd._lib import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcr.h")
P = ctypes.c_void_p(4096)          # a non-null pointer that is never dereferenced on the host
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("liblcr.so is not built (run python -m learned_chunk_routed_amd.build)")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(lcr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ["lcr_chunk_summary", "lcr_route_score_topk", "lcr_routed_attention", "lcr_swa_attention",
              "lcr_workspace_bytes", "lcr_status_string", "lcr_version"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (lcr_[a-z_]+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in declared_functions():
        assert hasattr(lib, n)
    assert set(_lib.SIGNATURES) == set(declared_functions())


def test_status_strings(lib):
    for code in [0, -1, -2, -3, -4, -5]:
        assert lib.lcr_status_string(code)
    assert lib.lcr_status_string(0) == b"ok"
    assert lib.lcr_version() >= 10000


def dims(**kw):
    base = dict(B=1, Hq=28, Hkv=4, N=256, d=128, dtype=1)
    base.update(kw)
    return Dims(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.LCR_ERR_DTYPE),
    (dict(B=0), _lib.LCR_ERR_ARG),
    (dict(Hq=27), _lib.LCR_ERR_ARG),
    (dict(N=0), _lib.LCR_ERR_ARG),
    (dict(d=96), _lib.LCR_ERR_UNSUPPORTED),
    (dict(Hq=36, Hkv=4), _lib.LCR_ERR_UNSUPPORTED),
    (dict(N=1 << 26), _lib.LCR_ERR_ARG),
])
def test_chunk_summary_rejects_bad_dims(lib, kw, code):
    assert lib.lcr_chunk_summary(dims(**kw), P, P, 0.1, P, P, NULL) == code


@pytest.mark.parametrize("c0,nc,code", [
    (-1, 1, _lib.LCR_ERR_ARG), (0, -1, _lib.LCR_ERR_ARG), (250, 7, _lib.LCR_ERR_ARG), (256, 1, _lib.LCR_ERR_ARG),
    (256, 0, _lib.LCR_OK), (3, 0, _lib.LCR_OK),
])
def test_chunk_summary_range_checks(lib, c0, nc, code):
    # an empty range is accepted and launches nothing, so it runs without a GPU
    assert lib.lcr_chunk_summary_range(dims(), P, P, 0.1, c0, nc, P, P, NULL) == code
    assert lib.lcr_chunk_summary_range(dims(B=0), P, P, 0.1, 0, 0, P, P, NULL) == _lib.LCR_ERR_ARG


def test_chunk_summary_rejects_nulls_and_scale(lib):
    assert lib.lcr_chunk_summary(None, P, P, 0.1, P, P, NULL) == _lib.LCR_ERR_ARG
    for i in range(4):
        ptrs = [P] * 4
        ptrs[i] = NULL
        assert lib.lcr_chunk_summary(dims(), ptrs[0], ptrs[1], 0.1, ptrs[2], ptrs[3], NULL) == _lib.LCR_ERR_ARG
    assert lib.lcr_chunk_summary(dims(), P, P, float("nan"), P, P, NULL) == _lib.LCR_ERR_ARG


def score_call(lib, dm=None, D=3584, r=64, beta=0.0, scale=0.1, K=32, R=256, q0=0, nq=100, ptrs=None,
               ws=NULL, ws_bytes=0):
    pt = ptrs or [P] * 8
    return lib.lcr_route_score_topk(dm or dims(), pt[0], pt[1], pt[2], pt[3], D, r, pt[4], pt[5], beta, scale,
                                    K, R, q0, nq, pt[6], pt[7], ws, ws_bytes, NULL)


def test_route_score_topk_validation(lib):
    T = 256 * 63
    assert score_call(lib, K=-1) == _lib.LCR_ERR_ARG
    assert score_call(lib, K=65) == _lib.LCR_ERR_UNSUPPORTED
    assert score_call(lib, R=-1) == _lib.LCR_ERR_ARG
    assert score_call(lib, r=0) == _lib.LCR_ERR_ARG
    assert score_call(lib, r=129) == _lib.LCR_ERR_UNSUPPORTED
    assert score_call(lib, D=0) == _lib.LCR_ERR_ARG
    assert score_call(lib, q0=-1) == _lib.LCR_ERR_ARG
    assert score_call(lib, q0=T - 10, nq=11) == _lib.LCR_ERR_ARG
    assert score_call(lib, nq=-1) == _lib.LCR_ERR_ARG
    assert score_call(lib, beta=float("inf")) == _lib.LCR_ERR_ARG
    assert score_call(lib, dm=dims(N=5000)) == _lib.LCR_ERR_UNSUPPORTED
    for i in range(8):
        pt = [P] * 8
        pt[i] = NULL
        assert score_call(lib, ptrs=pt) == _lib.LCR_ERR_ARG
    # valid arguments but no workspace: rejected before any launch
    assert score_call(lib) == _lib.LCR_ERR_WORKSPACE
    need = lib.lcr_workspace_bytes(_lib.OP_ROUTE_SCORE_TOPK, dims(), 3584, 64, 32, 256, 100)
    assert score_call(lib, ws=P, ws_bytes=need - 1) == _lib.LCR_ERR_WORKSPACE
    # nothing to do: K = 0 or nq = 0 succeed without touching the device, NULL outputs allowed
    assert score_call(lib, K=0, ptrs=[P] * 6 + [NULL, NULL]) == _lib.LCR_OK
    assert score_call(lib, nq=0) == _lib.LCR_OK


def test_workspace_sizes(lib):
    dm = dims(dtype=0)
    nq = 1000
    got = lib.lcr_workspace_bytes(_lib.OP_ROUTE_SCORE_TOPK, dm, 3584, 64, 32, 256, nq)
    al = lambda x: (x + 255) // 256 * 256
    # float32: q~ rows, group maxima and per-head scores, plus the partial x.A sums
    assert got >= al(28 * nq * 128 * 4) + al(4 * nq * 256 * 4) + al(28 * nq * 256 * 4) + al(nq * 64 * 4)
    assert got % 256 == 0
    # bf16 at prefill size: the fused scoring kernel keeps only the partial x.A sums and the
    # summaries as bf16 planes; no per-head scores
    fused = lib.lcr_workspace_bytes(_lib.OP_ROUTE_SCORE_TOPK, dims(), 3584, 64, 32, 256, nq)
    assert al(nq * 64 * 4) + al(28 * 256 * 128 * 4) <= fused < al(28 * nq * 256 * 4) and fused % 256 == 0
    dm = dims()
    assert lib.lcr_workspace_bytes(_lib.OP_ROUTE_SCORE_TOPK, dm, 3584, 64, 0, 256, nq) == 0
    assert lib.lcr_workspace_bytes(_lib.OP_CHUNK_SUMMARY, dm, 0, 0, 0, 0, 0) == 0
    assert lib.lcr_workspace_bytes(_lib.OP_SWA_ATTENTION, dm, 0, 0, 0, 0, 0) == 0
    # prefill-sized routed attention needs no workspace; decode-sized splits need partials
    assert lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION, dm, 0, 0, 32, 256, 256 * 63) == 0
    dec = lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION, dims(N=2048), 0, 0, 32, 256, 32)
    assert dec > 0 and dec % 256 == 0
    # one partial (d + 4 floats) per query row and run of entries: a 2-query tile has 2K selected
    # + its window chunks as entries, cut into runs so that about 512 single-wave blocks fill the chip
    entries = 2 * 32 + (2 * 256 + 2) // 63 + 3
    tiles = 16 * 4
    runs = min(-(-512 // tiles), entries // 2)
    epb = -(-entries // runs)
    assert dec == al(-(-entries // epb) * 28 * 32 * (128 + 4) * 4)
    # a window over the whole sequence makes too many entries: the chunk list is split instead
    wide = lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION, dims(N=2048), 0, 0, 32, 10 ** 6, 32)
    assert wide == al(8 * 28 * 32 * (128 + 4) * 4)
    assert lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION, dims(N=2048), 0, 0, 32, -1, 32) == 0
    # a decode-sized plan with a single run per tile still writes one partial per row
    tiny = lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION, dims(N=24, Hq=4, Hkv=2, d=64, dtype=0), 0, 0, 0, 64,
                                   24 * 63)
    assert tiny == al(1 * 4 * 24 * 63 * (64 + 4) * 4)
    assert lib.lcr_workspace_bytes(_lib.OP_ROUTE_SCORE_TOPK, dims(dtype=9), 1, 1, 1, 1, 1) == 0


def test_routed_attention_validation(lib):
    def call(dm=None, K=32, R=256, scale=0.1, q0=0, nq=100, ptrs=None, ws=NULL, ws_bytes=0):
        pt = ptrs or [P] * 6
        return lib.lcr_routed_attention(dm or dims(), pt[0], pt[1], pt[2], pt[3], pt[4], K, R, scale, q0, nq,
                                        pt[5], NULL, ws, ws_bytes, NULL)
    assert call(K=-1) == _lib.LCR_ERR_ARG
    assert call(K=65) == _lib.LCR_ERR_UNSUPPORTED
    assert call(R=-5) == _lib.LCR_ERR_ARG
    assert call(q0=256 * 63, nq=1) == _lib.LCR_ERR_ARG
    assert call(scale=float("nan")) == _lib.LCR_ERR_ARG
    for i in range(6):
        pt = [P] * 6
        pt[i] = NULL
        assert call(ptrs=pt) == _lib.LCR_ERR_ARG
    assert call(nq=0) == _lib.LCR_OK
    # decode-sized problems need the partial-sum workspace
    assert call(dm=dims(N=2048), q0=2048 * 63 - 32, nq=32) == _lib.LCR_ERR_WORKSPACE


def test_routed_attention_backward_validation(lib):
    def call(dm=None, K=32, R=256, scale=0.1, q0=0, nq=100, ptrs=None, ws=P, ws_bytes=1 << 40):
        pt = ptrs or [P] * 13
        return lib.lcr_routed_attention_backward(dm or dims(), pt[0], pt[1], pt[2], pt[3], pt[4], K, R, scale, q0,
                                                 nq, pt[5], pt[6], pt[7], pt[8], pt[9], pt[10], pt[11], ws,
                                                 ws_bytes, NULL)
    assert call(dm=dims(dtype=4)) == _lib.LCR_ERR_DTYPE                # bf16 and float32 only
    assert call(K=-1) == _lib.LCR_ERR_ARG
    assert call(K=65) == _lib.LCR_ERR_UNSUPPORTED
    assert call(R=-5) == _lib.LCR_ERR_ARG
    assert call(q0=256 * 63, nq=1) == _lib.LCR_ERR_ARG
    assert call(scale=float("inf")) == _lib.LCR_ERR_ARG
    for i in range(12):          # q k v idx zsel o lse dO dq dk dv dzsel: every one is required
        pt = [P] * 13
        pt[i] = NULL
        assert call(ptrs=pt) == _lib.LCR_ERR_ARG, i
    # K = 0: idx, zsel and dzsel may be NULL
    pt = [P] * 13
    pt[3] = pt[4] = pt[11] = NULL
    need0 = lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION_BACKWARD, dims(), 0, 0, 0, 256, 100)
    assert need0 > 0
    assert call(K=0, ptrs=pt, ws=NULL) == _lib.LCR_ERR_WORKSPACE
    need = lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION_BACKWARD, dims(), 0, 0, 32, 256, 100)
    assert call(ws_bytes=need - 1) == _lib.LCR_ERR_WORKSPACE
    al = lambda x: (x + 255) // 256 * 256
    rows, bgn = 28 * 100, 4 * 256
    # D per row; bias and U per (row, selected chunk); counts and offsets per chunk; per-tile counts of
    # 256-row tiles; the entry lists
    assert need == al(rows * 4) + 2 * al(rows * 32 * 4) + al(bgn * 4) + al(4 * 257 * 4) + al(4 * 1 * 256 * 4) \
        + al(4 * 100 * 32 * 4)
    assert call(dm=dims(N=32769)) == _lib.LCR_ERR_UNSUPPORTED


def test_chunk_summary_backward_validation(lib):
    def call(dm=None, scale=0.1, ptrs=None):
        pt = ptrs or [P] * 6
        return lib.lcr_chunk_summary_backward(dm or dims(), pt[0], pt[1], scale, pt[2], pt[3], pt[4], pt[5], NULL)
    assert call(dm=dims(dtype=4)) == _lib.LCR_ERR_DTYPE
    assert call(dm=dims(d=96)) == _lib.LCR_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == _lib.LCR_ERR_ARG
    for i in range(6):
        pt = [P] * 6
        pt[i] = NULL
        assert call(ptrs=pt) == _lib.LCR_ERR_ARG, i


def test_route_score_backward_validation(lib):
    def call(dm=None, D=3584, r=64, K=32, q0=0, nq=100, beta=0.0, scale=0.1, ptrs=None, ws=P, ws_bytes=1 << 40):
        pt = ptrs or [P] * 13
        return lib.lcr_route_score_backward(dm or dims(), pt[0], pt[1], pt[2], pt[3], D, r, pt[4], beta, scale, K, q0,
                                            nq, pt[5], pt[6], pt[7], pt[8], pt[9], pt[10], pt[11], pt[12], ws,
                                            ws_bytes, NULL)
    assert call(r=129) == _lib.LCR_ERR_UNSUPPORTED
    assert call(r=0) == _lib.LCR_ERR_ARG
    assert call(K=-1) == _lib.LCR_ERR_ARG
    assert call(beta=float("nan")) == _lib.LCR_ERR_ARG
    assert call(q0=10, nq=256 * 63) == _lib.LCR_ERR_ARG
    for i in range(13):
        pt = [P] * 13
        pt[i] = NULL
        assert call(ptrs=pt) == _lib.LCR_ERR_ARG, i
    need = lib.lcr_workspace_bytes(_lib.OP_ROUTE_SCORE_BACKWARD, dims(), 3584, 64, 32, 0, 100)
    assert need > 0 and need % 256 == 0
    assert call(ws_bytes=need - 1) == _lib.LCR_ERR_WORKSPACE
    assert call(ws=NULL) == _lib.LCR_ERR_WORKSPACE
    assert call(dm=dims(N=40000)) == _lib.LCR_ERR_UNSUPPORTED


def test_swa_validation(lib):
    def call(B=1, Hq=28, Hkv=4, L=4096, d=128, dtype=1, R=1280, scale=0.1, ptrs=None):
        pt = ptrs or [P] * 4
        return lib.lcr_swa_attention(B, Hq, Hkv, L, d, dtype, pt[0], pt[1], pt[2], R, scale, pt[3], NULL, NULL)
    assert call(dtype=3) == _lib.LCR_ERR_DTYPE
    assert call(L=0) == _lib.LCR_ERR_ARG
    assert call(R=-1) == _lib.LCR_ERR_ARG
    assert call(Hq=30) == _lib.LCR_ERR_ARG
    assert call(d=32) == _lib.LCR_ERR_UNSUPPORTED
    assert call(Hq=72, Hkv=4) == _lib.LCR_ERR_UNSUPPORTED
    for i in range(4):
        pt = [P] * 4
        pt[i] = NULL
        assert call(ptrs=pt) == _lib.LCR_ERR_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_wait_limit_setting(lib):
    """The failure-handling hook keeps one process-wide setting: it returns the previous
    value, and a value below one restores the default (2^22 polls)."""
    default = 1 << 22
    assert lib.lcr_set_wait_limit(5) == default
    assert lib.lcr_set_wait_limit(0) == 5
    assert lib.lcr_set_wait_limit(-3) == default
    assert lib.lcr_set_wait_limit(0) == default


def test_tile_order_setting(lib):
    """The order-independence hook: any nonzero value means reversed, the previous
    setting comes back, and the default is the XCD-aware order (0)."""
    assert lib.lcr_set_tile_order(7) == 0
    assert lib.lcr_set_tile_order(1) == 1
    assert lib.lcr_set_tile_order(0) == 1
    assert lib.lcr_set_tile_order(0) == 0


def test_noalloc_rejects_plans_beyond_the_scratch(lib):
    """lcr_routed_attention_noalloc checks on the host that the plan's partials fit its
    static scratch; a decode-sized plan of 1,000 queries (one partial per row, 14.8 MB)
    does not, and is rejected before anything is enqueued."""
    d = dims(N=2048)
    K, R, nq = 32, 256, 1000
    need = lib.lcr_workspace_bytes(_lib.OP_ROUTED_ATTENTION, d, 0, 0, K, R, nq)
    assert need > _lib.LCR_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(256)   # never dereferenced: the call is rejected on the host
    rc = lib.lcr_routed_attention_noalloc(d, p, p, p, p, p, K, R, 0.1, 0, nq, p, None, None)
    assert rc == _lib.LCR_ERR_UNSUPPORTED
    assert lib.lcr_routed_attention_noalloc(d, p, p, p, p, p, K, R, 0.1, 0, 0, p, None, None) == _lib.LCR_OK
    assert lib.lcr_routed_attention_noalloc(d, None, p, p, p, p, K, R, 0.1, 0, nq, p, None, None) == \
        _lib.LCR_ERR_ARG
