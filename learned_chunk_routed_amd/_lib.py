"""ctypes loader for liblcr.so (the HIP library built in-tree by build.py).

Fails loudly when the library is missing: there is no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblcr.so")

LCR_OK, LCR_ERR_ARG, LCR_ERR_DTYPE, LCR_ERR_WORKSPACE, LCR_ERR_HIP, LCR_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
LCR_F32, LCR_BF16 = 0, 1
OP_CHUNK_SUMMARY, OP_ROUTE_SCORE_TOPK, OP_ROUTED_ATTENTION, OP_SWA_ATTENTION = 0, 1, 2, 3
OP_ROUTED_ATTENTION_BACKWARD, OP_ROUTE_SCORE_BACKWARD = 4, 5
LCR_NOALLOC_SCRATCH_BYTES = 8 << 20   # static scratch of lcr_routed_attention_noalloc


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("N", ctypes.c_int),
                ("d", ctypes.c_int), ("dtype", ctypes.c_int)]


_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_pd = ctypes.POINTER(Dims)

SIGNATURES = {
    "lcr_version": (_i, []),
    "lcr_status_string": (ctypes.c_char_p, [_i]),
    "lcr_set_wait_limit": (_i, [_i]),
    "lcr_set_tile_order": (_i, [_i]),
    "lcr_workspace_bytes": (_sz, [_i, _pd, _i, _i, _i, _i, _i]),
    "lcr_chunk_summary": (_i, [_pd, _vp, _vp, _f, _vp, _vp, _vp]),
    "lcr_chunk_summary_range": (_i, [_pd, _vp, _vp, _f, _i, _i, _vp, _vp, _vp]),
    "lcr_chunk_summary_mean": (_i, [_pd, _vp, _vp, _vp, _vp]),
    "lcr_route_score_topk": (_i, [_pd, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _f, _f, _i, _i, _i, _i,
                                  _vp, _vp, _vp, _sz, _vp]),
    "lcr_routed_attention": (_i, [_pd, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "lcr_routed_attention_noalloc": (_i, [_pd, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _i, _vp, _vp, _vp]),
    "lcr_routed_attention_backward": (_i, [_pd, _vp, _vp, _vp, _vp, _vp, _i, _i, _f, _i, _i, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lcr_route_score_backward": (_i, [_pd, _vp, _vp, _vp, _vp, _i, _i, _vp, _f, _f, _i, _i, _i, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lcr_chunk_summary_backward": (_i, [_pd, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp]),
    "lcr_swa_attention": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _i, _f, _vp, _vp, _vp]),
}

_lib = None


def load():
    """Load liblcr.so once and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m learned_chunk_routed_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().lcr_status_string(code).decode()


def check(code: int, what: str):
    if code != LCR_OK:
        raise RuntimeError(f"{what} failed: {status_string(code)} ({code})")
