"""Route-layer attention with learned chunk routing, and bidirectional sliding-window
attention, on AMD Instinct MI355X (gfx950).

The compute path is the HIP library liblcr.so (C ABI in include/lcr.h); the
functions here marshal torch tensors into it. Import fails loudly only when a
call is made without the library: build it with
``python -m learned_chunk_routed_amd.build``.
"""
from ._lib import LIB_PATH, load  # noqa: F401
from .ops import (  # noqa: F401
    chunk_summary,
    chunk_summary_mean,
    chunk_summary_backward,
    route_score_backward,
    route_score_topk,
    routed_attention,
    routed_attention_backward,
    swa_attention,
    route_layer,
    route_layer_backward,
    workspace_bytes,
    set_wait_limit,
    set_tile_order,
    make_dims,
    default_scale,
)
