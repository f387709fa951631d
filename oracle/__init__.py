"""fp64 CPU oracle for route-layer attention and bidirectional sliding-window attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package. The
product path (the HIP library and its Python binding) never calls it, and this
package shares no code with that path: the two have in common only the seeded
input generators in ``lcr_inputs``.

Every function is plain numpy in float64; bf16 or fp32 inputs are upcast
exactly. Sources: "Prefilling-dLLM v2: Learned Chunk Routing for Long-Context
Diffusion Language Models" (Abstract; Figure 2 and Figure 3 captions; Table 3)
and "The 172x Speedup Has an Evidence Budget" (section "How learned routing
controls what the model can read").

Gradients (module ``backward``) hold the chosen chunks fixed and follow the
chain rule through the forward's steps in reverse.

Pins (all in tests/oracle_pins.py, run with ``-m "not gpu"``): every function
here is pinned by closed forms, invariants, brute force or a library routine;
none is "parity unpinned".
"""
from .route import (  # noqa: F401
    SLOTS, CONTENT, slot_of,
    softmax, entropy,
    chunk_summary, chunk_summary_from_mask,
    routing_query, window_bounds, candidate_mask,
    route_scores, group_max, select_topk, gather_zsel,
    routed_attention, route_layer, route_layer_rows, swa_attention,
)
from .backward import (  # noqa: F401
    routed_attention_backward, route_score_backward, chunk_summary_backward,
    route_layer_backward,
)
