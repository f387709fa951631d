/*
 * lcr.h - route-layer attention with learned chunk routing, and bidirectional
 * sliding-window attention, for AMD Instinct MI355X (gfx950).
 *
 * The method is the route layer of "Prefilling-dLLM v2: Learned Chunk Routing
 * for Long-Context Diffusion Language Models" (Abstract; Figure 3 caption;
 * Table 3) as also described in "The 172x Speedup Has an Evidence Budget"
 * (section "How learned routing controls what the model can read").
 *
 * Sequence layout. A sequence of N chunks has L = 64*N slots. Chunk c holds 63
 * content tokens in slots 64c..64c+62 and its routing mask in slot 64c+63.
 * Content index i (0 <= i < T = 63*N) lives in slot 64*(i/63) + i%63.
 * Query head h belongs to KV group g = h / G with G = Hq / Hkv.
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a DEVICE pointer owned by the caller; the
 *    library never allocates, frees or synchronises. Tensors are contiguous,
 *    row-major, in the shapes given below.
 *  - dtype LCR_BF16: q, k, v, x, A, Bm and o are bfloat16; LCR_F32: float32.
 *    s, H, zsel and lse are always float32; idx is int32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and runs asynchronously. A call returns LCR_OK once its kernels are
 *    enqueued.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    negative return nothing was enqueued and no output was touched.
 *    LCR_ERR_HIP means a launch was rejected by the HIP runtime; earlier
 *    kernels of the same call may already have been enqueued.
 *  - Limits: d in {64, 128}; 1 <= G <= 8; 0 <= K <= 64; radius >= 0.
 *  - The library keeps no state between calls (apart from the wait limit of
 *    lcr_set_wait_limit and the tile order of lcr_set_tile_order) and may be
 *    called from several host threads on different streams.
 */
#ifndef LCR_H
#define LCR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCR_CHUNK_SLOTS 64
#define LCR_CHUNK_CONTENT 63
#define LCR_MAX_GROUP 8
#define LCR_MAX_TOPK 64

typedef enum {
  LCR_OK = 0,
  LCR_ERR_ARG = -1,          /* a size, range or pointer is invalid */
  LCR_ERR_DTYPE = -2,        /* dtype is not LCR_F32 or LCR_BF16 */
  LCR_ERR_WORKSPACE = -3,    /* ws is NULL or smaller than lcr_workspace_bytes() */
  LCR_ERR_HIP = -4,          /* the HIP runtime rejected a launch */
  LCR_ERR_UNSUPPORTED = -5   /* valid, but outside this library's limits (d, G, K, LDS) */
} lcr_status;

typedef enum { LCR_F32 = 0, LCR_BF16 = 1 } lcr_dtype;

/* Shape of a route layer: batch, query heads, KV heads, chunks, head dim, dtype. */
typedef struct {
  int B, Hq, Hkv, N, d;
  int dtype; /* lcr_dtype */
} lcr_dims;

typedef enum {
  LCR_OP_CHUNK_SUMMARY = 0,
  LCR_OP_ROUTE_SCORE_TOPK = 1,
  LCR_OP_ROUTED_ATTENTION = 2,
  LCR_OP_SWA_ATTENTION = 3,
  LCR_OP_ROUTED_ATTENTION_BACKWARD = 4,
  LCR_OP_ROUTE_SCORE_BACKWARD = 5
} lcr_op;

/*
 * Failure-handling hook. The pooled kernels (bf16 routed attention of
 * prefill-sized problems, the query side of its backward, and the split routed
 * attention of wide windows) coordinate their waves through counters in LDS.
 * Every wait on such a counter gives up after `polls` polls (default 2^22, a
 * fraction of a second), so a logic error cannot hang the GPU. A wave whose
 * wait gives up stops and writes NaN to every output row it owns (o and lse of
 * the forward; dq and dzsel of the backward), so an incomplete result never
 * passes for a valid one; the call still returns LCR_OK. Rows of waves that
 * completed their walk are exact. polls < 1 restores the default. The setting
 * is process-wide (the one piece of state the library keeps) and applies to
 * calls enqueued after this returns. Returns the previous setting.
 */
int lcr_set_wait_limit(int polls);

/*
 * Test hook for order independence. The tiled kernels (the pooled routed
 * attention of prefill-sized problems, the query side of its backward and the
 * fused bf16 scoring) map their blocks onto (batch, KV group, query block)
 * tiles in an XCD-aware order; reversed != 0 walks the same tiles in the
 * opposite order. No block depends on another, so every output is bit for bit
 * the same either way; tests compare the two. Process-wide, for calls enqueued
 * after this returns; returns the previous setting (0 or 1). Default 0.
 */
int lcr_set_tile_order(int reversed);

/* Library version as 10000*major + 100*minor + patch. */
int lcr_version(void);

/* Human-readable name of a status code (static string; never NULL). */
const char* lcr_status_string(int status);

/*
 * Bytes of device workspace `op` needs for these sizes (0 if none). D and r are
 * used by LCR_OP_ROUTE_SCORE_TOPK only; K and nq by the two routing calls;
 * radius by LCR_OP_ROUTED_ATTENTION (decode-sized problems keep one partial
 * result per selected or window chunk). Returns 0 for invalid sizes as well;
 * the call itself reports those.
 */
size_t lcr_workspace_bytes(int op, const lcr_dims* dims, int D, int r, int K, int radius, int nq);

/*
 * Summary keys and pooling entropies ("Prefilling-dLLM v2", Figure 3 caption:
 * the routing mask's query pools its chunk's content keys with an intra-chunk
 * softmax; the weighted sum is the summary key. "The 172x Speedup...": the
 * entropy of these pooling weights is the second ranking signal).
 *
 *   alpha_j = softmax_j(scale * q[b,h,64c+63] . k[b,g,64c+j]),  j = 0..62
 *   s[b,h,c] = sum_j alpha_j k[b,g,64c+j]
 *   H[b,h,c] = -sum_j alpha_j ln alpha_j
 *
 * q [B,Hq,L,d]: only the mask-slot rows 64c+63 are read.
 * k [B,Hkv,L,d]: only content rows are read.
 * s [B,Hq,N,d] float32 (written), H [B,Hq,N] float32 (written).
 * Arithmetic in float32.
 */
int lcr_chunk_summary(const lcr_dims* dims, const void* q, const void* k, float scale,
                      float* s, float* H, void* stream);

/*
 * The same summaries for chunks c0 .. c0 + nc - 1 only: the refresh a decode
 * loop needs after the keys of some chunks changed (the block being decoded),
 * since a chunk's summary and entropy depend on that chunk's keys and mask
 * query alone (same sources as lcr_chunk_summary). Rows of s and H outside the
 * range are not touched; the refreshed rows equal those of a whole
 * lcr_chunk_summary call on the same inputs bit for bit. nc = 0 does nothing.
 * Errors: as lcr_chunk_summary, and LCR_ERR_ARG unless 0 <= c0, 0 <= nc and
 * c0 + nc <= N.
 */
int lcr_chunk_summary_range(const lcr_dims* dims, const void* q, const void* k, float scale, int c0, int nc,
                            float* s, float* H, void* stream);

/*
 * Mean summaries: the "Mean summary" ablation of "Prefilling-dLLM v2" (Table 6)
 * and of "The 172x Speedup Has an Evidence Budget" (section "The mechanism tests
 * reveal what actually contributes"): attention-weighted summaries replaced by
 * mean pooling.
 * The pooling weights are uniform, so
 *
 *   s[b,h,c] = (1/63) sum_j k[b,g(h),64c+j]   (the same for every head of a group)
 *   H[b,h,c] = ln 63
 *
 * which is lcr_chunk_summary with zero mask queries. k [B,Hkv,L,d]; s [B,Hq,N,d]
 * and H [B,Hq,N] float32 (written); dims as lcr_chunk_summary. The result feeds
 * lcr_route_score_topk unchanged. Errors: as lcr_chunk_summary (no q).
 */
int lcr_chunk_summary_mean(const lcr_dims* dims, const void* k, float* s, float* H, void* stream);

/*
 * Residual-augmented scoring, GQA maximum and top-K selection ("Prefilling-dLLM
 * v2", Figure 3 caption: a content query adds a low-rank residual and scores the
 * summaries; scores are reduced by a maximum inside each GQA group; the top K
 * chunks are shared by every head of the group. Table 3: the remote chunks lie
 * beyond the local window).
 *
 * For content queries i = q0 .. q0+nq-1 (t = i - q0):
 *   q~[b,h,t] = q[b,h,slot(i)] + (x[b,slot(i)] . A . Bm)[h*d .. h*d+d-1]
 *   z[b,h,t,c] = scale * q~[b,h,t] . s[b,h,c] - beta * H[b,h,c]
 *   zhat[b,g,t,c] = max over the G heads of group g of z[b,h,t,c]
 *   candidates: chunks none of whose content indices 63c..63c+62 lies within
 *               [i-radius, i+radius]
 *   idx[b,g,t,:] = the min(K, #candidates) candidates with the largest zhat,
 *                  ties to the smaller chunk index, in ascending chunk order,
 *                  padded with -1
 *   zsel[b,h,t,k] = z[b,h,t,idx[b,g,t,k]] (-INFINITY where idx is -1)
 *
 * q [B,Hq,L,d]; x [B,L,D] (rows at the query slots are read); A [D,r];
 * Bm [r,Hq*d]; s [B,Hq,N,d]; H [B,Hq,N]. idx [B,Hkv,nq,K] int32 and
 * zsel [B,Hq,nq,K] float32 are written; with K = 0 both may be NULL.
 * Scores are computed to near-float32 accuracy (split-bfloat16 products with
 * float32 accumulation). ws: lcr_workspace_bytes(LCR_OP_ROUTE_SCORE_TOPK, ...)
 * bytes of device memory, contents need not be initialised.
 * Limits: 1 <= r <= 128, D >= 1, 0 <= q0, q0 + nq <= T.
 */
int lcr_route_score_topk(const lcr_dims* dims, const void* q, const void* x, const void* A,
                         const void* Bm, int D, int r, const float* s, const float* H,
                         float beta, float scale, int K, int radius, int q0, int nq,
                         int32_t* idx, float* zsel, void* ws, size_t ws_bytes, void* stream);

/*
 * Routed attention ("Prefilling-dLLM v2", Figure 3 caption: the selected chunk
 * scores and the local window's log-sum-exp share one softmax partition; a
 * second softmax spreads each chunk's mass over its content tokens).
 *
 * For content query i (t = i - q0), head h, group g:
 *   W = {u : |u - i| <= radius, 0 <= u < T}; a_u = scale * q[b,h,slot(i)] . k[b,g,slot(u)]
 *   chunk logits z_k = zsel[b,h,t,k] for idx[b,g,t,k] >= 0
 *   P = softmax over {a_u : u in W} joined with {z_k}
 *   u_bar_k = sum_j softmax_j(scale * q . k[b,g,64c+j]) v[b,g,64c+j], j = 0..62, c = idx
 *   o[b,h,slot(i)] = sum_u P_u v[b,g,slot(u)] + sum_k P_k u_bar_k
 *   lse[b,h,t] = log of the partition's normaliser
 *
 * idx must list, for each row, chunks that are remote from i (as produced by
 * lcr_route_score_topk), ascending, -1 padded. q, k, v as above;
 * o [B,Hq,L,d]: only rows slot(i) for the queried i are written; lse
 * [B,Hq,nq] float32 or NULL. ws: lcr_workspace_bytes(LCR_OP_ROUTED_ATTENTION,
 * ...) bytes (may be 0 and ws NULL). Arithmetic: bf16 products with float32
 * accumulation for bf16 inputs, split-bf16 (near float32) for float32 inputs.
 */
int lcr_routed_attention(const lcr_dims* dims, const void* q, const void* k, const void* v,
                         const int32_t* idx, const float* zsel, int K, int radius, float scale,
                         int q0, int nq, void* o, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * lcr_routed_attention for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, semantics and results as lcr_routed_attention,
 * without ws/ws_bytes: where the plan needs workspace (decode-sized problems
 * keep partial results), it uses a static device array of
 * LCR_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs on
 * until the process ends (its device address is looked up on the first call on
 * each device; nothing is allocated or freed by the call). Every call on one
 * GPU shares that array: calls that overlap in time on the same GPU (different
 * streams, or threads) race and give wrong results; calls ordered on one
 * stream are safe. The array needs no clearing (every partial a call reads is
 * written by that call first). Errors: as lcr_routed_attention, and
 * LCR_ERR_UNSUPPORTED when lcr_workspace_bytes(LCR_OP_ROUTED_ATTENTION, ...)
 * exceeds LCR_NOALLOC_SCRATCH_BYTES.
 */
#define LCR_NOALLOC_SCRATCH_BYTES (8u << 20)
int lcr_routed_attention_noalloc(const lcr_dims* dims, const void* q, const void* k, const void* v,
                                 const int32_t* idx, const float* zsel, int K, int radius, float scale,
                                 int q0, int nq, void* o, float* lse, void* stream);

/*
 * Gradients of lcr_routed_attention with the chosen chunks held fixed ("The 172x
 * Speedup Has an Evidence Budget", section "How learned routing controls what
 * the model can read": chunk membership is not differentiable; the router is
 * trained through the masses of the selected chunks, i.e. through zsel).
 *
 * With P, pi and u_bar as in lcr_routed_attention, dO the upstream gradient on
 * o and D = dO . o per (head, query):
 *   dzsel[b,h,t,k] = P_k (dO . u_bar_k - D)          (0 where idx is -1)
 *   dq, dk, dv     = the gradients of o through every window key and every
 *                    content key of the selected chunks (chain rule through the
 *                    joint partition and the intra-chunk softmax)
 *
 * Inputs exactly as passed to (and produced by) the forward call: q, k, v, idx,
 * zsel, K, radius, scale, q0, nq; o [B,Hq,L,d] and lse [B,Hq,nq] (both
 * required); dO [B,Hq,L,d] (rows slot(i) read); q, k, v, o, dO in dims->dtype.
 * Outputs, float32: dq [B,Hq,L,d] (only rows slot(i) of the queried i are
 * written); dk, dv [B,Hkv,L,d] (every row written: rows no queried row reads,
 * mask slots included, are zero); dzsel [B,Hq,nq,K] (may be NULL when K = 0).
 * Only the nq queried rows contribute. ws: lcr_workspace_bytes(
 * LCR_OP_ROUTED_ATTENTION_BACKWARD, dims, 0, 0, K, radius, nq) bytes, contents
 * need not be initialised. Arithmetic: LCR_BF16 takes bf16 products
 * (probabilities and their gradients rounded to bf16 for the products) with
 * float32 accumulation; LCR_F32 takes float32 throughout on the vector ALUs (a
 * plain path for parity-sized problems, not tuned for speed). Either way the
 * order is fixed: results are reproducible bit for bit.
 * Errors: as lcr_routed_attention; LCR_ERR_UNSUPPORTED for N > 32768.
 */
int lcr_routed_attention_backward(const lcr_dims* dims, const void* q, const void* k, const void* v,
                                  const int32_t* idx, const float* zsel, int K, int radius, float scale,
                                  int q0, int nq, const void* o, const float* lse, const void* dO,
                                  float* dq, float* dk, float* dv, float* dzsel, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * Gradients of the scoring with the chosen chunks fixed ("Prefilling-dLLM v2",
 * Figure 3 caption: the residual-augmented query scores the summaries; "The
 * 172x Speedup...": similarity minus beta times the pooling entropy). For
 * zsel[b,h,t,k] = scale q~[b,h,t] . s[b,h,c] - beta H[b,h,c], c = idx[b,g,t,k],
 * q~ = q + (x A Bm)[h*d .. h*d+d-1] and an upstream dzsel (e.g. from
 * lcr_routed_attention_backward):
 *   dq~ = scale sum_k dzsel s[c_k]; dq[b,h,slot(i)] += dq~          (added)
 *   ds[b,h,c] = scale sum over (t,k) with idx = c of dzsel q~[b,h,t] (written)
 *   dH[b,h,c] = -beta sum over the same entries of dzsel             (written)
 *   with U = x A per row: dBm = U^T dq~, dA = x^T (dq~ Bm^T),
 *   dx[b,slot(i)] = (dq~ Bm^T) A^T                                   (written)
 * The group maximum and the top-K choice only decide idx and get no gradient.
 * q, x, A, Bm, s as in lcr_route_score_topk (dims->dtype); idx [B,Hkv,nq,K];
 * dzsel [B,Hq,nq,K] float32. Outputs, float32: dq [B,Hq,L,d] (rows slot(i)
 * accumulated into), dx [B,L,D] (rows slot(i) written), dA [D,r] and
 * dBm [r,Hq*d] (written; sums over the nq rows and the batch), ds [B,Hq,N,d],
 * dH [B,Hq,N] (written; zero for chunks no row selected). ws:
 * lcr_workspace_bytes(LCR_OP_ROUTE_SCORE_BACKWARD, dims, D, r, K, 0, nq)
 * bytes. Arithmetic in float32, in a fixed order (reproducible bit for bit).
 * Errors: as lcr_route_score_topk; N > 32768 is LCR_ERR_UNSUPPORTED.
 */
int lcr_route_score_backward(const lcr_dims* dims, const void* q, const void* x, const void* A, const void* Bm,
                             int D, int r, const float* s, float beta, float scale, int K, int q0, int nq,
                             const int32_t* idx, const float* dzsel, float* dq, float* dx, float* dA, float* dBm,
                             float* ds, float* dH, void* ws, size_t ws_bytes, void* stream);

/*
 * Gradients of lcr_chunk_summary ("Prefilling-dLLM v2", Figure 3 caption: mask-
 * query pooling; "The 172x Speedup...": the pooling entropy) for upstream
 * gradients ds [B,Hq,N,d] and dH [B,Hq,N] (float32), e.g. from the scoring's
 * backward. With alpha, s and H as in lcr_chunk_summary:
 *   g_j = ds . k_j - (ln alpha_j + 1) dH,  dlam_j = alpha_j (g_j - sum_i alpha_i g_i)
 *   dq[b,h,64c+63] = scale sum_j dlam_j k_j                        (written)
 *   dk[b,g,64c+j] += sum over the group's heads of alpha_j ds + scale dlam_j q_m
 *                                                              (j < 63, added)
 * q, k as in lcr_chunk_summary (dims->dtype); dq [B,Hq,L,d] float32: only the
 * mask-slot rows are written; dk [B,Hkv,L,d] float32: content rows are
 * accumulated into, mask rows untouched, so the call adds the pooling's share to
 * the gradient lcr_routed_attention_backward wrote. Arithmetic in float32.
 */
int lcr_chunk_summary_backward(const lcr_dims* dims, const void* q, const void* k, float scale, const float* ds,
                               const float* dH, float* dq, float* dk, void* stream);

/*
 * Bidirectional sliding-window attention for the layers that do not route
 * ("Prefilling-dLLM v2", Abstract and Table 3: the other layers use a
 * bidirectional sliding window, radius 1280). Every slot, content or mask, is
 * an ordinary token:
 *   o[b,h,t] = sum_u softmax_u(scale * q[b,h,t] . k[b,g,u]) v[b,g,u],
 *   |u - t| <= radius, 0 <= u < L.
 * q [B,Hq,L,d], k, v [B,Hkv,L,d], o [B,Hq,L,d]; lse [B,Hq,L] float32 or NULL.
 */
int lcr_swa_attention(int B, int Hq, int Hkv, int L, int d, int dtype, const void* q,
                      const void* k, const void* v, int radius, float scale, void* o,
                      float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LCR_H */
