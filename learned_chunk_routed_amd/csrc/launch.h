// Internal launch interface between the C ABI (api.cpp) and the kernel files.
// Every launcher assumes its arguments were validated by validate.cpp and
// returns the HIP status of its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcr {

typedef uint16_t bf16_t;

struct RouteDims {
  int B, Hq, Hkv, N, d, dtype;  // dtype: 0 = float32, 1 = bfloat16
};

// ---- chunk_summary (summary.hip)
// chunks c0 .. c0 + nc - 1 (nc >= 1)
hipError_t launch_chunk_summary(const RouteDims& dm, const void* q, const void* k, float scale,
                                float* s, float* H, int c0, int nc, hipStream_t st);
// uniform pooling weights (mean summaries), all chunks
hipError_t launch_chunk_summary_mean(const RouteDims& dm, const void* k, float* s, float* H, hipStream_t st);

// ---- route_score_topk (score.hip)
struct ScoreWs {
  float* qt;    // [B,Hq,nq,d]  routing queries q~ (float32)
  float* zhat;  // [B,Hkv,nq,N] group maximum of the scores
  float* z;     // [B,Hq,nq,N]  per-head scores
  float* upart; // [splits,B,nq,rank padded to 32/64/128]  partial x A
  bf16_t* splanes; // [B,Hq,N,2d] summaries as bf16 hi then lo, k-permuted (fused path)
  bf16_t* qplanes; // [B,Hq,32,2d] q~ as bf16 hi then lo (decode-sized path)
  bf16_t* at;      // [rank padded, D padded to 32] A transposed (bf16 prefill path)
  bf16_t* bt;      // [Hq*d, rank padded] B transposed (bf16 prefill path)
};
size_t score_ws_bytes(const RouteDims& dm, int D, int r, int nq, int K);
ScoreWs score_ws_carve(void* ws, const RouteDims& dm, int D, int r, int nq, int K);
hipError_t launch_route_score_topk(const RouteDims& dm, const void* q, const void* x, const void* A,
                                   const void* Bm, int D, int r, const float* s, const float* H,
                                   float beta, float scale, int K, int radius, int q0, int nq,
                                   int32_t* idx, float* zsel, const ScoreWs& ws, hipStream_t st);

// q~ and the partial sums of u = x A (general path) for the scoring's backward
int qtilde_u_splits(const RouteDims& dm, int Dh, int nq);
int qtilde_rank_pad(int r);
hipError_t launch_qtilde_with_u(const RouteDims& dm, const void* q, const void* x, const void* A, const void* Bm,
                                int Dh, int r, float* qt, float* upart, int q0, int nq, hipStream_t st);

// ---- routed_attention and swa_attention (attention.hip)
struct AttnPlan {
  int waves;       // waves per block
  int tiles;       // 16-row tiles per wave (a tile = 2 queries x 8 head rows)
  int qblock;      // queries per block = 2 * waves * tiles
  int nsplit;      // partials per query row, merged by combine_kernel when > 1
  int kind;        // 0: blocks walk a chunk list; 1: one block per (2-query tile, chunk entry);
                   // 2: producer / consumer waves over a chunk ring (bf16 prefill)
  int nbuf;        // kind 2: K-or-V halves in the LDS pool
  int nent;        // kind 1: entries per 2-query tile (2K selected + window chunks)
  int epb;         // kind 1: entries per block (nsplit = ceil(nent / epb) runs)
  size_t lds;      // dynamic LDS bytes per block
  size_t ws;       // workspace bytes for the split partials
};
AttnPlan plan_routed_attention(const RouteDims& dm, int K, int radius, int nq);
// polls before a wait on an LDS counter gives up (< 1: the default); returns the previous value
int set_wait_limit(int polls);
int set_tile_order(int reversed);
int tile_order();
// the static scratch of lcr_routed_attention_noalloc: its size, and its device
// address on the current device (looked up on the first call per device)
constexpr size_t kScratchBytes = (size_t)8 << 20;
size_t routed_scratch_bytes();
hipError_t routed_scratch(void** out);
size_t routed_lds_limit();
hipError_t launch_routed_attention(const RouteDims& dm, const AttnPlan& plan, const void* q,
                                   const void* k, const void* v, const int32_t* idx,
                                   const float* zsel, int K, int radius, float scale, int q0,
                                   int nq, void* o, float* lse, void* ws, hipStream_t st);

// ---- routed attention backward (backward.hip), bf16 only
size_t routed_bwd_ws_bytes(const RouteDims& dm, int K, int nq);
size_t routed_bwd_lds_bytes(int d);
hipError_t launch_routed_attention_backward(const RouteDims& dm, const void* q, const void* k, const void* v,
                                            const int32_t* idx, const float* zsel, int K, int radius,
                                            float scale, int q0, int nq, const void* o, const float* lse,
                                            const void* dO, float* dq, float* dk, float* dv, float* dzsel,
                                            void* ws, hipStream_t st);

size_t score_bwd_ws_bytes(const RouteDims& dm, int Dh, int r, int K, int nq);
hipError_t launch_route_score_backward(const RouteDims& dm, const void* q, const void* x, const void* A,
                                       const void* Bm, int Dh, int r, const float* s, float beta, float scale, int K,
                                       int q0, int nq, const int32_t* idx, const float* dzsel, float* dq, float* dx,
                                       float* dA, float* dBm, float* ds, float* dH, void* ws, hipStream_t st);
hipError_t launch_chunk_summary_backward(const RouteDims& dm, const void* q, const void* k, float scale,
                                         const float* ds, const float* dH, float* dq, float* dk, hipStream_t st);

// query side of the routed attention backward through the forward's chunk pool (bf16)
size_t bwd_query_pool_lds(int d, int N);
hipError_t launch_bwd_query_pool(const RouteDims& dm, const void* q, const void* k, const void* v, const void* o,
                                 const void* dO, const int32_t* idx, const float* zsel, const float* lse, int K,
                                 int radius, float scale, int q0, int nq, float* dq, float* dzsel, float* dsum,
                                 float* cbias, float* cu, hipStream_t st);

size_t swa_lds_bytes(int d, int dtype);
hipError_t launch_swa_attention(int B, int Hq, int Hkv, int L, int d, int dtype, const void* q,
                                const void* k, const void* v, int radius, float scale, void* o,
                                float* lse, hipStream_t st);

}  // namespace lcr
