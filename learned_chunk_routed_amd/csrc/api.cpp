// C ABI of the route-layer attention library (declared in include/lcr.h).
// Each entry point validates its arguments on the host (validate.cpp), then
// enqueues its kernels on the caller's stream. No allocation, no
// synchronisation, no state kept between calls.
#include <hip/hip_runtime.h>

#include "../../include/lcr.h"
#include "launch.h"
#include "validate.h"

using namespace lcr;

static RouteDims to_route_dims(const lcr_dims* d) {
  RouteDims r;
  r.B = d->B;
  r.Hq = d->Hq;
  r.Hkv = d->Hkv;
  r.N = d->N;
  r.d = d->d;
  r.dtype = d->dtype;
  return r;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? LCR_OK : LCR_ERR_HIP; }

extern "C" {

int lcr_version(void) { return 10000; }

const char* lcr_status_string(int status) {
  switch (status) {
    case LCR_OK: return "ok";
    case LCR_ERR_ARG: return "invalid argument";
    case LCR_ERR_DTYPE: return "invalid dtype";
    case LCR_ERR_WORKSPACE: return "workspace missing or too small";
    case LCR_ERR_HIP: return "HIP runtime error";
    case LCR_ERR_UNSUPPORTED: return "outside this library's limits";
    default: return "unknown status";
  }
}

int lcr_set_wait_limit(int polls) { return set_wait_limit(polls); }

int lcr_set_tile_order(int reversed) { return set_tile_order(reversed); }

size_t lcr_workspace_bytes(int op, const lcr_dims* dims, int D, int r, int K, int radius, int nq) {
  if (check_dims(dims) != LCR_OK || K < 0 || nq < 0 || radius < 0) return 0;
  const RouteDims dm = to_route_dims(dims);
  switch (op) {
    case LCR_OP_ROUTE_SCORE_TOPK:
      return (K > 0 && nq > 0 && D > 0 && r > 0 && r <= 128) ? score_ws_bytes(dm, D, r, nq, K) : 0;
    case LCR_OP_ROUTED_ATTENTION:
      return nq > 0 ? plan_routed_attention(dm, K, radius, nq).ws : 0;
    case LCR_OP_ROUTED_ATTENTION_BACKWARD:
      return routed_bwd_ws_bytes(dm, K, nq);
    case LCR_OP_ROUTE_SCORE_BACKWARD:
      return (D > 0 && r > 0 && r <= 128) ? score_bwd_ws_bytes(dm, D, r, K, nq) : 0;
    default:
      return 0;
  }
}

int lcr_chunk_summary(const lcr_dims* dims, const void* q, const void* k, float scale, float* s, float* H,
                      void* stream) {
  const int st = check_chunk_summary(dims, q, k, scale, s, H);
  if (st != LCR_OK) return st;
  return hip_status(launch_chunk_summary(to_route_dims(dims), q, k, scale, s, H, 0, dims->N, (hipStream_t)stream));
}

int lcr_chunk_summary_mean(const lcr_dims* dims, const void* k, float* s, float* H, void* stream) {
  const int st = check_chunk_summary_mean(dims, k, s, H);
  if (st != LCR_OK) return st;
  return hip_status(launch_chunk_summary_mean(to_route_dims(dims), k, s, H, (hipStream_t)stream));
}

int lcr_chunk_summary_range(const lcr_dims* dims, const void* q, const void* k, float scale, int c0, int nc,
                            float* s, float* H, void* stream) {
  int st = check_chunk_summary(dims, q, k, scale, s, H);
  if (st != LCR_OK) return st;
  st = check_chunk_range(dims, c0, nc);
  if (st != LCR_OK) return st;
  if (nc == 0) return LCR_OK;
  return hip_status(launch_chunk_summary(to_route_dims(dims), q, k, scale, s, H, c0, nc, (hipStream_t)stream));
}

int lcr_route_score_topk(const lcr_dims* dims, const void* q, const void* x, const void* A, const void* Bm,
                         int D, int r, const float* s, const float* H, float beta, float scale, int K,
                         int radius, int q0, int nq, int32_t* idx, float* zsel, void* ws, size_t ws_bytes,
                         void* stream) {
  const int st = check_route_score_topk(dims, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel);
  if (st != LCR_OK) return st;
  if (K == 0 || nq == 0) return LCR_OK;
  const RouteDims dm = to_route_dims(dims);
  const size_t need = score_ws_bytes(dm, D, r, nq, K);
  if (ws == nullptr || ws_bytes < need) return LCR_ERR_WORKSPACE;
  return hip_status(launch_route_score_topk(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx,
                                            zsel, score_ws_carve(ws, dm, D, r, nq, K), (hipStream_t)stream));
}

int lcr_routed_attention(const lcr_dims* dims, const void* q, const void* k, const void* v, const int32_t* idx,
                         const float* zsel, int K, int radius, float scale, int q0, int nq, void* o, float* lse,
                         void* ws, size_t ws_bytes, void* stream) {
  const int st = check_routed_attention(dims, q, k, v, idx, zsel, K, radius, scale, q0, nq, o);
  if (st != LCR_OK) return st;
  if (nq == 0) return LCR_OK;
  const RouteDims dm = to_route_dims(dims);
  const AttnPlan plan = plan_routed_attention(dm, K, radius, nq);
  if (plan.lds > routed_lds_limit()) return LCR_ERR_UNSUPPORTED;
  if (plan.ws > 0 && (ws == nullptr || ws_bytes < plan.ws)) return LCR_ERR_WORKSPACE;
  return hip_status(launch_routed_attention(dm, plan, q, k, v, K > 0 ? idx : nullptr, K > 0 ? zsel : nullptr, K,
                                            radius, scale, q0, nq, o, lse, ws, (hipStream_t)stream));
}

int lcr_routed_attention_noalloc(const lcr_dims* dims, const void* q, const void* k, const void* v,
                                 const int32_t* idx, const float* zsel, int K, int radius, float scale, int q0,
                                 int nq, void* o, float* lse, void* stream) {
  const int st = check_routed_attention(dims, q, k, v, idx, zsel, K, radius, scale, q0, nq, o);
  if (st != LCR_OK) return st;
  if (nq == 0) return LCR_OK;
  const RouteDims dm = to_route_dims(dims);
  const AttnPlan plan = plan_routed_attention(dm, K, radius, nq);
  if (plan.lds > routed_lds_limit()) return LCR_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (plan.ws > 0) {
    if (plan.ws > routed_scratch_bytes()) return LCR_ERR_UNSUPPORTED;
    if (routed_scratch(&ws) != hipSuccess) return LCR_ERR_HIP;
  }
  return hip_status(launch_routed_attention(dm, plan, q, k, v, K > 0 ? idx : nullptr, K > 0 ? zsel : nullptr, K,
                                            radius, scale, q0, nq, o, lse, ws, (hipStream_t)stream));
}

int lcr_routed_attention_backward(const lcr_dims* dims, const void* q, const void* k, const void* v,
                                  const int32_t* idx, const float* zsel, int K, int radius, float scale, int q0,
                                  int nq, const void* o, const float* lse, const void* dO, float* dq, float* dk,
                                  float* dv, float* dzsel, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_routed_attention_backward(dims, q, k, v, idx, zsel, K, radius, scale, q0, nq, o, lse, dO,
                                                 dq, dk, dv, dzsel);
  if (st != LCR_OK) return st;
  const RouteDims dm = to_route_dims(dims);
  const size_t need = routed_bwd_ws_bytes(dm, K, nq);
  if (ws == nullptr || ws_bytes < need) return LCR_ERR_WORKSPACE;
  return hip_status(launch_routed_attention_backward(dm, q, k, v, K > 0 ? idx : nullptr, K > 0 ? zsel : nullptr, K,
                                                     radius, scale, q0, nq, o, lse, dO, dq, dk, dv,
                                                     K > 0 ? dzsel : nullptr, ws, (hipStream_t)stream));
}

int lcr_route_score_backward(const lcr_dims* dims, const void* q, const void* x, const void* A, const void* Bm, int D,
                             int r, const float* s, float beta, float scale, int K, int q0, int nq, const int32_t* idx,
                             const float* dzsel, float* dq, float* dx, float* dA, float* dBm, float* ds, float* dH,
                             void* ws, size_t ws_bytes, void* stream) {
  const int st = check_route_score_backward(dims, q, x, A, Bm, D, r, s, beta, scale, K, q0, nq, idx, dzsel, dq, dx,
                                            dA, dBm, ds, dH);
  if (st != LCR_OK) return st;
  const RouteDims dm = to_route_dims(dims);
  if (ws == nullptr || ws_bytes < score_bwd_ws_bytes(dm, D, r, K, nq)) return LCR_ERR_WORKSPACE;
  return hip_status(launch_route_score_backward(dm, q, x, A, Bm, D, r, s, beta, scale, K, q0, nq,
                                                K > 0 ? idx : nullptr, K > 0 ? dzsel : nullptr, dq, dx, dA, dBm, ds,
                                                dH, ws, (hipStream_t)stream));
}

int lcr_chunk_summary_backward(const lcr_dims* dims, const void* q, const void* k, float scale, const float* ds,
                               const float* dH, float* dq, float* dk, void* stream) {
  int st = check_chunk_summary(dims, q, k, scale, ds, dH);
  if (st != LCR_OK) return st;
  if (!dq || !dk) return LCR_ERR_ARG;
  return hip_status(
      launch_chunk_summary_backward(to_route_dims(dims), q, k, scale, ds, dH, dq, dk, (hipStream_t)stream));
}

int lcr_swa_attention(int B, int Hq, int Hkv, int L, int d, int dtype, const void* q, const void* k, const void* v,
                      int radius, float scale, void* o, float* lse, void* stream) {
  const int st = check_swa(B, Hq, Hkv, L, d, dtype, q, k, v, radius, scale, o);
  if (st != LCR_OK) return st;
  if (swa_lds_bytes(d, dtype) > routed_lds_limit()) return LCR_ERR_UNSUPPORTED;
  return hip_status(
      launch_swa_attention(B, Hq, Hkv, L, d, dtype, q, k, v, radius, scale, o, lse, (hipStream_t)stream));
}

}  // extern "C"
