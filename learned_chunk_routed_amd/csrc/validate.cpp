// Host-side argument checks (see validate.h). No HIP dependency.
#include "validate.h"

#include <cmath>
#include <limits>

namespace lcr {

static bool finite(float x) { return std::isfinite(x); }

int check_dims(const lcr_dims* d) {
  if (d == nullptr) return LCR_ERR_ARG;
  if (d->dtype != LCR_F32 && d->dtype != LCR_BF16) return LCR_ERR_DTYPE;
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->N < 1 || d->d < 1) return LCR_ERR_ARG;
  if (d->Hq % d->Hkv != 0) return LCR_ERR_ARG;
  if (d->d != 64 && d->d != 128) return LCR_ERR_UNSUPPORTED;
  if (d->Hq / d->Hkv > LCR_MAX_GROUP) return LCR_ERR_UNSUPPORTED;
  // 64*N slots must be indexable and the grids must fit.
  if ((long long)d->N * LCR_CHUNK_SLOTS > (long long)std::numeric_limits<int>::max()) return LCR_ERR_ARG;
  if ((long long)d->B * d->Hkv > 65535) return LCR_ERR_UNSUPPORTED;
  return LCR_OK;
}

int check_chunk_summary(const lcr_dims* d, const void* q, const void* k, float scale, const float* s,
                        const float* H) {
  int st = check_dims(d);
  if (st != LCR_OK) return st;
  if (!q || !k || !s || !H) return LCR_ERR_ARG;
  if (!finite(scale)) return LCR_ERR_ARG;
  return LCR_OK;
}

int check_chunk_summary_mean(const lcr_dims* d, const void* k, const float* s, const float* H) {
  int st = check_dims(d);
  if (st != LCR_OK) return st;
  if (!k || !s || !H) return LCR_ERR_ARG;
  return LCR_OK;
}

int check_chunk_range(const lcr_dims* d, int c0, int nc) {
  if (c0 < 0 || nc < 0 || (long long)c0 + nc > d->N) return LCR_ERR_ARG;
  return LCR_OK;
}

static int check_query_range(const lcr_dims* d, int q0, int nq) {
  const long long T = (long long)d->N * LCR_CHUNK_CONTENT;
  if (q0 < 0 || nq < 0) return LCR_ERR_ARG;
  if ((long long)q0 + nq > T) return LCR_ERR_ARG;
  return LCR_OK;
}

int check_route_score_topk(const lcr_dims* d, const void* q, const void* x, const void* A, const void* Bm,
                           int D, int r, const float* s, const float* H, float beta, float scale, int K,
                           int radius, int q0, int nq, const int32_t* idx, const float* zsel) {
  int st = check_dims(d);
  if (st != LCR_OK) return st;
  if (D < 1 || r < 1) return LCR_ERR_ARG;
  if (r > 128) return LCR_ERR_UNSUPPORTED;
  if (K < 0 || radius < 0) return LCR_ERR_ARG;
  if (K > LCR_MAX_TOPK) return LCR_ERR_UNSUPPORTED;
  if (!finite(beta) || !finite(scale)) return LCR_ERR_ARG;
  st = check_query_range(d, q0, nq);
  if (st != LCR_OK) return st;
  if (K > 0 && nq > 0) {
    if (!q || !x || !A || !Bm || !s || !H || !idx || !zsel) return LCR_ERR_ARG;
    if (d->N > kMaxChunksTopK) return LCR_ERR_UNSUPPORTED;
  }
  return LCR_OK;
}

int check_routed_attention(const lcr_dims* d, const void* q, const void* k, const void* v,
                           const int32_t* idx, const float* zsel, int K, int radius, float scale, int q0,
                           int nq, const void* o) {
  int st = check_dims(d);
  if (st != LCR_OK) return st;
  if (K < 0 || radius < 0) return LCR_ERR_ARG;
  if (K > LCR_MAX_TOPK) return LCR_ERR_UNSUPPORTED;
  if (!finite(scale)) return LCR_ERR_ARG;
  st = check_query_range(d, q0, nq);
  if (st != LCR_OK) return st;
  if (nq > 0) {
    if (!q || !k || !v || !o) return LCR_ERR_ARG;
    if (K > 0 && (!idx || !zsel)) return LCR_ERR_ARG;
  }
  return LCR_OK;
}

int check_routed_attention_backward(const lcr_dims* d, const void* q, const void* k, const void* v,
                                    const int32_t* idx, const float* zsel, int K, int radius, float scale,
                                    int q0, int nq, const void* o, const float* lse, const void* dO,
                                    const float* dq, const float* dk, const float* dv, const float* dzsel) {
  int st = check_routed_attention(d, q, k, v, idx, zsel, K, radius, scale, q0, nq, o);
  if (st != LCR_OK) return st;
  if (!dk || !dv) return LCR_ERR_ARG;
  if (nq > 0) {
    if (!lse || !dO || !dq) return LCR_ERR_ARG;
    if (K > 0 && !dzsel) return LCR_ERR_ARG;
  }
  // entry lists index nq*K entries per (batch, group) with int32; per-tile chunk counts live in LDS
  if ((long long)nq * K > (long long)std::numeric_limits<int>::max()) return LCR_ERR_UNSUPPORTED;
  if (d->N > kMaxChunksBackward) return LCR_ERR_UNSUPPORTED;
  return LCR_OK;
}

int check_route_score_backward(const lcr_dims* d, const void* q, const void* x, const void* A, const void* Bm,
                               int D, int r, const float* s, float beta, float scale, int K, int q0, int nq,
                               const int32_t* idx, const float* dzsel, const float* dq, const float* dx,
                               const float* dA, const float* dBm, const float* ds, const float* dH) {
  int st = check_dims(d);
  if (st != LCR_OK) return st;
  if (D < 1 || r < 1 || K < 0) return LCR_ERR_ARG;
  if (r > 128) return LCR_ERR_UNSUPPORTED;
  if (K > LCR_MAX_TOPK) return LCR_ERR_UNSUPPORTED;
  if (!finite(beta) || !finite(scale)) return LCR_ERR_ARG;
  st = check_query_range(d, q0, nq);
  if (st != LCR_OK) return st;
  if (!A || !Bm || !dA || !dBm || !ds || !dH) return LCR_ERR_ARG;
  if (nq > 0) {
    if (!q || !x || !s || !dq || !dx) return LCR_ERR_ARG;
    if (K > 0 && (!idx || !dzsel)) return LCR_ERR_ARG;
  }
  if ((long long)nq * K > (long long)std::numeric_limits<int>::max()) return LCR_ERR_UNSUPPORTED;
  if ((long long)d->B * nq > (long long)std::numeric_limits<int>::max() / 2) return LCR_ERR_UNSUPPORTED;
  if (d->N > kMaxChunksBackward) return LCR_ERR_UNSUPPORTED;
  return LCR_OK;
}

int check_swa(int B, int Hq, int Hkv, int L, int d, int dtype, const void* q, const void* k, const void* v,
              int radius, float scale, const void* o) {
  if (dtype != LCR_F32 && dtype != LCR_BF16) return LCR_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || d < 1 || radius < 0) return LCR_ERR_ARG;
  if (Hq % Hkv != 0) return LCR_ERR_ARG;
  if (d != 64 && d != 128) return LCR_ERR_UNSUPPORTED;
  if (Hq / Hkv > LCR_MAX_GROUP) return LCR_ERR_UNSUPPORTED;
  if ((long long)B * Hkv > 65535) return LCR_ERR_UNSUPPORTED;
  if (!finite(scale)) return LCR_ERR_ARG;
  if (!q || !k || !v || !o) return LCR_ERR_ARG;
  return LCR_OK;
}

}  // namespace lcr
