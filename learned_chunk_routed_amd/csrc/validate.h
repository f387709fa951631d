// Host-side argument checks for every C entry point. Pure C++ (no HIP), so the
// rules can be exercised on a machine without a GPU: each check returns an
// lcr_status and the entry points call nothing else before a check passes.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/lcr.h"

namespace lcr {

int check_dims(const lcr_dims* d);
int check_chunk_range(const lcr_dims* d, int c0, int nc);
int check_chunk_summary_mean(const lcr_dims* d, const void* k, const float* s, const float* H);
int check_chunk_summary(const lcr_dims* d, const void* q, const void* k, float scale, const float* s,
                        const float* H);
int check_route_score_topk(const lcr_dims* d, const void* q, const void* x, const void* A, const void* Bm,
                           int D, int r, const float* s, const float* H, float beta, float scale, int K,
                           int radius, int q0, int nq, const int32_t* idx, const float* zsel);
int check_routed_attention(const lcr_dims* d, const void* q, const void* k, const void* v,
                           const int32_t* idx, const float* zsel, int K, int radius, float scale, int q0,
                           int nq, const void* o);
int check_routed_attention_backward(const lcr_dims* d, const void* q, const void* k, const void* v,
                                    const int32_t* idx, const float* zsel, int K, int radius, float scale,
                                    int q0, int nq, const void* o, const float* lse, const void* dO,
                                    const float* dq, const float* dk, const float* dv, const float* dzsel);
int check_route_score_backward(const lcr_dims* d, const void* q, const void* x, const void* A, const void* Bm,
                               int D, int r, const float* s, float beta, float scale, int K, int q0, int nq,
                               const int32_t* idx, const float* dzsel, const float* dq, const float* dx,
                               const float* dA, const float* dBm, const float* ds, const float* dH);
int check_swa(int B, int Hq, int Hkv, int L, int d, int dtype, const void* q, const void* k, const void* v,
              int radius, float scale, const void* o);

// Largest N the top-K kernel handles (64 chunks per lane step, 64 steps).
constexpr int kMaxChunksTopK = 4096;

// Largest N the backward's inverse index handles (one int per chunk in LDS).
constexpr int kMaxChunksBackward = 32768;

}  // namespace lcr
