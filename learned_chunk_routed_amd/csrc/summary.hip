// Chunk summaries: mask-query pooling of each chunk's 63 content keys.
// "Prefilling-dLLM v2: Learned Chunk Routing for Long-Context Diffusion Language
// Models", Figure 3 caption: the routing mask's query pools the content keys
// with an intra-chunk softmax; the weighted sum is the summary key. "The 172x
// Speedup Has an Evidence Budget", section "How learned routing controls what
// the model can read": the entropy of the pooling weights ranks chunks too.
//
// One block of four waves per (batch, KV head, chunk of the requested range c0 ..):
// the chunk's keys are read
// from HBM once into LDS with 16-byte loads (float32 rows 4 banks apart, so that lane j
// reading row j with 16-byte LDS reads is bank-conflict free) and serve the G mask queries of the group,
// wave w taking heads w, w + 4, ... Lane j < 63 owns content key j for the logits
// (four independent partial sums over d); for the weighted sum lanes own output
// columns. Work is tiny next to the routed attention (4*63*d flops per head and
// chunk), so plain float32 VALU arithmetic with exact expf/logf is used.
#include "device.h"
#include "launch.h"

namespace lcr {

constexpr int kSumWaves = 4;

// MEAN: the mean-summary ablation ("Prefilling-dLLM v2", Table 6, row "Mean
// summary"): every pooling logit is zero, so the weights are uniform (1/63), s is
// the mean content key and H = ln 63; q is not read.
template <typename T, int D, bool MEAN>
__global__ __launch_bounds__(64 * kSumWaves) void chunk_summary_kernel(const T* __restrict__ q,
                                                                       const T* __restrict__ k, float scale,
                                                                       float* __restrict__ s,
                                                                       float* __restrict__ Hout, int Hq, int Hkv,
                                                                       int N, int c0) {
  const int c = c0 + blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = Hq / Hkv;
  const size_t L = (size_t)N * kSlots;
  constexpr int VE = 16 / sizeof(T);   // elements per 16-byte load
  __shared__ __align__(16) float ks[kContent][D + 4];   // rows 16-byte aligned, 4 banks apart
  __shared__ __align__(16) float qs[kSumWaves][D];
  __shared__ float al[kSumWaves][64];

  const T* kc = k + (((size_t)b * Hkv + g) * L + (size_t)c * kSlots) * D;
  for (int e = VE * tid; e < kContent * D; e += VE * 64 * kSumWaves) {
    typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
    const u32x4 v = *reinterpret_cast<const u32x4*>(kc + e);
    const T* pv = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int j = 0; j < VE; ++j) ks[(e + j) / D][(e + j) % D] = Elem<T>::to_f(pv[j]);
  }
  __syncthreads();

  for (int hh = w; hh < G; hh += kSumWaves) {
    const int h = g * G + hh;
    float logit = -INFINITY;
    if constexpr (MEAN) {
      if (lane < kContent) logit = 0.f;
    } else {
      const T* qm = q + (((size_t)b * Hq + h) * L + (size_t)c * kSlots + (kSlots - 1)) * D;
      for (int e = lane; e < D; e += 64) qs[w][e] = Elem<T>::to_f(qm[e]);
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the row is in LDS for the whole wave
      __builtin_amdgcn_wave_barrier();
    }
    if (!MEAN && lane < kContent) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int e = 0; e < D; e += 4) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(&qs[w][e]);
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&ks[lane][e]);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = fmaf(qv[u], kv[u], acc[u]);
      }
      logit = scale * ((acc[0] + acc[1]) + (acc[2] + acc[3]));
    }
    const float m = wave_max(logit);
    const float ex = lane < kContent ? expf(logit - m) : 0.f;
    const float sum = wave_sum(ex);
    const float a = ex / sum;
    // H = -sum a ln a = ln(sum) - sum a (logit - m), with ln a = logit - m - ln(sum)
    const float Hv = logf(sum) - wave_sum(lane < kContent ? a * (logit - m) : 0.f);
    al[w][lane] = a;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    float* so = s + (((size_t)b * Hq + h) * N + c) * D;
    for (int e = lane; e < D; e += 64) {
      float acc[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kContent; j += 3)
#pragma unroll
        for (int u = 0; u < 3; ++u) acc[u] = fmaf(al[w][j + u], ks[j + u][e], acc[u]);
      so[e] = (acc[0] + acc[1]) + acc[2];
    }
    if (lane == 0) Hout[((size_t)b * Hq + h) * N + c] = Hv;
    __builtin_amdgcn_wave_barrier();   // this wave's rows of qs and al are reused by its next head
  }
}

template <typename T, int D, bool MEAN>
static hipError_t launch_summary_t(const RouteDims& dm, const void* q, const void* k, float scale,
                                   float* s, float* H, int c0, int nc, hipStream_t st) {
  dim3 grid(nc, dm.Hkv, dm.B);
  hipLaunchKernelGGL((chunk_summary_kernel<T, D, MEAN>), grid, dim3(64 * kSumWaves), 0, st, (const T*)q,
                     (const T*)k, scale, s, H, dm.Hq, dm.Hkv, dm.N, c0);
  return hipGetLastError();
}

template <bool MEAN>
static hipError_t launch_summary_m(const RouteDims& dm, const void* q, const void* k, float scale,
                                   float* s, float* H, int c0, int nc, hipStream_t st) {
  if (dm.dtype == 1) {
    return dm.d == 64 ? launch_summary_t<bf16_t, 64, MEAN>(dm, q, k, scale, s, H, c0, nc, st)
                      : launch_summary_t<bf16_t, 128, MEAN>(dm, q, k, scale, s, H, c0, nc, st);
  }
  return dm.d == 64 ? launch_summary_t<float, 64, MEAN>(dm, q, k, scale, s, H, c0, nc, st)
                    : launch_summary_t<float, 128, MEAN>(dm, q, k, scale, s, H, c0, nc, st);
}

hipError_t launch_chunk_summary(const RouteDims& dm, const void* q, const void* k, float scale,
                                float* s, float* H, int c0, int nc, hipStream_t st) {
  return launch_summary_m<false>(dm, q, k, scale, s, H, c0, nc, st);
}

hipError_t launch_chunk_summary_mean(const RouteDims& dm, const void* k, float* s, float* H, hipStream_t st) {
  return launch_summary_m<true>(dm, nullptr, k, 0.f, s, H, 0, dm.N, st);
}

}  // namespace lcr
