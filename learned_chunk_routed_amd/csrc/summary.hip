// Chunk summaries: mask-query pooling of each chunk's 63 content keys.
// "Prefilling-dLLM v2: Learned Chunk Routing for Long-Context Diffusion Language
// Models", Figure 3 caption: the routing mask's query pools the content keys
// with an intra-chunk softmax; the weighted sum is the summary key. "The 172x
// Speedup Has an Evidence Budget", section "How learned routing controls what
// the model can read": the entropy of the pooling weights ranks chunks too.
//
// One 64-lane wave per (batch, KV head, chunk): the chunk's keys are read from
// HBM once into LDS (float32, padded rows so lane j reading row j is bank-
// conflict free) and serve the G mask queries of the group. Lane j < 63 owns
// content key j for the logits; for the weighted sum lanes own output columns.
// Work is tiny next to the routed attention (4*63*d flops per head and chunk),
// so plain float32 VALU arithmetic with exact expf/logf is used.
#include "device.h"
#include "launch.h"

namespace lcr {

template <typename T, int D>
__global__ __launch_bounds__(64) void chunk_summary_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ k, float scale,
                                                           float* __restrict__ s,
                                                           float* __restrict__ Hout, int Hq,
                                                           int Hkv, int N) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = Hq / Hkv;
  const size_t L = (size_t)N * kSlots;
  __shared__ float ks[kContent][D + 1];
  __shared__ float qs[D];
  __shared__ float al[64];

  const T* kc = k + (((size_t)b * Hkv + g) * L + (size_t)c * kSlots) * D;
  for (int e = lane; e < kContent * D; e += 64) ks[e / D][e % D] = Elem<T>::to_f(kc[e]);
  __syncthreads();

  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const T* qm = q + (((size_t)b * Hq + h) * L + (size_t)c * kSlots + (kSlots - 1)) * D;
    for (int e = lane; e < D; e += 64) qs[e] = Elem<T>::to_f(qm[e]);
    __syncthreads();
    float logit = -INFINITY;
    if (lane < kContent) {
      float acc = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) acc = fmaf(qs[e], ks[lane][e], acc);
      logit = scale * acc;
    }
    const float m = wave_max(logit);
    const float ex = lane < kContent ? expf(logit - m) : 0.f;
    const float sum = wave_sum(ex);
    const float a = ex / sum;
    // H = -sum a ln a = ln(sum) - sum a (logit - m), with ln a = logit - m - ln(sum)
    const float Hv = logf(sum) - wave_sum(lane < kContent ? a * (logit - m) : 0.f);
    al[lane] = a;
    __syncthreads();
    float* so = s + (((size_t)b * Hq + h) * N + c) * D;
    for (int e = lane; e < D; e += 64) {
      float acc = 0.f;
#pragma unroll 9
      for (int j = 0; j < kContent; ++j) acc = fmaf(al[j], ks[j][e], acc);
      so[e] = acc;
    }
    if (lane == 0) Hout[((size_t)b * Hq + h) * N + c] = Hv;
    __syncthreads();
  }
}

template <typename T, int D>
static hipError_t launch_summary_t(const RouteDims& dm, const void* q, const void* k, float scale,
                                   float* s, float* H, hipStream_t st) {
  dim3 grid(dm.N, dm.Hkv, dm.B);
  hipLaunchKernelGGL((chunk_summary_kernel<T, D>), grid, dim3(64), 0, st, (const T*)q,
                     (const T*)k, scale, s, H, dm.Hq, dm.Hkv, dm.N);
  return hipGetLastError();
}

hipError_t launch_chunk_summary(const RouteDims& dm, const void* q, const void* k, float scale,
                                float* s, float* H, hipStream_t st) {
  if (dm.dtype == 1) {
    return dm.d == 64 ? launch_summary_t<bf16_t, 64>(dm, q, k, scale, s, H, st)
                      : launch_summary_t<bf16_t, 128>(dm, q, k, scale, s, H, st);
  }
  return dm.d == 64 ? launch_summary_t<float, 64>(dm, q, k, scale, s, H, st)
                    : launch_summary_t<float, 128>(dm, q, k, scale, s, H, st);
}

}  // namespace lcr
