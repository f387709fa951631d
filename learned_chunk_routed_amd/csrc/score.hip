// Residual-augmented summary scoring, GQA maximum and exact top-K selection.
// "Prefilling-dLLM v2: Learned Chunk Routing for Long-Context Diffusion Language
// Models", Figure 3 caption: a content query adds a low-rank residual and scores
// the summaries; the scores are reduced by a maximum inside each GQA group and
// the top K chunks are shared by every head of the group. Table 3: the remote
// chunks are gathered beyond the local window. "The 172x Speedup Has an Evidence
// Budget": rank-64 residual; similarity and pooling entropy rank the chunks.
//
// Paths, chosen by problem size and dtype:
//  - general (float32 inputs, or bf16 beyond the fused path's limits):
//    u_kernel + q_kernel (u = x A, then q~ = q + u B per head with u split into
//    bf16 hi + lo), score_kernel (z = scale * q~ . s - beta * H per head on MFMA
//    with both operands split into bf16 planes: hi.hi + hi.lo + lo.hi for bf16
//    inputs, hi + mid + lo for float32; float32 accumulation, so the top-K set
//    matches an exact computation wherever the K-th/(K+1)-th margin is not tiny;
//    plus the group maximum), topk_kernel (one wave per (batch, group, query):
//    bisection on an order-preserving key with ballot counts, ties to the
//    smaller index; zsel gathered from the per-head scores);
//  - bf16 prefill (section 1d and 4): u_stream_kernel, then route_score3_kernel
//    from q~ to idx and zsel without per-head scores in memory;
//  - bf16 decode-sized, at most 32 queries (section 5).
#include "device.h"
#include "launch.h"

namespace lcr {

__device__ __forceinline__ long long slot_of(long long i) { return (i / kContent) * kSlots + (i % kContent); }

// Load 8 consecutive elements [k, k+8) of a row of length n as floats (zero beyond n).
template <typename T>
__device__ __forceinline__ void load_row8(const T* row, long long k, long long n, float* out) {
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = (k + j < n) ? Elem<T>::to_f(row[k + j]) : 0.f;
}
template <>
__device__ __forceinline__ void load_row8<bf16_t>(const bf16_t* row, long long k, long long n, float* out) {
  if (k + 8 <= n && ((k & 7) == 0) && ((((uintptr_t)row) & 15) == 0)) {
    s16x8 v = load8(row + k);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = bf2f((bf16_t)v[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = (k + j < n) ? bf2f(row[k + j]) : 0.f;
  }
}

// ---------------------------------------------------------------------------- 1. q~
//
// 1a. u_kernel: partial u = x[rows] A over a range of the hidden dimension.
//     Block = 4 waves x 16 rows. A is staged through LDS in 64-row slices
//     (bf16 planes; row stride RP+16 keeps the transpose reads conflict free)
//     with the next slice prefetched into registers; x fragments come straight
//     from HBM (16 bytes per lane). Small query counts split the hidden
//     dimension over several blocks (grid.z); q_kernel sums the partials.
// 1b. q_kernel: q~ = q + u B_h for one head per block. B's slice for the head
//     is staged into LDS; u is split into bf16 hi + lo (B is exact for bf16
//     inputs; float32 inputs also split B).

constexpr int kUKc = 64;   // rows of A per LDS slice

template <typename T, int RP>
__global__ __launch_bounds__(256) void u_kernel(const T* __restrict__ x, const T* __restrict__ A, int Dh, int r,
                                                float* __restrict__ upart, int N, int q0, int nq, int kslices_per_split) {
  constexpr bool kSplit = sizeof(T) == 4;
  constexpr int NPL = kSplit ? 2 : 1;
  constexpr int AS = RP + 16;
  constexpr int kElems = kUKc * RP;                 // elements per slice
  constexpr int kPer = (kElems + 255) / 256;        // elements per thread per slice
  __shared__ __align__(16) bf16_t a_s[NPL][kUKc * AS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4, L16 = lane & 15;
  const int b = blockIdx.y, split = blockIdx.z;
  const int t0 = blockIdx.x * 64 + 16 * w;
  const long long L = (long long)N * kSlots;
  const int nslices = (Dh + kUKc - 1) / kUKc;
  const int sl_beg = split * kslices_per_split;
  const int sl_end = min(nslices, sl_beg + kslices_per_split);

  const int my_t = t0 + L16;
  const T* xrow = (my_t < nq) ? x + ((size_t)b * L + slot_of((long long)q0 + my_t)) * Dh : nullptr;

  f32x4 acc[RP / 16];
#pragma unroll
  for (int nt = 0; nt < RP / 16; ++nt) acc[nt] = zero4();

  float pre[kPer];
  auto fetch = [&](int sl) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = tid + 256 * j;
      const int kk = e / RP, n = e - kk * RP;
      const int k = sl * kUKc + kk;
      pre[j] = (e < kElems && k < Dh && n < r) ? Elem<T>::to_f(A[(size_t)k * r + n]) : 0.f;
    }
  };
  if (sl_beg < sl_end) fetch(sl_beg);
  for (int sl = sl_beg; sl < sl_end; ++sl) {
    __syncthreads();   // previous slice fully consumed
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = tid + 256 * j;
      if (e < kElems) {
        const int kk = e / RP, n = e - kk * RP;
        if (kSplit) {
          bf16_t h, l;
          split_bf16(pre[j], h, l);
          a_s[0][kk * AS + n] = h;
          a_s[NPL - 1][kk * AS + n] = l;
        } else {
          a_s[0][kk * AS + n] = f2bf(pre[j]);
        }
      }
    }
    __syncthreads();
    if (sl + 1 < sl_end) fetch(sl + 1);
#pragma unroll
    for (int ks = 0; ks < kUKc / 32; ++ks) {
      const int k0 = sl * kUKc + 32 * ks;
      float xv[8];
      if (xrow) load_row8<T>(xrow, k0 + 8 * g16, Dh, xv);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = 0.f;
      }
      s16x8 xh, xl;
      if (kSplit) pack8_split_hw(xv, xh, xl);
      else xh = pack8(xv);
#pragma unroll
      for (int nt = 0; nt < RP / 16; ++nt) {
        const s16x8 bh = lds_col_frag(a_s[0], AS, 32 * ks + 8 * g16, 32 * ks + 8 * g16 + 4, 16 * nt, lane);
        if (kSplit) {
          const s16x8 bl = lds_col_frag(a_s[NPL - 1], AS, 32 * ks + 8 * g16, 32 * ks + 8 * g16 + 4, 16 * nt, lane);
          acc[nt] = mfma16(xh, bl, acc[nt]);
          acc[nt] = mfma16(xl, bh, acc[nt]);
        }
        acc[nt] = mfma16(xh, bh, acc[nt]);
      }
    }
  }
  // D layout: lane holds u[row 4*g16 + i][col 16*nt + L16] of this wave's 16 rows
  float* up = upart + ((size_t)split * gridDim.y + b) * (size_t)nq * RP;
#pragma unroll
  for (int nt = 0; nt < RP / 16; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g16 + i;
      if (t < nq) up[(size_t)t * RP + 16 * nt + L16] = acc[nt][i];
    }
}

template <typename T, int D, int RP>
__global__ __launch_bounds__(256) void q_kernel(const T* __restrict__ q, const T* __restrict__ Bm, int r,
                                                const float* __restrict__ upart, int nsplit,
                                                float* __restrict__ qt, int Hq, int N, int q0, int nq) {
  constexpr bool kSplit = sizeof(T) == 4;
  constexpr int NPL = kSplit ? 2 : 1;
  constexpr int BS = D + 16;
  __shared__ __align__(16) bf16_t b_s[NPL][RP * BS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4, L16 = lane & 15;
  const int h = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * 64 + 16 * w;
  const long long L = (long long)N * kSlots;
  const int B = gridDim.z;

  for (int e = tid; e < RP * D; e += 256) {
    const int kk = e / D, n = e - kk * D;
    const float val = (kk < r) ? Elem<T>::to_f(Bm[(size_t)kk * Hq * D + (size_t)h * D + n]) : 0.f;
    if (kSplit) {
      bf16_t hh, ll;
      split_bf16(val, hh, ll);
      b_s[0][kk * BS + n] = hh;
      b_s[NPL - 1][kk * BS + n] = ll;
    } else {
      b_s[0][kk * BS + n] = f2bf(val);
    }
  }
  // u fragments (A operand: row L16 of this wave, k = rank index), partials summed
  s16x8 uh[RP / 32], ul[RP / 32];
  const int my_t = t0 + L16;
#pragma unroll
  for (int ks = 0; ks < RP / 32; ++ks) {
    float uv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) uv[j] = 0.f;
    if (my_t < nq) {
      // partials in groups of 8 so that 16 loads are in flight at once
      const size_t sstride = (size_t)B * nq * RP;
      const float* up0 = upart + ((size_t)b * nq + my_t) * RP + 32 * ks + 8 * g16;
      int sp = 0;
      for (; sp + 8 <= nsplit; sp += 8) {
        f32x4 a[8][2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[e][0] = *reinterpret_cast<const f32x4*>(up0 + (sp + e) * sstride);
          a[e][1] = *reinterpret_cast<const f32x4*>(up0 + (sp + e) * sstride + 4);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uv[j] += a[e][0][j];
            uv[4 + j] += a[e][1][j];
          }
      }
      for (; sp < nsplit; ++sp) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(up0 + sp * sstride);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(up0 + sp * sstride + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uv[j] += a0[j];
          uv[4 + j] += a1[j];
        }
      }
    }
    pack8_split_hw(uv, uh[ks], ul[ks]);
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) {
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < RP / 32; ++ks) {
      const s16x8 bh = lds_col_frag(b_s[0], BS, 32 * ks + 8 * g16, 32 * ks + 8 * g16 + 4, 16 * nt, lane);
      acc = mfma16(ul[ks], bh, acc);
      if (kSplit) {
        const s16x8 bl = lds_col_frag(b_s[NPL - 1], BS, 32 * ks + 8 * g16, 32 * ks + 8 * g16 + 4, 16 * nt, lane);
        acc = mfma16(uh[ks], bl, acc);
      }
      acc = mfma16(uh[ks], bh, acc);
    }
    const int dd = 16 * nt + L16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g16 + i;
      if (t < nq) {
        const long long sl = slot_of((long long)q0 + t);
        const float qv = Elem<T>::to_f(q[((size_t)b * Hq + h) * L * D + (size_t)sl * D + dd]);
        qt[(((size_t)b * Hq + h) * nq + t) * D + dd] = qv + acc[i];
      }
    }
  }
}

// LDS block barrier that leaves vector-memory loads in flight: every wave's LDS
// accesses before it have completed; loads issued earlier keep running (__syncthreads
// would wait for them too).
__device__ __forceinline__ void lds_block_barrier() {
  wait_lgkm0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 1d. u_stream_kernel (bf16, prefill-sized): u = x A for 64 queries per block, 8
//     waves. x passes through LDS 256 columns (one stage) at a time: consecutive
//     threads load consecutive 16-byte pieces of one row, so every row is read as
//     512-byte runs (HBM serves scattered 64-byte pieces of thousands of rows at a
//     third of its bandwidth), with kUsPD stages of loads in flight in registers.
//     Wave w multiplies k-step w of each stage for all 64 rows against A transposed
//     (rows = rank, zero-padded to whole stages; plain 16-byte loads from L2, in
//     flight with the stage's x). The wave partials are summed through LDS and one
//     partial set is written (no split of the hidden dimension in memory).
constexpr int kUsPD = 2;               // stages of loads in flight per thread
constexpr int kUsCols = 256;           // x columns per stage (8 k-steps, one per wave)
constexpr int kUsRow = kUsCols + 8;    // LDS row stride of a staged x tile (elements)

template <int RP>
__global__ __launch_bounds__(256) void transpose_a_kernel(const bf16_t* __restrict__ A, int Dh, int r, int Dhp,
                                                          bf16_t* __restrict__ At) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)RP * Dhp) return;
  const int n = (int)(e / Dhp), k = (int)(e - (long long)n * Dhp);
  At[e] = (n < r && k < Dh) ? A[(size_t)k * r + n] : (bf16_t)0;
}

// B transposed for the fused scoring kernel: Bt[n][rr] = B[rr][n] for n < Hq * d,
// rank rr < RP (zero past r), so each head's q~ product reads rank-contiguous rows.
template <int D, int RP>
__global__ __launch_bounds__(256) void transpose_b_kernel(const bf16_t* __restrict__ Bm, int r, int HD,
                                                          bf16_t* __restrict__ Bt) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)HD * RP) return;
  const int n = (int)(e / RP), rr = (int)(e - (long long)n * RP);
  Bt[e] = rr < r ? Bm[(size_t)rr * HD + n] : (bf16_t)0;
}

template <int RP>
__global__ __launch_bounds__(512) void u_stream_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ At,
                                                       int Dh, int Dhp, float* __restrict__ upart, int N, int q0,
                                                       int nq) {
  constexpr int NTR = RP / 16;
  constexpr int US = RP + 4;
  constexpr int PPT = 64 * kUsCols / 8 / 512;   // 16-byte pieces of a stage per thread (4)
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem);       // [2][64][kUsRow] staged x
  float* red = reinterpret_cast<float*>(smem);        // after the walk: wave partials [8][64][US]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4, L16 = lane & 15;
  const int b = blockIdx.y, t0 = blockIdx.x * 64;
  const long long L = (long long)N * kSlots;
  const int nst = (Dhp + kUsCols - 1) / kUsCols;     // stages (the last one may be partial)
  // this thread's pieces: rows (tid >> 5) + 16 j, 8-column group tid & 31 of every stage;
  // rows past nq read the block's first row (never stored)
  const int c8 = 8 * (tid & 31);
  const bf16_t* xr[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int t = t0 + (tid >> 5) + 16 * j;
    xr[j] = x + ((size_t)b * L + slot_of((long long)q0 + (t < nq ? t : t0))) * Dh;
  }
  f32x4 acc[4][NTR];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTR; ++nt) acc[mt][nt] = zero4();
  s16x8 xv[kUsPD][PPT], av[kUsPD][NTR];
  // stage st into register slot p. Pieces past Dh read the row's first piece, which meets
  // the zero padding of the transposed A; k-steps past Dhp read A's first k-step and are
  // not multiplied. Nothing is masked, so no load waits for another.
  auto load = [&](int st, int p) {
    st = min(st, nst - 1);
    const int col = kUsCols * st + c8;
#pragma unroll
    for (int j = 0; j < PPT; ++j) xv[p][j] = load8(xr[j] + (col < Dh ? col : 0));
    const int kg = kUsCols * st + 32 * w + 8 * g16;
#pragma unroll
    for (int nt = 0; nt < NTR; ++nt) av[p][nt] = load8(At + (size_t)(16 * nt + L16) * Dhp + (kg < Dhp ? kg : 8 * g16));
  };
  // stage st (its x in slot p) through LDS buffer st & 1, then this wave's k-step of it
  auto step = [&](int st, int p) {
    bf16_t* xb = xs + (size_t)(st & 1) * 64 * kUsRow;
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      *reinterpret_cast<s16x8*>(xb + ((tid >> 5) + 16 * j) * kUsRow + c8) = xv[p][j];
    lds_block_barrier();   // the stage is in LDS; every wave is done with the buffer's previous stage
    s16x8 af[NTR];
#pragma unroll
    for (int nt = 0; nt < NTR; ++nt) af[nt] = av[p][nt];
    load(st + kUsPD, p);   // the slot is free: the next stage but kUsPD - 1 goes in flight
    if (kUsCols * st + 32 * w < Dhp) {   // wave-uniform: this wave's k-step exists
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const s16x8 xf = *reinterpret_cast<const s16x8*>(xb + (16 * mt + L16) * kUsRow + 32 * w + 8 * g16);
#pragma unroll
        for (int nt = 0; nt < NTR; ++nt) acc[mt][nt] = mfma16(xf, af[nt], acc[mt][nt]);
      }
    }
  };
#pragma unroll
  for (int p = 0; p < kUsPD; ++p) load(p, p);
  int st = 0;
  for (; st + kUsPD <= nst; st += kUsPD) {
#pragma unroll
    for (int p = 0; p < kUsPD; ++p) step(st + p, p);
  }
#pragma unroll
  for (int p = 0; p < kUsPD; ++p)
    if (st + p < nst) step(st + p, p);
  __syncthreads();   // every wave is done with the staged x: the partials overlay it
  // D layout: lane holds u[query 16 mt + 4 g16 + i][rank 16 nt + L16]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTR; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(w * 64 + 16 * mt + 4 * g16 + i) * US + 16 * nt + L16] = acc[mt][nt][i];
  __syncthreads();
  for (int e = tid; e < 64 * RP; e += 512) {
    const int t = e / RP, nn = e - t * RP;
    if (t0 + t < nq) {
      float a = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) a += red[(ww * 64 + t) * US + nn];
      upart[((size_t)b * nq + t0 + t) * RP + nn] = a;
    }
  }
}
static size_t u_stream_lds(int RP) {
  const size_t xs = (size_t)2 * 64 * kUsRow * 2, part = (size_t)8 * 64 * (RP + 4) * 4;
  return xs > part ? xs : part;
}

// 1c. qtilde_small_kernel (bf16, at most 32 queries, as in a decode step): one
//     block per head computes u = x A for all the queries itself, then
//     q~ = q + u B_h. Wave w takes every eighth 64-row slice of A (staged in
//     its own LDS region, next slice prefetched into registers) and the eight
//     partial u are summed through LDS. No split partials in HBM, one launch.
constexpr int kSmallQ = 32;
constexpr int kSmallW = 8;   // waves per block

template <int D, int RP>
__global__ __launch_bounds__(64 * kSmallW) void qtilde_small_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bm,
                                                           int Dh, int r, float* __restrict__ qt, int Hq, int N,
                                                           int q0, int nq) {
  constexpr int AS = RP + 16;                       // staged A slice row stride (elements)
  constexpr int US = RP + 4;                        // u row stride (floats)
  constexpr int BS = D + 16;
  constexpr int kAPer = kUKc * RP / 8 / 64;         // 16-byte pieces of a slice per lane
  static_assert(kUKc * AS * 2 >= kSmallQ * US * 4, "u partials alias the A staging area");
  __shared__ __align__(16) unsigned char stage[kSmallW * kUKc * AS * 2];
  __shared__ __align__(16) bf16_t b_s[RP * BS];
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4, L16 = lane & 15;
  const int h = blockIdx.x, b = blockIdx.y;
  const long long L = (long long)N * kSlots;
  bf16_t* a_s = reinterpret_cast<bf16_t*>(stage) + w * kUKc * AS;
  const bool vec = (r == RP) && (Dh % kUKc == 0);

  // B_h slice [RP][D] into LDS (rows >= r are zero)
  for (int e = tid; e < RP * D / 8; e += 64 * kSmallW) {
    const int kk = (8 * e) / D, n = (8 * e) % D;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (kk < r) v = *reinterpret_cast<const u32x4*>(Bm + (size_t)kk * Hq * D + (size_t)h * D + n);
    *reinterpret_cast<u32x4*>(b_s + kk * BS + n) = v;
  }

  // query rows of this lane's A-operand fragments (two 16-row tiles)
  const bf16_t* xrow[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int t = 16 * mt + L16;
    xrow[mt] = t < nq ? x + ((size_t)b * L + slot_of((long long)q0 + t)) * Dh : nullptr;
  }
  const bf16_t* x0 = x + ((size_t)b * L + slot_of((long long)q0)) * Dh;
  const int nslices = (Dh + kUKc - 1) / kUKc;
  u32x4 apre[kAPer];
  s16x8 xpre[2][kUKc / 32];
  auto fetch = [&](int sl) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int e = 8 * (lane + 64 * j);            // element of the slice, row-major [64][RP]
      const int kk = e / RP, n = e % RP;
      const long long k = (long long)sl * kUKc + kk;
      if (vec) {
        apre[j] = *reinterpret_cast<const u32x4*>(A + (size_t)k * r + n);
      } else {
        s16x8 t;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) t[jj] = (k < Dh && n + jj < r) ? (short)A[(size_t)k * r + n + jj] : (short)0;
        apre[j] = __builtin_bit_cast(u32x4, t);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < kUKc / 32; ++ks) {
        const long long k0 = (long long)sl * kUKc + 32 * ks + 8 * g16;
        if (vec) {
          // rows past nq read row 0's data (always valid) and are zeroed after
          const s16x8 v = load8((xrow[mt] ? xrow[mt] : x0) + k0);
          xpre[mt][ks] = xrow[mt] ? v : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
        } else {
          float xv[8];
          if (xrow[mt]) load_row8<bf16_t>(xrow[mt], k0, Dh, xv);
          else {
#pragma unroll
            for (int j = 0; j < 8; ++j) xv[j] = 0.f;
          }
          xpre[mt][ks] = pack8(xv);
        }
      }
  };
  f32x4 acc[2][RP / 16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < RP / 16; ++nt) acc[mt][nt] = zero4();
  if (w < nslices) fetch(w);
  for (int sl = w; sl < nslices; sl += kSmallW) {
    // this wave's region only: its earlier LDS reads were consumed by MFMAs already
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int e = 8 * (lane + 64 * j);
      *reinterpret_cast<u32x4*>(a_s + (e / RP) * AS + (e % RP)) = apre[j];
    }
    s16x8 xf[2][kUKc / 32];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < kUKc / 32; ++ks) xf[mt][ks] = xpre[mt][ks];
    if (sl + kSmallW < nslices) fetch(sl + kSmallW);
#pragma unroll
    for (int ks = 0; ks < kUKc / 32; ++ks)
#pragma unroll
      for (int nt = 0; nt < RP / 16; ++nt) {
        const s16x8 bf = lds_col_frag(a_s, AS, 32 * ks + 8 * g16, 32 * ks + 8 * g16 + 4, 16 * nt, lane);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma16(xf[mt][ks], bf, acc[mt][nt]);
      }
  }
  __syncthreads();   // every wave is done with its A staging area
  float* u_s = reinterpret_cast<float*>(stage);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < RP / 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) u_s[(w * kSmallQ + 16 * mt + 4 * g16 + i) * US + 16 * nt + L16] = acc[mt][nt][i];
  __syncthreads();
  for (int e = tid; e < kSmallQ * RP; e += 64 * kSmallW) {
    const int row = e / RP, col = e % RP;
    float sum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kSmallW; ++ww) sum += u_s[(ww * kSmallQ + row) * US + col];
    u_s[row * US + col] = sum;   // wave 0's partial is overwritten only by its own sum
  }
  __syncthreads();

  // q~ = q + u B_h: wave w takes row tile w & 1 and a quarter of the D columns
  const int mt = w & 1, nh = w >> 1;
  s16x8 uh[RP / 32], ul[RP / 32];
#pragma unroll
  for (int ks = 0; ks < RP / 32; ++ks) {
    float uv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) uv[j] = u_s[(16 * mt + L16) * US + 32 * ks + 8 * g16 + j];
    pack8_split_hw(uv, uh[ks], ul[ks]);
  }
#pragma unroll
  for (int nn = 0; nn < D / 64; ++nn) {
    const int nt = nh * (D / 64) + nn;
    f32x4 c = zero4();
#pragma unroll
    for (int ks = 0; ks < RP / 32; ++ks) {
      const s16x8 bh = lds_col_frag(b_s, BS, 32 * ks + 8 * g16, 32 * ks + 8 * g16 + 4, 16 * nt, lane);
      c = mfma16(ul[ks], bh, c);
      c = mfma16(uh[ks], bh, c);
    }
    const int dd = 16 * nt + L16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g16 + i;
      if (t < nq) {
        const long long sl = slot_of((long long)q0 + t);
        const float qv = bf2f(q[((size_t)b * Hq + h) * L * D + (size_t)sl * D + dd]);
        qt[(((size_t)b * Hq + h) * nq + t) * D + dd] = qv + c[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------- 2. scores

// Split a float into NS bf16 planes (2: 16 significant bits, 3: 24 bits): each plane
// is the round-to-nearest-even bf16 of what the planes before it leave, converted two
// values per instruction (v_cvt_pk_bf16_f32).
template <int NS>
__device__ __forceinline__ void split_ns(const float* v, s16x8* out) {
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  u32x4 w[NS];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = v[2 * j], b = v[2 * j + 1];
#pragma unroll
    for (int pl = 0; pl < NS; ++pl) {
      const uint32_t pw = pack2_bf16(a, b);
      w[pl][j] = pw;
      if (pl + 1 < NS) {
        a -= __uint_as_float(pw << 16);
        b -= __uint_as_float(pw & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int pl = 0; pl < NS; ++pl) out[pl] = __builtin_bit_cast(s16x8, w[pl]);
}

// NS = 2 for bf16 inputs (hi.hi + hi.lo + lo.hi), 3 for float32 inputs (six plane pairs).
// PIPE: load the next head's operands while the current head is multiplied
// (few blocks, as in a decode step); without it fewer registers, more waves.
template <int D, int NS, bool PIPE>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qt, const float* __restrict__ s,
                                                    const float* __restrict__ H, float beta, float scale,
                                                    float* __restrict__ z, float* __restrict__ zhat,
                                                    int Hq, int Hkv, int N, int nq) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g16 = lane >> 4, L16 = lane & 15;
  const int c0 = blockIdx.x * 64 + 16 * w, t0 = blockIdx.y * 16;
  const int bg = blockIdx.z, b = bg / Hkv, g = bg - b * Hkv;
  const int G = Hq / Hkv;
  const int ca = c0 + L16;   // A-operand row (chunk) of this lane
  const int tb = t0 + L16;   // B-operand column (query) of this lane
  float zmax[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  // operands of head hh + 1 are loaded while head hh is multiplied
  f32x4 sa[D / 32][2], qb[D / 32][2];
  float hv[4];
  auto fetch = [&](int hh) {
    const int h = g * G + hh;
    const float* srow = s + (((size_t)b * Hq + h) * N + (ca < N ? ca : 0)) * D;
    const float* qrow = qt + (((size_t)b * Hq + h) * nq + (tb < nq ? tb : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int kk = 32 * ks + 8 * g16;
      sa[ks][0] = *reinterpret_cast<const f32x4*>(srow + kk);
      sa[ks][1] = *reinterpret_cast<const f32x4*>(srow + kk + 4);
      qb[ks][0] = *reinterpret_cast<const f32x4*>(qrow + kk);
      qb[ks][1] = *reinterpret_cast<const f32x4*>(qrow + kk + 4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 4 * g16 + i;
      hv[i] = H[((size_t)b * Hq + h) * N + (c < N ? c : N - 1)];
    }
  };
  if (PIPE) fetch(0);
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    if (!PIPE) fetch(hh);
    s16x8 a[D / 32][NS], bb[D / 32][NS];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      float av[8], bv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        av[j] = ca < N ? sa[ks][0][j] : 0.f;
        av[4 + j] = ca < N ? sa[ks][1][j] : 0.f;
        bv[j] = tb < nq ? qb[ks][0][j] : 0.f;
        bv[4 + j] = tb < nq ? qb[ks][1][j] : 0.f;
      }
      split_ns<NS>(av, a[ks]);
      split_ns<NS>(bv, bb[ks]);
    }
    float hcur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hcur[i] = hv[i];
    if (PIPE && hh + 1 < G) fetch(hh + 1);
    f32x4 acc_hi = zero4(), acc_x = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      if constexpr (NS == 3) {
        acc_x = mfma16(a[ks][0], bb[ks][2], acc_x);
        acc_x = mfma16(a[ks][2], bb[ks][0], acc_x);
        acc_x = mfma16(a[ks][1], bb[ks][1], acc_x);
      }
      acc_x = mfma16(a[ks][0], bb[ks][1], acc_x);
      acc_x = mfma16(a[ks][1], bb[ks][0], acc_x);
      acc_hi = mfma16(a[ks][0], bb[ks][0], acc_hi);
    }
    // D layout: lane holds chunk c0 + 4*g16 + i (rows), query t0 + L16 (column)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 4 * g16 + i;
      const int t = t0 + L16;
      if (c < N && t < nq) {
        const float zz = (acc_hi[i] + acc_x[i]) * scale - beta * hcur[i];
        z[(((size_t)b * Hq + h) * nq + t) * N + c] = zz;
        zmax[i] = fmaxf(zmax[i], zz);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = c0 + 4 * g16 + i;
    const int t = t0 + L16;
    if (c < N && t < nq) zhat[((size_t)bg * nq + t) * N + c] = zmax[i];
  }
}

// ---------------------------------------------------------------------------- 3. top-K

template <int P>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ zhat, const float* __restrict__ z,
                                                   int32_t* __restrict__ idx, float* __restrict__ zsel,
                                                   int Hq, int Hkv, int N, int nq, int q0, int K, int R,
                                                   long long nrows) {
  __shared__ int chosen[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + w;
  const bool live = row < nrows;
  const long long rr = live ? row : 0;
  const int t = (int)(rr % nq);
  const long long bg = rr / nq;
  const int b = (int)(bg / Hkv), g = (int)(bg % Hkv);
  const int G = Hq / Hkv;
  const long long i = (long long)q0 + t;
  const float* zr = zhat + rr * N;
  const unsigned long long lt = (1ull << lane) - 1ull;

  // All P loads are issued before any is used: the empty asm "redefines" each
  // value, which keeps the compiler from sinking a load into the branch that
  // tests its candidate (that would serialise P memory round trips).
  float zv[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int c = 64 * j + lane;
    zv[j] = zr[c < N ? c : N - 1];   // always in bounds
  }
#pragma unroll
  for (int j = 0; j < P; ++j) asm volatile("" : "+v"(zv[j]));
  uint32_t key[P];
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int c = 64 * j + lane;
    const bool cand = (c < N) & ((63LL * c + 62 < i - R) | (63LL * c > i + R));
    key[j] = cand ? order_key(zv[j]) : 0u;
    ncand += __popcll(__ballot(key[j] != 0u));
  }
  // counts are taken with ballots (scalar popcounts), no cross-lane shuffles
  const bool take_all = ncand <= K;
  uint32_t theta = 0u;
  int need = 0;
  if (!take_all) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t trial = theta | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < P; ++j) cnt += __popcll(__ballot(key[j] >= trial));
      if (cnt >= K) theta = trial;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) gt += __popcll(__ballot(key[j] > theta));
    need = K - gt;
  }
  int base = 0, ties = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const bool nz = key[j] != 0u;
    const bool gt = take_all ? nz : key[j] > theta;
    const bool eq = !take_all && nz && key[j] == theta;
    const unsigned long long em = __ballot(eq);
    const bool take = gt || (eq && ties + __popcll(em & lt) < need);
    const unsigned long long tm = __ballot(take);
    if (take) chosen[w][base + __popcll(tm & lt)] = 64 * j + lane;
    base += __popcll(tm);
    ties += __popcll(em);
  }
  __syncthreads();
  if (live && lane < K) {
    const int c = lane < base ? chosen[w][lane] : -1;
    idx[rr * K + lane] = c;
    for (int hh = 0; hh < G; ++hh) {
      const size_t hrow = ((size_t)b * Hq + g * G + hh) * nq + t;
      zsel[hrow * K + lane] = c >= 0 ? z[hrow * N + c] : -INFINITY;
    }
  }
}

// Top K of a wave's keys: lane l holds key[j] for element 64 j + l (elements in
// their order); keys are order_key values, 0 = not a candidate. The K largest
// keys are chosen, ties going to the smaller element. Two parts:
//  - wave_topk_thresholds: theta = the largest key with at least K keys >= theta,
//    found one bit per step; once exactly K keys reach the threshold, the chosen
//    set (ties included) is fixed and the search stops. It runs Q selections at
//    once, interleaved, so that their ballot -> count chains overlap;
//  - wave_topk_select: emit(slot, j) is called by the owning lane for every chosen
//    element, slots 0 .. count - 1 in element order; returns count = min(K, number
//    of candidates) (wave-uniform).
template <int P, int Q>
__device__ __forceinline__ void wave_topk_thresholds(const uint32_t (*key)[P], int K, uint32_t* theta, bool* take_all) {
  unsigned done = 0u;   // selections whose threshold is final (wave-uniform)
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    int ncand = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) ncand += __popcll(__ballot(key[q][j] != 0u));
    take_all[q] = ncand <= K;
    theta[q] = 0u;
    if (take_all[q]) done |= 1u << q;
  }
  for (int bit = 31; bit >= 0 && done != (1u << Q) - 1u; --bit) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      if ((done >> q) & 1u) continue;
      const uint32_t trial = theta[q] | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < P; ++j) cnt += __popcll(__ballot(key[q][j] >= trial));
      if (cnt >= K) theta[q] = trial;
      if (cnt == K) done |= 1u << q;
    }
  }
}

template <int P, typename Emit>
__device__ __forceinline__ int wave_topk_select(const uint32_t* key, int K, uint32_t theta, bool take_all, int lane,
                                                Emit emit) {
  const unsigned long long lt = (1ull << lane) - 1ull;
  int need = 0;
  if (!take_all) {
    int gt = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) gt += __popcll(__ballot(key[j] > theta));
    need = K - gt;
  }
  int base = 0, ties = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const bool nz = key[j] != 0u;
    const bool gt = take_all ? nz : key[j] > theta;
    const bool eq = !take_all && nz && key[j] == theta;
    const unsigned long long em = __ballot(eq);
    const bool take = gt || (eq && ties + __popcll(em & lt) < need);
    const unsigned long long tm = __ballot(take);
    if (take) emit(base + __popcll(tm & lt), j);
    base += __popcll(tm);
    ties += __popcll(em);
  }
  return base;
}

template <int P, typename Emit>
__device__ __forceinline__ int wave_topk(const uint32_t* key, int K, int lane, Emit emit) {
  uint32_t theta;
  bool take_all;
  wave_topk_thresholds<P, 1>(reinterpret_cast<const uint32_t(*)[P]>(key), K, &theta, &take_all);
  return wave_topk_select<P>(key, K, theta, take_all, lane, emit);
}

// The same selection, narrowed first: the K-th largest of the 64 lane maxima is at
// most the K-th largest key, so the keys at or above it hold the whole top K (ties
// at the threshold included). Up to kNarrow of them are compacted in element order
// into two keys per lane through buf (this wave's 2 kNarrow words of LDS) and the
// selection runs on those; with more, on all keys. emit(slot, e, key) is called
// for every chosen element e = 64 j + l, slots in element order.
constexpr int kNarrow = 128;

template <int P, typename Emit>
__device__ __forceinline__ int wave_topk_narrow(const uint32_t* key, int K, int lane, uint32_t* buf, Emit emit) {
  uint32_t lm[1][1] = {{key[0]}};
#pragma unroll
  for (int j = 1; j < P; ++j) lm[0][0] = max(lm[0][0], key[j]);
  uint32_t thl;
  bool tal;
  wave_topk_thresholds<1, 1>(lm, K, &thl, &tal);
  const uint32_t lq = tal ? 1u : max(thl, 1u);
  const unsigned long long lt = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const bool in = key[j] >= lq;
    const unsigned long long m = __ballot(in);
    const int pos = base + __popcll(m & lt);
    if (in && pos < kNarrow) {
      buf[pos] = key[j];
      buf[kNarrow + pos] = 64 * j + lane;
    }
    base += __popcll(m);
  }
  if (base > kNarrow) return wave_topk<P>(key, K, lane, [&](int slot, int j) { emit(slot, 64 * j + lane, key[j]); });
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  uint32_t ck[2];
  int ci[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int pos = 64 * jj + lane;
    ck[jj] = pos < base ? buf[pos] : 0u;
    ci[jj] = (int)buf[kNarrow + pos];
  }
  return wave_topk<2>(ck, K, lane, [&](int slot, int jj) { emit(slot, ci[jj], ck[jj]); });
}

// ---------------------------------------------------------------------------- 4. fused scoring (bf16)
//
// route_score3_kernel: for QT = 16 NT consecutive queries of one KV group,
// everything between the residual partials and the selection in one block of 8
// waves, without writing per-head scores or q~ to memory. Wave w < G owns head w:
//  0. it forms q~ = q + u B_h of its head for the block's queries on MFMA (u split
//     into bf16 hi + lo, B exact; B comes transposed per call so its fragments are
//     plain loads) and keeps it in registers as the hi/lo B operand of the scoring
//     product (the q~^T output fragment already has that lane -> k assignment);
//  A. it computes z^T = s q~^T for every chunk row tile of its head with both
//     operands split into hi + lo (hi.hi + hi.lo + lo.hi), scaled, minus beta * H
//     (summaries as fragment-major split planes, 1 KB contiguous per load, the
//     next tile in flight while the current one is multiplied), and folds the
//     scores into the group maximum with LDS atomic max on order-preserving keys;
//  B. exact top-K per query from those keys (all waves; bisection with ballot
//     counts, ties to the smaller chunk), written as idx, with a [QT][N] rank table;
//  C. the same products again (bit-identical); the scores of chosen (query,
//     chunk) pairs go straight to zsel, each tile's ranks read with its planes.
// The keys are dead once every wave holds its queries' keys in registers, so the
// rank table and the zsel staging rows of phases B and C overlay them: the block's
// LDS is the key table plus the chosen lists, which admits 32 queries per block at
// N = 1024 within the 160 KB of a CU.
constexpr int kRsWaves = 8;
constexpr int kMaxGroup = 8;   // query heads per KV group of the fused scoring kernels

// Row strides chosen for the LDS banks (64 banks of 4 bytes): key rows of rs3_zs(N)
// words, 3 modulo 64, so that the group-maximum atomics of a wave (16 query rows x 16
// chunks per tile) meet at most two to a bank; rank rows of rs3_rn(N) bytes (all of a
// row's 16-chunk tiles, a multiple of 16 bytes, 4 words modulo 64), so that a wave's
// 4-byte rank reads of 16 rows x 4 chunk groups hit 64 distinct banks.
__host__ __device__ inline int rs3_zs(int N) { return N + (((3 - N % 64) % 64) + 64) % 64; }
__host__ __device__ inline int rs3_rn(int N) {
  int r4 = (N + 15) / 16 * 4;
  r4 += (((4 - r4 % 64) % 64) + 64) % 64;
  return 4 * r4;
}
__host__ __device__ inline size_t rs3_keys(int NT, int N) { return (size_t)16 * NT * rs3_zs(N) * 4; }
__host__ __device__ inline size_t rs3_off_z(int NT, int N) { return ((size_t)16 * NT * rs3_rn(N) + 15) & ~(size_t)15; }
__host__ __device__ inline size_t rs3_stage(int NT, int K) { return (size_t)kRsWaves * 16 * NT * K * 4; }
// offset of the chosen lists: past the keys, or past ranks + staging rows if longer
__host__ __device__ inline size_t rs3_off_c(int NT, int N, int K, bool stage) {
  const size_t over = rs3_off_z(NT, N) + (stage ? rs3_stage(NT, K) : 0);
  return ((rs3_keys(NT, N) > over ? rs3_keys(NT, N) : over) + 15) & ~(size_t)15;
}
__host__ __device__ inline size_t rs3_lds(int NT, int N, int K, bool stage) {
  return rs3_off_c(NT, N, K, stage) + kRsWaves * 64 * 4;
}

// Summaries as the A operand of the scoring product, fragment-major: for each
// (batch, head, 16-chunk row tile, k-step, plane) the 64 lanes' 16-byte fragments
// are contiguous. Lane l holds chunk 16 mt + l % 16 and d = 32 ks + 4 (l / 16) +
// {0..3}, 32 ks + 16 + 4 (l / 16) + {0..3}; plane 0 is bf16 hi, plane 1 lo. Rows
// past N are zero.
template <int D>
__global__ __launch_bounds__(256) void split_frag_kernel(const float* __restrict__ s, bf16_t* __restrict__ sp, int N,
                                                         long long heads) {
  constexpr int KS = D / 32, GPR = D / 8;
  const int NMT = (N + 15) / 16;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;   // one (head, row, group of 8) per thread
  if (e >= heads * NMT * 16 * GPR) return;
  const int gi = (int)(e % GPR);
  const long long rowg = e / GPR;
  const long long hd = rowg / (NMT * 16);
  const int row = (int)(rowg - hd * NMT * 16);
  const int mt = row >> 4, L16 = row & 15, ks = gi >> 2, gg = gi & 3;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  if (row < N) {
    const float* src = s + (hd * N + row) * D + 32 * ks + 4 * gg;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a0[i];
      v[4 + i] = a1[i];
    }
  }
  s16x8 hi, lo;
  pack8_split_hw(v, hi, lo);
  bf16_t* dst = sp + ((((hd * NMT + mt) * KS + ks) * 2) * 64 + gg * 16 + L16) * 8;
  *reinterpret_cast<s16x8*>(dst) = hi;
  *reinterpret_cast<s16x8*>(dst + 64 * 8) = lo;
}

// q~ = q + u B_h of head h for the 16 NT queries t0 .. t0 + 16 NT - 1 (u summed from
// its nsplit partials; rows past nq are zero), split into bf16 hi + lo as the B
// operand of the scoring product: lane l holds query 16 nt + l % 16 and
// d = 32 ks + 8 (l / 16) + {0..7}, the layout of the q~^T output fragment. The product
// u B_h runs on MFMA with u split into hi + lo and B exact (B comes transposed, so its
// fragments are plain loads).
template <int D, int RP, int NT>
__device__ __forceinline__ void rs_qtilde(const bf16_t* __restrict__ q, const bf16_t* __restrict__ Bt,
                                          const float* __restrict__ upart, int nsplit, int B, int b, int h, int Hq,
                                          long long L, int q0, int t0, int nq, int lane, s16x8 (&qh)[NT][D / 32],
                                          s16x8 (&ql)[NT][D / 32]) {
  constexpr int KS = D / 32, RK = RP / 32;
  const int g16 = lane >> 4, L16 = lane & 15;
  s16x8 bt[KS][2][RK];   // B_h^T: d rows 16 (2 ks + half) + L16, ranks 32 rk + 8 g16 + {0..7}
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int rk = 0; rk < RK; ++rk)
        bt[ks][half][rk] = load8(Bt + ((size_t)h * D + 16 * (2 * ks + half) + L16) * RP + 32 * rk + 8 * g16);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int tq = t0 + 16 * nt + L16;
    const int tc = tq < nq ? tq : nq - 1;
    const bf16_t* qrow = q + ((size_t)b * Hq + h) * L * D + (size_t)slot_of((long long)q0 + tc) * D;
    s16x4 q4[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        q4[ks][half] = *reinterpret_cast<const s16x4*>(qrow + 16 * (2 * ks + half) + 4 * g16);
    s16x8 uh[RK], ul[RK];
#pragma unroll
    for (int rk = 0; rk < RK; ++rk) {
      float uv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) uv[j] = 0.f;
      for (int sp2 = 0; sp2 < nsplit; ++sp2) {
        const float* up = upart + (((size_t)sp2 * B + b) * nq + tc) * RP + 32 * rk + 8 * g16;
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(up);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(up + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uv[j] += a0[j];
          uv[4 + j] += a1[j];
        }
      }
      if (tq >= nq) {
#pragma unroll
        for (int j = 0; j < 8; ++j) uv[j] = 0.f;
      }
      pack8_split_hw(uv, uh[rk], ul[rk]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float qv[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x4 acc = zero4();
#pragma unroll
        for (int rk = 0; rk < RK; ++rk) {
          acc = mfma16(bt[ks][half][rk], ul[rk], acc);
          acc = mfma16(bt[ks][half][rk], uh[rk], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[4 * half + i] = acc[i] + bf2f((bf16_t)q4[ks][half][i]);
      }
      pack8_split_hw(qv, qh[nt][ks], ql[nt][ks]);
    }
  }
}

template <int D, int RP, int NT, int P, bool STAGE>
__global__ __launch_bounds__(64 * kRsWaves) void route_score3_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Bt, const float* __restrict__ upart, int nsplit,
    const bf16_t* __restrict__ sp, const float* __restrict__ H, float beta, float scale, int32_t* __restrict__ idx,
    float* __restrict__ zsel, int B, int Hq, int Hkv, int N, int q0, int nq, int K, int R, int rev) {
  constexpr int QT = 16 * NT, KS = D / 32, RK = RP / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, L16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (nq + QT - 1) / QT;
  const int tile = xcd_tile(nqb * B * Hkv, rev);   // (batch-group, query block), batch-group major
  if (tile < 0) return;
  const int bg = tile / nqb, b = bg / Hkv, g = bg - b * Hkv;
  const int G = Hq / Hkv;
  const int t0 = (tile - bg * nqb) * QT;
  const long long L = (long long)N * kSlots;
  const int NMT = (N + 15) / 16, ZS = rs3_zs(N), RN = rs3_rn(N);
  uint32_t* zk = reinterpret_cast<uint32_t*>(smem);             // A, B: [QT][ZS] group-maximum keys
  uint8_t* rank_t = smem;                                       // B, C: [QT][RN] rank in zsel, 0xFF if not chosen
  float* zst = reinterpret_cast<float*>(smem + rs3_off_z(NT, N));   // C (STAGE): per wave [QT][K] zsel rows
  int* chosen = reinterpret_cast<int*>(smem + rs3_off_c(NT, N, K, STAGE));
  for (int e = tid; e < QT * ZS; e += 64 * kRsWaves) zk[e] = 0u;

  const bool hw = w < G;   // this wave owns head w (wave-uniform)
  const int h = g * G + (hw ? w : 0);

  // ---- 0. q~ of head h as the scoring B operand, in registers
  s16x8 qh[NT][KS], ql[NT][KS];
  if (hw) rs_qtilde<D, RP, NT>(q, Bt, upart, nsplit, B, b, h, Hq, L, q0, t0, nq, lane, qh, ql);
  __syncthreads();   // keys initialised

  struct TileBuf {
    s16x8 sf[KS][2];
    float hv[4];
    uint32_t rk[NT];
  };
  const bf16_t* sph = sp + (size_t)(b * Hq + h) * NMT * KS * 2 * 64 * 8;
  auto load_tile = [&](int mt, TileBuf& t, bool ranks) {
    const bf16_t* base = sph + (size_t)mt * KS * 2 * 64 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) t.sf[ks][pl] = load8(base + ((ks * 2 + pl) * 64 + lane) * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * mt + 4 * g16 + i;
      t.hv[i] = H[((size_t)b * Hq + h) * N + (c < N ? c : N - 1)];
    }
    if (ranks) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // chunks past N read the row's 0xFF fill
        t.rk[nt] = *reinterpret_cast<const uint32_t*>(rank_t + (16 * nt + L16) * RN + 16 * mt + 4 * g16);
      }
    }
  };
  auto tile_scores = [&](const TileBuf& t, f32x4 (&zz)[NT]) {
    f32x4 ahi[NT], ax[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ahi[nt] = zero4();
      ax[nt] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ax[nt] = mfma16(t.sf[ks][0], ql[nt][ks], ax[nt]);
        ax[nt] = mfma16(t.sf[ks][1], qh[nt][ks], ax[nt]);
        ahi[nt] = mfma16(t.sf[ks][0], qh[nt][ks], ahi[nt]);
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) zz[nt][i] = (ahi[nt][i] + ax[nt][i]) * scale - beta * t.hv[i];
  };
  // every chunk row tile of the head, the loads of the next tile (the next two where
  // two query tiles leave the registers for a third buffer) in flight; wave w starts
  // at tile w so that the waves' atomic updates of the group maximum rarely meet
  auto sweep = [&](bool ranks, auto&& emit) {
    f32x4 zz[NT];
    auto tile_at = [&](int it) { return (w + it) % NMT; };
    if constexpr (NT <= 2) {
      TileBuf ta, tb, tc;
      load_tile(tile_at(0), ta, ranks);
      if (1 < NMT) load_tile(tile_at(1), tb, ranks);
      for (int it = 0; it < NMT; it += 3) {
        if (it + 2 < NMT) load_tile(tile_at(it + 2), tc, ranks);
        tile_scores(ta, zz);
        emit(tile_at(it), ta, zz);
        if (it + 1 < NMT) {
          if (it + 3 < NMT) load_tile(tile_at(it + 3), ta, ranks);
          tile_scores(tb, zz);
          emit(tile_at(it + 1), tb, zz);
        }
        if (it + 2 < NMT) {
          if (it + 4 < NMT) load_tile(tile_at(it + 4), tb, ranks);
          tile_scores(tc, zz);
          emit(tile_at(it + 2), tc, zz);
        }
      }
    } else {
      TileBuf ta, tb;
      load_tile(tile_at(0), ta, ranks);
      for (int it = 0; it < NMT; it += 2) {
        if (it + 1 < NMT) load_tile(tile_at(it + 1), tb, ranks);
        tile_scores(ta, zz);
        emit(tile_at(it), ta, zz);
        if (it + 1 < NMT) {
          if (it + 2 < NMT) load_tile(tile_at(it + 2), ta, ranks);
          tile_scores(tb, zz);
          emit(tile_at(it + 1), tb, zz);
        }
      }
    }
  };

  // ---- A: group maximum through LDS atomic max on order-preserving keys
  if (hw)
    sweep(false, [&](int mt, const TileBuf&, const f32x4 (&zz)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * mt + 4 * g16 + i;
          if (c < N) atomicMax(&zk[(16 * nt + L16) * ZS + c], order_key(zz[nt][i]));
        }
    });
  __syncthreads();

  // ---- B: top-K per query (wave w: queries w, w + 8, ..., their thresholds found
  //      together) and the rank table
  {
    constexpr int QW = QT / kRsWaves;
    static_assert(QT % kRsWaves == 0, "queries per wave");
    uint32_t key[QW][P];
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
      const int qi = w + kRsWaves * qq, t = t0 + qi;
      const long long i = (long long)q0 + t;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int c = 64 * j + lane;
        const bool cand = (t < nq) & (c < N) & ((63LL * c + 62 < i - R) | (63LL * c > i + R));
        const uint32_t kv = zk[qi * ZS + (c < N ? c : N - 1)];
        key[qq][j] = cand ? kv : 0u;
      }
    }
    __syncthreads();   // every wave holds its keys: the table becomes ranks and staging rows
    for (int e = tid; e < QT * RN / 4; e += 64 * kRsWaves) reinterpret_cast<uint32_t*>(rank_t)[e] = 0xFFFFFFFFu;
    if constexpr (STAGE)
      for (int e = tid; e < kRsWaves * QT * K; e += 64 * kRsWaves) zst[e] = -INFINITY;   // unfilled slots
    __syncthreads();
    uint32_t theta[QW];
    bool take_all[QW];
    wave_topk_thresholds<P, QW>(key, K, theta, take_all);
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
      const int qi = w + kRsWaves * qq, t = t0 + qi;
      if (t >= nq) break;
      const int cnt = wave_topk_select<P>(key[qq], K, theta[qq], take_all[qq], lane,
                                          [&](int slot, int j) { chosen[w * 64 + slot] = 64 * j + lane; });
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane < K) {
        const int c = lane < cnt ? chosen[w * 64 + lane] : -1;
        idx[((size_t)bg * nq + t) * K + lane] = c;
        if (c >= 0) rank_t[qi * RN + c] = (uint8_t)lane;
        else if constexpr (!STAGE)
          for (int hh = 0; hh < G; ++hh) zsel[(((size_t)b * Hq + g * G + hh) * nq + t) * K + lane] = -INFINITY;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  // ---- C: the chosen scores of head h to zsel: through the wave's LDS rows and out
  //      as whole contiguous rows (STAGE), or straight to zsel
  if (hw) {
    float* zrow = zsel + (((size_t)b * Hq + h) * nq + t0) * K;
    float* zw = zst + (size_t)w * QT * K;
    sweep(true, [&](int, const TileBuf& tbuf, const f32x4 (&zz)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t r8 = (tbuf.rk[nt] >> (8 * i)) & 0xFFu;
          if (r8 != 0xFFu) {
            if constexpr (STAGE) zw[(16 * nt + L16) * K + r8] = zz[nt][i];
            else zrow[(size_t)(16 * nt + L16) * K + r8] = zz[nt][i];
          }
        }
    });
    if constexpr (STAGE) {
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's rows are in LDS
      __builtin_amdgcn_wave_barrier();
      const int len = min(QT, nq - t0) * K;   // the block's rows of head h are contiguous in zsel
      if ((K & 3) == 0) {
        for (int e = 4 * lane; e < len; e += 256)
          *reinterpret_cast<f32x4*>(zrow + e) = *reinterpret_cast<const f32x4*>(zw + e);
      } else {
        for (int e = lane; e < len; e += 64) zrow[e] = zw[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------- 4b. one-sweep scoring
//
// route_score_stream_kernel: the block, the q~ registers and the split products of
// route_score3_kernel, with the selection taken during the one sweep over the
// summaries, so that no product is formed twice. The chunk row tiles are walked in
// batches of TB tiles (CB = 16 TB chunks):
//  A. wave w < G forms the scores of head w for the batch's chunks (each wave starts
//     at another tile of the batch) and stores them as order-preserving keys in the
//     batch table, one row per (head, query);
//  B. after a block barrier, every wave takes QT / 8 of the queries: one lane per
//     chunk of the batch forms the group maximum over the heads' keys, drops chunks
//     that are not candidates (past N or in the query's window range) and keeps the
//     ones whose key is strictly above the key of the query's K-th place (the chunks
//     arrive in ascending order, so a tie belongs to the earlier chunk). These are
//     merged into the query's list (in LDS, best first: key descending, chunk
//     ascending among equal keys) by ranks: an entering chunk goes behind every
//     entry with a key at least as large and every entering chunk ahead of it in
//     that order; an entry moves back by the entering chunks with larger keys; the
//     places past K leave. Each entry owns a row of per-head keys: the rows of the
//     leaving entries pass to the entering chunks and are filled from the batch
//     table. A second barrier frees the table for the next batch.
// After the last batch the list of a query is its top K: written as idx in ascending
// chunk order, with the per-head scores (keys mapped back to floats bit for bit) as
// zsel; unfilled places are -1 and -inf. The selection is the same as the one of
// route_score3_kernel (the order of chunks with equal keys decides ties in both); the
// LDS does not grow with N: the batch table is G x QT x (CB + 4) words, the lists
// QT x K x (3 + G) words and 64 words per wave hand rows over.
__host__ __device__ inline size_t ss_lds(int NT, int G, int TB, int K) {
  const size_t QT = (size_t)16 * NT;
  return (size_t)G * QT * (16 * TB + 4) * 4 + QT * K * (3 + (size_t)G) * 4 + (size_t)kRsWaves * 64 * 4 + QT * 4;
}

// The order-preserving key of a float back to the float (the inverse of order_key on
// every value that order_key does not clamp).
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Minimum of a wave's values, in every lane: rotations within each 16-lane row
// (DPP row_ror 8, 4, 2, 1), then the row pairs l ^ 16 and l ^ 32 (permlane swaps).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min((uint32_t)r[0], (uint32_t)r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min((uint32_t)r[0], (uint32_t)r[1]);
}

// Selections with at most this many elements past the K best drop them one at a time;
// more take the bisection of wave_topk_thresholds.
constexpr int kDropRounds = 8;

template <int D, int RP, int NT, int TB>
__global__ __launch_bounds__(64 * kRsWaves) void route_score_stream_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Bt, const float* __restrict__ upart, int nsplit,
    const bf16_t* __restrict__ sp, const float* __restrict__ H, float beta, float scale, int32_t* __restrict__ idx,
    float* __restrict__ zsel, int B, int Hq, int Hkv, int N, int q0, int nq, int K, int R, int rev) {
  constexpr int QT = 16 * NT, KS = D / 32, CB = 16 * TB, CBS = CB + 4;
  constexpr int NBUF = NT <= 2 ? 3 : 2;   // tile buffers in the ring (registers allow three for two query tiles)
  constexpr int QW = QT / kRsWaves;       // queries per wave in the selection
  static_assert(TB % NBUF == 0, "a batch is a whole number of rounds of the tile ring");
  static_assert(CB <= 64 && QT % kRsWaves == 0, "one lane per chunk of a batch");
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, L16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (nq + QT - 1) / QT;
  const int tile = xcd_tile(nqb * B * Hkv, rev);   // (batch-group, query block), batch-group major
  if (tile < 0) return;
  const int bg = tile / nqb, b = bg / Hkv, g = bg - b * Hkv;
  const int G = Hq / Hkv;
  const int t0 = (tile - bg * nqb) * QT;
  const long long L = (long long)N * kSlots;
  const int NMT = (N + 15) / 16;
  const int nbatch = (NMT + TB - 1) / TB;
  uint32_t* st = reinterpret_cast<uint32_t*>(smem);          // [G][QT][CBS] keys of the batch per head
  uint32_t* lk = st + (size_t)G * QT * CBS;                  // [QT][K] list keys, best first (0: empty)
  int* lc = reinterpret_cast<int*>(lk + QT * K);             // [QT][K] their chunks (-1: empty)
  int* ls = lc + QT * K;                                     // [QT][K] their rows of lh
  uint32_t* lh = reinterpret_cast<uint32_t*>(ls + QT * K);   // [QT][K][G] per-head keys of a row's entry
  for (int e = tid; e < QT * K; e += 64 * kRsWaves) {
    lk[e] = 0u;
    lc[e] = -1;
    ls[e] = e % K;
  }
  for (int e = tid; e < QT; e += 64 * kRsWaves) ls[QT * K + QT * K * G + kRsWaves * 64 + e] = 0;   // lth

  const bool hw = w < G;   // this wave owns head w (wave-uniform)
  const int h = g * G + (hw ? w : 0);
  s16x8 qh[NT][KS], ql[NT][KS];
  if (hw) rs_qtilde<D, RP, NT>(q, Bt, upart, nsplit, B, b, h, Hq, L, q0, t0, nq, lane, qh, ql);
  __syncthreads();   // lists initialised

  struct TileBuf {
    s16x8 sf[KS][2];
    float hv[4];
  };
  const bf16_t* sph = sp + (size_t)(b * Hq + h) * NMT * KS * 2 * 64 * 8;
  // tile of step it: batch it / TB, rotated by w within the batch
  auto tile_at = [&](int it) {
    const int b0 = it - it % TB, bs = min(TB, NMT - b0);
    return b0 + (it - b0 + w) % bs;
  };
  auto load_tile = [&](int it, TileBuf& t) {
    const int mt = tile_at(it);
    const bf16_t* base = sph + (size_t)mt * KS * 2 * 64 * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) t.sf[ks][pl] = load8(base + ((ks * 2 + pl) * 64 + lane) * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * mt + 4 * g16 + i;
      t.hv[i] = H[((size_t)b * Hq + h) * N + (c < N ? c : N - 1)];
    }
  };
  // scores of the step's tile, as keys into the batch table (row (w, query), column
  // chunk - first chunk of the batch)
  auto score_tile = [&](int it, const TileBuf& t) {
    f32x4 ahi[NT], ax[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ahi[nt] = zero4();
      ax[nt] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ax[nt] = mfma16(t.sf[ks][0], ql[nt][ks], ax[nt]);
        ax[nt] = mfma16(t.sf[ks][1], qh[nt][ks], ax[nt]);
        ahi[nt] = mfma16(t.sf[ks][0], qh[nt][ks], ahi[nt]);
      }
    const int col = 16 * (tile_at(it) - (it - it % TB)) + 4 * g16;
    typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      u32x4 kv;
#pragma unroll
      for (int i = 0; i < 4; ++i) kv[i] = order_key((ahi[nt][i] + ax[nt][i]) * scale - beta * t.hv[i]);
      *reinterpret_cast<u32x4*>(st + ((size_t)w * QT + 16 * nt + L16) * CBS + col) = kv;
    }
  };
  // B: the batch's candidates into the lists of this wave's queries. A list holds its
  // entries in ascending chunk order in places 0 .. K - 1 (key 0: an empty place), with
  // lth the K-th largest key of a full list (0 otherwise). Lane p holds place p of the
  // list, lane l chunk c0 + l of the batch: the top K of the two, in element order, is
  // the new list.
  int* wscr = ls + QT * K + QT * K * G + w * 64;   // this wave's row hand-over slots
  uint32_t* lth = reinterpret_cast<uint32_t*>(wscr + (kRsWaves - w) * 64);   // [QT]
  auto select_batch = [&](int bi) {
    const int c0 = CB * bi;
    const int c = c0 + lane;
    const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll 1
    for (int qq = 0; qq < QW; ++qq) {
      const int qi = w + kRsWaves * qq, t = t0 + qi;
      if (t >= nq) break;   // wave-uniform
      const long long i = (long long)q0 + t;
      uint32_t hk[kMaxGroup];   // every head's key at once (rows past G repeat the last head)
#pragma unroll
      for (int hh = 0; hh < kMaxGroup; ++hh)
        hk[hh] = st[((size_t)min(hh, G - 1) * QT + qi) * CBS + (lane < CB ? lane : 0)];
      uint32_t kb = hk[0];
#pragma unroll
      for (int hh = 1; hh < kMaxGroup; ++hh) kb = max(kb, hk[hh]);
      const bool cand = lane < CB && c < N && ((63LL * c + 62 < i - R) | (63LL * c > i + R));
      // only a key above the K-th of the list can enter (a tie belongs to the earlier chunk)
      uint32_t key[2];
      key[1] = cand && kb > lth[qi] ? kb : 0u;
      if (__ballot(key[1] != 0u) == 0ull) continue;
      key[0] = lane < K ? lk[qi * K + lane] : 0u;
      const int pc = lane < K ? lc[qi * K + lane] : -1;
      const int ps = lane < K ? ls[qi * K + lane] : 0;
      uint32_t theta;
      bool take_all;
      int slot0 = -1, slot1 = -1;   // new places of this lane's list entry and batch chunk
      int cnt;
      const int n0 = __popcll(__ballot(key[0] != 0u));
      const int drop = n0 + __popcll(__ballot(key[1] != 0u)) - K;   // elements past the K best
      if (drop > kDropRounds) {
        wave_topk_thresholds<2, 1>(reinterpret_cast<const uint32_t(*)[2]>(key), K, &theta, &take_all);
        cnt = wave_topk_select<2>(key, K, theta, take_all, lane, [&](int slot, int j) {
          if (j == 0) slot0 = slot;
          else slot1 = slot;
        });
      } else {
        // few past the K best: drop the smallest key drop times, among equal keys the
        // last element (batch after list, higher lanes later), then keep the rest in order
        for (int r = 0; r < drop; ++r) {
          const uint32_t mn =
              wave_min_u32(min(key[0] != 0u ? key[0] : ~0u, key[1] != 0u ? key[1] : ~0u));
          const unsigned long long b1 = __ballot(key[1] == mn);
          if (b1 != 0ull) {
            if (lane == 63 - __builtin_clzll(b1)) key[1] = 0u;
          } else {
            const unsigned long long b0 = __ballot(key[0] == mn);
            if (lane == 63 - __builtin_clzll(b0)) key[0] = 0u;
          }
        }
        const unsigned long long m0 = __ballot(key[0] != 0u), m1 = __ballot(key[1] != 0u);
        if (key[0] != 0u) slot0 = __popcll(m0 & lt);
        if (key[1] != 0u) slot1 = __popcll(m0) + __popcll(m1 & lt);
        cnt = __popcll(m0) + __popcll(m1);
        take_all = cnt < K;
        theta = take_all ? 0u : wave_min_u32(min(key[0] != 0u ? key[0] : ~0u, key[1] != 0u ? key[1] : ~0u));
      }
      // rows of lh: those of the list places not kept pass to the entering chunks, then
      // to the places left empty, both in lane order
      const bool freed = lane < K && slot0 < 0, enter = slot1 >= 0;
      const unsigned long long fm = __ballot(freed), em = __ballot(enter);
      const int nenter = __popcll(em);
      if (freed) wscr[__popcll(fm & lt)] = ps;
      __builtin_amdgcn_wave_barrier();
      int row = 0;
      if (enter) row = wscr[__popcll(em & lt)];
      const bool empty = lane >= cnt && lane < K;
      int erow = 0;
      if (empty) erow = wscr[nenter + lane - cnt];
      __builtin_amdgcn_wave_barrier();
      if (slot0 >= 0) {
        lk[qi * K + slot0] = key[0];
        lc[qi * K + slot0] = pc;
        ls[qi * K + slot0] = ps;
      }
      if (enter) {
        lk[qi * K + slot1] = key[1];
        lc[qi * K + slot1] = c;
        ls[qi * K + slot1] = row;
#pragma unroll
        for (int hh = 0; hh < kMaxGroup; ++hh)
          if (hh < G) lh[((size_t)qi * K + row) * G + hh] = hk[hh];
      }
      if (empty) {
        lk[qi * K + lane] = 0u;
        lc[qi * K + lane] = -1;
        ls[qi * K + lane] = erow;
      }
      if (lane == 0) lth[qi] = take_all ? 0u : theta;
    }
  };
  auto end_batch = [&](int bi) {
    lds_block_barrier();   // the batch's keys are in the table
    select_batch(bi);
    lds_block_barrier();   // the table is free for the next batch
  };

  if (K > 0) {
    if (hw) {
      TileBuf tb[NBUF];
#pragma unroll
      for (int u = 0; u < NBUF - 1; ++u)
        if (u < NMT) load_tile(u, tb[u]);
      for (int bi = 0; bi < nbatch; ++bi) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          const int it = bi * TB + u;
          if (it < NMT) {   // wave-uniform
            if (it + NBUF - 1 < NMT) load_tile(it + NBUF - 1, tb[(u + NBUF - 1) % NBUF]);
            score_tile(it, tb[u % NBUF]);
          }
        }
        end_batch(bi);
      }
    } else {
      for (int bi = 0; bi < nbatch; ++bi) end_batch(bi);
    }
  }

  // the lists out (already in ascending chunk order, empty places last)
  for (int qq = 0; qq < QW; ++qq) {
    const int qi = w + kRsWaves * qq, t = t0 + qi;
    if (t >= nq || K == 0) break;
    if (lane < K) {
      const bool valid = lk[qi * K + lane] != 0u;
      const int ps = ls[qi * K + lane];
      idx[((size_t)bg * nq + t) * K + lane] = valid ? lc[qi * K + lane] : -1;
      for (int hh = 0; hh < G; ++hh)
        zsel[(((size_t)b * Hq + g * G + hh) * nq + t) * K + lane] =
            valid ? key_to_float(lh[((size_t)qi * K + ps) * G + hh]) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------- 5. decode-sized scoring (bf16)
//
// A decode step routes at most 32 queries: the residual weights and the
// summaries are the only large operands, so these kernels put every CU's loads
// in flight at once instead of walking them from a few blocks.
//  5a. u_small_kernel: partial u = x A over 256 rows of A per block. The block's
//      rows of A go to LDS in one pass, each wave multiplies a quarter of the
//      k-steps for all queries, and the four wave partials are summed in LDS.
//  5b. qtilde_dec_kernel: one block per head sums the block partials and forms
//      q~ = q + u B_h (u split into bf16 hi + lo, B exact), stored as bf16 hi
//      and lo planes: the B operand of the scoring product.
//  5c. score_small_kernel: one block per (batch, group, 32 chunks). The
//      summaries of every head of the group are moved into LDS with
//      direct-to-LDS loads in one burst (16-byte pieces XOR-swizzled by row so
//      that the fragment reads are conflict free); wave w scores heads w,
//      w + 4 for all 32 chunks x 32 queries with the split products of
//      score_kernel, and the group maximum is taken through LDS. (Every block
//      reads its group's q~, so smaller chunk tiles would re-read more of it.)
//  5d. topk_small_kernel: one block per (batch, group, query). Each wave finds
//      the top K of its own range of chunks; every member of the overall top K
//      is in the top K of its range, so one wave then selects the final K from
//      the at most 4K survivors with the same bisection and tie rule.
constexpr int kDecQ = 32;          // queries of the decode-sized path
constexpr int kUSmallRows = 256;   // rows of A per u_small_kernel block

template <int RP>
__global__ __launch_bounds__(256) void u_small_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ A,
                                                      int Dh, int r, float* __restrict__ upart, int N, int q0,
                                                      int nq) {
  constexpr int AS = RP + 16;                        // LDS row stride of A (elements)
  constexpr int US = RP + 4;                         // LDS row stride of the wave partials (floats)
  constexpr int kPer = kUSmallRows * RP / 8 / 256;   // 16-byte pieces of A per thread
  constexpr int KSW = kUSmallRows / 32 / 4;          // 32-wide k-steps per wave
  constexpr int kABytes = kUSmallRows * AS * 2, kRBytes = 4 * kDecQ * US * 4;
  __shared__ __align__(16) unsigned char smem[kABytes > kRBytes ? kABytes : kRBytes];
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  bf16_t* a_s = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4, L16 = lane & 15;
  const int split = blockIdx.x, b = blockIdx.y;
  const long long L = (long long)N * kSlots;
  const int k0 = split * kUSmallRows;
  const bool vec = (r == RP) && (Dh % 8 == 0);

  // the block's rows of A (zero past Dh and past r) and this wave's x fragments;
  // every load is issued before any is used
  u32x4 av[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = 8 * (tid + 256 * j);
    const int kk = e / RP, n = e % RP, k = k0 + kk;
    if (vec) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(A + (size_t)(k < Dh ? k : Dh - 1) * r + n);
      av[j] = k < Dh ? v : u32x4{0u, 0u, 0u, 0u};
    } else {
      s16x8 t;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) t[jj] = (k < Dh && n + jj < r) ? (short)A[(size_t)k * r + n + jj] : (short)0;
      av[j] = __builtin_bit_cast(u32x4, t);
    }
  }
  s16x8 xf[KSW][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int t = 16 * mt + L16;
    const bf16_t* row = x + ((size_t)b * L + slot_of((long long)q0 + (t < nq ? t : 0))) * Dh;
#pragma unroll
    for (int kk = 0; kk < KSW; ++kk) {
      const int kg = k0 + 32 * (w + 4 * kk) + 8 * g16;
      if (vec) {
        const s16x8 v = load8(row + (kg < Dh ? kg : 0));
        xf[kk][mt] = (t < nq && kg < Dh) ? v : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
      } else {
        float xv[8];
        load_row8<bf16_t>(row, kg, Dh, xv);
        xf[kk][mt] = t < nq ? pack8(xv) : s16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = 8 * (tid + 256 * j);
    *reinterpret_cast<u32x4*>(a_s + (e / RP) * AS + (e % RP)) = av[j];
  }
  __syncthreads();
  f32x4 acc[2][RP / 16];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < RP / 16; ++nt) acc[mt][nt] = zero4();
#pragma unroll
  for (int kk = 0; kk < KSW; ++kk) {
    const int kl = 32 * (w + 4 * kk) + 8 * g16;   // row of A within the block
#pragma unroll
    for (int nt = 0; nt < RP / 16; ++nt) {
      const s16x8 bf = lds_col_frag(a_s, AS, kl, kl + 4, 16 * nt, lane);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma16(xf[kk][mt], bf, acc[mt][nt]);
    }
  }
  __syncthreads();   // every wave is done reading A
  float* red = reinterpret_cast<float*>(smem);
  // D layout: lane holds u[query 16 mt + 4 g16 + i][rank 16 nt + L16]
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < RP / 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(w * kDecQ + 16 * mt + 4 * g16 + i) * US + 16 * nt + L16] = acc[mt][nt][i];
  __syncthreads();
  float* up = upart + ((size_t)split * gridDim.y + b) * (size_t)nq * RP;
  for (int e = tid; e < nq * RP; e += 256) {
    const int t = e / RP, n = e - t * RP;
    up[e] = ((red[t * US + n] + red[(kDecQ + t) * US + n]) + red[(2 * kDecQ + t) * US + n]) +
            red[(3 * kDecQ + t) * US + n];
  }
}

template <int D, int RP>
__global__ __launch_bounds__(256) void qtilde_dec_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ Bm,
                                                         int r, const float* __restrict__ upart, int nsplit,
                                                         bf16_t* __restrict__ qp, int Hq, int N, int q0, int nq) {
  constexpr int BS = D + 16, US = RP + 4;
  constexpr int NTW = D / 32;                       // 16-column tiles per wave (two waves per query tile)
  constexpr int kBPer = RP * D / 8 / 256;           // 16-byte pieces of B_h per thread
  constexpr int kUPer = kDecQ * RP / 4 / 256;       // float4 groups of u per thread
  static_assert(kBPer >= 1 && kUPer >= 1, "tile sizes");
  __shared__ __align__(16) bf16_t b_s[RP * BS];
  __shared__ __align__(16) float u_s[kDecQ * US];
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4, L16 = lane & 15;
  const int h = blockIdx.x, b = blockIdx.y, B = gridDim.y;
  const long long L = (long long)N * kSlots;
  const int mt = w & 1, nh = w >> 1;

  // loads first: B_h slice, q values of this lane's outputs, the u partials
  u32x4 bv[kBPer];
#pragma unroll
  for (int j = 0; j < kBPer; ++j) {
    const int e = tid + 256 * j, kk = (8 * e) / D, n = (8 * e) % D;
    const u32x4 v = *reinterpret_cast<const u32x4*>(Bm + (size_t)(kk < r ? kk : 0) * Hq * D + (size_t)h * D + n);
    bv[j] = kk < r ? v : u32x4{0u, 0u, 0u, 0u};
  }
  float qv[NTW][4];
#pragma unroll
  for (int nn = 0; nn < NTW; ++nn)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g16 + i, dd = 16 * (nh * NTW + nn) + L16;
      const long long sl = slot_of((long long)q0 + (t < nq ? t : 0));
      qv[nn][i] = bf2f(q[((size_t)b * Hq + h) * L * D + (size_t)sl * D + dd]);
    }
  f32x4 us[kUPer];
#pragma unroll
  for (int j = 0; j < kUPer; ++j) us[j] = zero4();
  constexpr int kSB = 16;   // partials loaded per round (all of them for a hidden size up to 4096)
  for (int sp0 = 0; sp0 < nsplit; sp0 += kSB) {
    f32x4 v[kSB][kUPer];
#pragma unroll
    for (int qq = 0; qq < kSB; ++qq) {
      const int sp = sp0 + qq < nsplit ? sp0 + qq : nsplit - 1;
#pragma unroll
      for (int j = 0; j < kUPer; ++j) {
        const int e = 4 * (tid + 256 * j), t = e / RP, n = e % RP;
        v[qq][j] = *reinterpret_cast<const f32x4*>(upart + (((size_t)sp * B + b) * nq + (t < nq ? t : 0)) * RP + n);
      }
    }
#pragma unroll
    for (int qq = 0; qq < kSB; ++qq)
#pragma unroll
      for (int j = 0; j < kUPer; ++j) {
        const int t = 4 * (tid + 256 * j) / RP;
        if (sp0 + qq < nsplit && t < nq) us[j] += v[qq][j];
      }
  }
#pragma unroll
  for (int j = 0; j < kBPer; ++j) {
    const int e = tid + 256 * j;
    *reinterpret_cast<u32x4*>(b_s + ((8 * e) / D) * BS + (8 * e) % D) = bv[j];
  }
#pragma unroll
  for (int j = 0; j < kUPer; ++j) {
    const int e = 4 * (tid + 256 * j);
    *reinterpret_cast<f32x4*>(u_s + (e / RP) * US + e % RP) = us[j];
  }
  __syncthreads();

  // q~ tile: wave w takes query rows 16 (w & 1) .. + 15 and half of the head dimension
  s16x8 uh[RP / 32], ul[RP / 32];
#pragma unroll
  for (int ks = 0; ks < RP / 32; ++ks) {
    float uv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) uv[j] = u_s[(16 * mt + L16) * US + 32 * ks + 8 * g16 + j];
    pack8_split_hw(uv, uh[ks], ul[ks]);
  }
#pragma unroll
  for (int nn = 0; nn < NTW; ++nn) {
    const int nt = nh * NTW + nn;
    f32x4 c = zero4();
#pragma unroll
    for (int ks = 0; ks < RP / 32; ++ks) {
      const s16x8 bh = lds_col_frag(b_s, BS, 32 * ks + 8 * g16, 32 * ks + 8 * g16 + 4, 16 * nt, lane);
      c = mfma16(ul[ks], bh, c);
      c = mfma16(uh[ks], bh, c);
    }
    const int dd = 16 * nt + L16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g16 + i;
      bf16_t hi, lo;
      split_bf16(t < nq ? qv[nn][i] + c[i] : 0.f, hi, lo);
      bf16_t* dst = qp + (((size_t)b * Hq + h) * kDecQ + t) * 2 * D;
      dst[dd] = hi;
      dst[D + dd] = lo;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void score_small_kernel(const bf16_t* __restrict__ qp, const float* __restrict__ s,
                                                          const float* __restrict__ H, float beta, float scale,
                                                          float* __restrict__ z, float* __restrict__ zhat, int Hq,
                                                          int Hkv, int N, int nq) {
  extern __shared__ __align__(16) unsigned char smem[];   // summaries [G][32][D] f32, then wave maxima [4][16][64]
  constexpr int PR = D / 4;          // 16-byte pieces per summary row
  constexpr int RPI = 64 / PR;       // rows per 1 KB direct-to-LDS load
  constexpr int IPH = 32 / RPI;      // loads per head
  constexpr int KS = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, g16 = lane >> 4, L16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = blockIdx.x * 32, bg = blockIdx.y, b = bg / Hkv, g = bg - b * Hkv;
  const int G = Hq / Hkv;
  float* s_l = reinterpret_cast<float*>(smem);
  float* zm = s_l + (size_t)G * 32 * D;

  // 1. wave w moves rows c0 .. c0 + 31 (clamped to N - 1) of its own heads' summaries
  //    (heads w and w + 4) into LDS, each after that head's B operands and entropies:
  //    it scores its first head while the second one's rows are still in flight, and
  //    no wave waits for another one's loads. LDS piece p of row `row` holds source
  //    piece p ^ (row & 15).
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)smem);
  const int prow = lane / PR, pp = lane - prow * PR;
  const int nhw = G > w ? (G - w + 3) / 4 : 0;   // 0, 1 or 2 heads
  s16x8 qb[2][2][KS][2];                          // [head slot][query tile][k-step][plane]
  float hv[2][2][4];                              // [head slot][chunk tile][i]
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const int hh = min(w + 4 * hs, G - 1), h = g * G + hh;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const bf16_t* row = qp + (((size_t)b * Hq + h) * kDecQ + 16 * nt + L16) * 2 * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) qb[hs][nt][ks][pl] = load8(row + pl * D + 32 * ks + 8 * g16);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + 16 * mt + 4 * g16 + i;
        hv[hs][mt][i] = H[((size_t)b * Hq + h) * N + (c < N ? c : N - 1)];
      }
    if (hs < nhw) {
      const float* sh = s + ((size_t)b * Hq + h) * N * D;
#pragma unroll
      for (int ii = 0; ii < IPH; ++ii) {
        const int r0 = ii * RPI, row = r0 + prow;
        const int c = min(c0 + row, N - 1);
        const int voff = (c * D + ((pp ^ (row & 15)) << 2)) * 4;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(
                         lds0 + (uint32_t)((hh * 32 + r0) * D * 4)),
                     "v"(voff), "s"(sh)
                     : "memory", "m0");
      }
    }
  }

  // 3. scores of this wave's heads; the wave's maximum over them
  float zmx[2][2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) zmx[mt][nt][i] = -INFINITY;
  const bool vec_out = (N & 3) == 0;
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    if (hs >= nhw) break;
    // this head's rows and operands have landed: all of this wave's loads but the
    // second head's rows (the last IPH issued) for the first head, all for the second
    if (hs == 0 && nhw == 2) wait_vm<IPH>();
    else wait_vm<0>();
    const int hh = w + 4 * hs, h = g * G + hh;
    f32x4 ahi[2][2], ax[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        ahi[mt][nt] = zero4();
        ax[mt][nt] = zero4();
      }
      const int row = 16 * mt + L16;
      const float* rp = s_l + ((size_t)hh * 32 + row) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int pc = 8 * ks + 2 * g16;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(rp + ((pc ^ (row & 15)) << 2));
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(rp + (((pc + 1) ^ (row & 15)) << 2));
        const float av[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        s16x8 a[2];
        split_ns<2>(av, a);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          ax[mt][nt] = mfma16(a[0], qb[hs][nt][ks][1], ax[mt][nt]);
          ax[mt][nt] = mfma16(a[1], qb[hs][nt][ks][0], ax[mt][nt]);
          ahi[mt][nt] = mfma16(a[0], qb[hs][nt][ks][0], ahi[mt][nt]);
        }
      }
    }
    // D layout: lane holds chunk c0 + 16 mt + 4 g16 + i (rows), query 16 nt + L16 (column)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int t = 16 * nt + L16, cb = c0 + 16 * mt + 4 * g16;
        float zz[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          zz[i] = (ahi[mt][nt][i] + ax[mt][nt][i]) * scale - beta * hv[hs][mt][i];
          zmx[mt][nt][i] = fmaxf(zmx[mt][nt][i], zz[i]);
        }
        if (t < nq) {
          float* zr = z + (((size_t)b * Hq + h) * nq + t) * N + cb;
          if (vec_out && cb + 3 < N) {
            *reinterpret_cast<f32x4*>(zr) = f32x4{zz[0], zz[1], zz[2], zz[3]};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (cb + i < N) zr[i] = zz[i];
          }
        }
      }
  }
  // 4. group maximum over the four waves; wave w writes (chunk tile w >> 1, query tile w & 1)
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) zm[(w * 16 + (2 * mt + nt) * 4 + i) * 64 + lane] = zmx[mt][nt][i];
  __syncthreads();
  {
    const int mt = w >> 1, nt = w & 1;
    const int t = 16 * nt + L16, cb = c0 + 16 * mt + 4 * g16;
    if (t < nq) {
      float m4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) m = fmaxf(m, zm[(ww * 16 + (2 * mt + nt) * 4 + i) * 64 + lane]);
        m4[i] = m;
      }
      float* zr = zhat + ((size_t)bg * nq + t) * N + cb;
      if (vec_out && cb + 3 < N) {
        *reinterpret_cast<f32x4*>(zr) = f32x4{m4[0], m4[1], m4[2], m4[3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (cb + i < N) zr[i] = m4[i];
      }
    }
  }
}

template <int P>
__global__ __launch_bounds__(256) void topk_small_kernel(const float* __restrict__ zhat, const float* __restrict__ z,
                                                         int32_t* __restrict__ idx, float* __restrict__ zsel, int Hq,
                                                         int Hkv, int N, int nq, int q0, int K, int R) {
  __shared__ uint32_t ckey[4 * 64];   // per wave: its top K keys, in chunk order
  __shared__ int cidx[4 * 64];        // ... and their chunks
  __shared__ int ccount[4];
  __shared__ int chosen[64];
  __shared__ int s_count;
  __shared__ uint32_t nbuf[4][2 * kNarrow];   // per wave: the narrowed candidates
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long row = blockIdx.x;
  const int t = (int)(row % nq);
  const long long bg = row / nq;
  const int b = (int)(bg / Hkv), g = (int)(bg % Hkv);
  const int G = Hq / Hkv;
  const long long i = (long long)q0 + t;
  const float* zr = zhat + row * N;

  // 1. wave w: chunks 64 P w + 64 j + lane
  const int cw = 64 * P * w;
  float zv[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int c = cw + 64 * j + lane;
    zv[j] = zr[c < N ? c : N - 1];   // always in bounds
  }
#pragma unroll
  for (int j = 0; j < P; ++j) asm volatile("" : "+v"(zv[j]));   // keep every load ahead of its first use
  uint32_t key[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int c = cw + 64 * j + lane;
    const bool cand = (c < N) & ((63LL * c + 62 < i - R) | (63LL * c > i + R));
    key[j] = cand ? order_key(zv[j]) : 0u;
  }
  auto keep = [&](int slot, int e, uint32_t kv) {
    ckey[64 * w + slot] = kv;
    cidx[64 * w + slot] = cw + e;
  };
  int nw;
  if constexpr (P >= 8) nw = wave_topk_narrow<P>(key, K, lane, nbuf[w], keep);
  else nw = wave_topk<P>(key, K, lane, [&](int slot, int j) { keep(slot, 64 * j + lane, key[j]); });
  if (lane == 0) ccount[w] = nw;
  __syncthreads();
  // 2. wave 0: the final K from the survivors (element 64 e + l = entry l of wave e's list: chunk order)
  if (w == 0) {
    uint32_t k2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) k2[e] = lane < ccount[e] ? ckey[64 * e + lane] : 0u;
    const int n = wave_topk<4>(k2, K, lane, [&](int slot, int e) { chosen[slot] = cidx[64 * e + lane]; });
    if (lane == 0) s_count = n;
  }
  __syncthreads();
  if (lane < K) {
    const int c = lane < s_count ? chosen[lane] : -1;
    if (w == 0) idx[row * K + lane] = c;
    for (int hh = w; hh < G; hh += 4) {
      const size_t hrow = ((size_t)b * Hq + g * G + hh) * nq + t;
      zsel[hrow * K + lane] = c >= 0 ? z[hrow * N + c] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int rank_pad(int r) { return r <= 32 ? 32 : (r <= 64 ? 64 : 128); }

// Hidden-dimension split of u_kernel: enough blocks to spread small query counts.
static int u_splits(const RouteDims& dm, int Dh, int nq) {
  const int tiles = (nq + 63) / 64 * dm.B;
  const int nslices = (Dh + kUKc - 1) / kUKc;
  int s = (512 + tiles - 1) / tiles;
  if (s > 16) s = 16;   // q_kernel re-reads every partial once per head
  if (s > nslices) s = nslices;
  if (s < 1) s = 1;
  const int per = (nslices + s - 1) / s;
  return (nslices + per - 1) / per;
}

// The one-sweep scoring kernel's LDS (48 queries per block) fits with batches of 64
// chunks, else of 32 (0: neither).
constexpr size_t kScoreLdsMax = 160 * 1024;
static int stream_batch_tiles(const RouteDims& dm, int K) {
  const int G = dm.Hq / dm.Hkv;
  if (K < 1 || K > 64 || G > kMaxGroup) return 0;
  if (ss_lds(3, G, 4, K) <= kScoreLdsMax) return 4;
  if (ss_lds(3, G, 2, K) <= kScoreLdsMax) return 2;
  return 0;
}
constexpr int kStreamMaxN = 16384;   // chunks (about 1M slots)

// bf16 prefill-sized problems take a fused scoring kernel (no q~, z or zhat in memory):
// the two-sweep kernel up to 1,024 chunks (its key table grows with N), the one-sweep
// kernel beyond.
static bool fused_score_ok(const RouteDims& dm, int r, int nq, int K) {
  if (!(dm.dtype == 1 && r <= 64 && nq > kSmallQ && dm.Hq / dm.Hkv <= kMaxGroup)) return false;
  return dm.N <= 1024 || (dm.N <= kStreamMaxN && stream_batch_tiles(dm, K) > 0);
}

// bf16 decode-sized problems (at most 32 queries) take the kernels of section 5.
static bool small_score_ok(const RouteDims& dm, int r, int nq) {
  return dm.dtype == 1 && nq <= kDecQ && r <= 64 && dm.Hq / dm.Hkv <= 8 && dm.N <= 8192;
}
static int u_small_splits(int Dh) { return (Dh + kUSmallRows - 1) / kUSmallRows; }
static int dh_pad(int Dh) { return (Dh + 31) / 32 * 32; }
static size_t at_bytes(int Dh, int r) { return (size_t)rank_pad(r) * dh_pad(Dh) * 2; }   // A transposed
static size_t bt_bytes(const RouteDims& dm, int r) { return (size_t)dm.Hq * dm.d * rank_pad(r) * 2; }   // B transposed
// summaries as fragment-major bf16 hi/lo planes, rows padded to whole 16-chunk tiles
static size_t frag_bytes(const RouteDims& dm) { return (size_t)dm.B * dm.Hq * ((dm.N + 15) / 16 * 16) * 2 * dm.d * 2; }

size_t score_ws_bytes(const RouteDims& dm, int Dh, int r, int nq, int K) {
  const size_t rows_h = (size_t)dm.B * dm.Hq * nq, rows_g = (size_t)dm.B * dm.Hkv * nq;
  if (small_score_ok(dm, r, nq))
    return align256((size_t)u_small_splits(Dh) * dm.B * nq * rank_pad(r) * 4) +
           align256((size_t)dm.B * dm.Hq * kDecQ * 2 * dm.d * 2) + align256(rows_g * dm.N * 4) +
           align256(rows_h * dm.N * 4);
  const size_t upart = (size_t)u_splits(dm, Dh, nq) * dm.B * nq * rank_pad(r) * 4;
  if (fused_score_ok(dm, r, nq, K))
    return align256(upart) + align256(frag_bytes(dm)) + align256(at_bytes(Dh, r)) + align256(bt_bytes(dm, r));
  return align256(rows_h * dm.d * 4) + align256(rows_g * dm.N * 4) + align256(rows_h * dm.N * 4) + align256(upart);
}

ScoreWs score_ws_carve(void* ws, const RouteDims& dm, int Dh, int r, int nq, int K) {
  const size_t rows_h = (size_t)dm.B * dm.Hq * nq, rows_g = (size_t)dm.B * dm.Hkv * nq;
  char* p = (char*)ws;
  ScoreWs out;
  out.splanes = nullptr;
  out.qplanes = nullptr;
  out.at = nullptr;
  out.bt = nullptr;
  if (small_score_ok(dm, r, nq)) {
    out.qt = nullptr;
    out.upart = (float*)p;
    p += align256((size_t)u_small_splits(Dh) * dm.B * nq * rank_pad(r) * 4);
    out.qplanes = (bf16_t*)p;
    p += align256((size_t)dm.B * dm.Hq * kDecQ * 2 * dm.d * 2);
    out.zhat = (float*)p;
    p += align256(rows_g * dm.N * 4);
    out.z = (float*)p;
    return out;
  }
  if (fused_score_ok(dm, r, nq, K)) {
    out.qt = nullptr;
    out.zhat = nullptr;
    out.z = nullptr;
    out.upart = (float*)p;
    p += align256((size_t)u_splits(dm, Dh, nq) * dm.B * nq * rank_pad(r) * 4);
    out.splanes = (bf16_t*)p;
    p += align256(frag_bytes(dm));
    out.at = (bf16_t*)p;
    p += align256(at_bytes(Dh, r));
    out.bt = (bf16_t*)p;
    return out;
  }
  out.qt = (float*)p;
  p += align256(rows_h * dm.d * 4);
  out.zhat = (float*)p;
  p += align256(rows_g * dm.N * 4);
  out.z = (float*)p;
  p += align256(rows_h * dm.N * 4);
  out.upart = (float*)p;
  return out;
}

template <typename T, int D, int RP>
static void launch_qtilde(const RouteDims& dm, const void* q, const void* x, const void* A, const void* Bm,
                          int Dh, int r, const ScoreWs& ws, int q0, int nq, hipStream_t st) {
  if constexpr (sizeof(T) == 2 && RP <= 64) {   // rank 128 would not fit the LDS staging
    if (nq <= kSmallQ) {
      hipLaunchKernelGGL((qtilde_small_kernel<D, RP>), dim3(dm.Hq, dm.B), dim3(64 * kSmallW), 0, st, (const bf16_t*)q,
                         (const bf16_t*)x, (const bf16_t*)A, (const bf16_t*)Bm, Dh, r, ws.qt, dm.Hq, dm.N, q0, nq);
      return;
    }
  }
  const int nsplit = u_splits(dm, Dh, nq);
  const int nslices = (Dh + kUKc - 1) / kUKc;
  const int per = (nslices + nsplit - 1) / nsplit;
  hipLaunchKernelGGL((u_kernel<T, RP>), dim3((nq + 63) / 64, dm.B, nsplit), dim3(256), 0, st, (const T*)x,
                     (const T*)A, Dh, r, ws.upart, dm.N, q0, nq, per);
  hipLaunchKernelGGL((q_kernel<T, D, RP>), dim3((nq + 63) / 64, dm.Hq, dm.B), dim3(256), 0, st, (const T*)q,
                     (const T*)Bm, r, ws.upart, nsplit, ws.qt, dm.Hq, dm.N, q0, nq);
}

template <typename T, int D>
static void launch_qtilde_r(const RouteDims& dm, const void* q, const void* x, const void* A, const void* Bm,
                            int Dh, int r, const ScoreWs& ws, int q0, int nq, hipStream_t st) {
  if (r <= 32) launch_qtilde<T, D, 32>(dm, q, x, A, Bm, Dh, r, ws, q0, nq, st);
  else if (r <= 64) launch_qtilde<T, D, 64>(dm, q, x, A, Bm, Dh, r, ws, q0, nq, st);
  else launch_qtilde<T, D, 128>(dm, q, x, A, Bm, Dh, r, ws, q0, nq, st);
}

template <int P>
static void launch_topk(const RouteDims& dm, const ScoreWs& ws, int32_t* idx, float* zsel, int q0, int nq,
                        int K, int R, hipStream_t st) {
  const long long nrows = (long long)dm.B * dm.Hkv * nq;
  hipLaunchKernelGGL((topk_kernel<P>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, ws.zhat, ws.z, idx,
                     zsel, dm.Hq, dm.Hkv, dm.N, nq, q0, K, R, nrows);
}

template <int D, int RP>
static hipError_t launch_fused_score(const RouteDims& dm, const void* q, const void* x, const void* A,
                                     const void* Bm, int Dh, int r, const float* s, const float* H, float beta,
                                     float scale, int K, int radius, int q0, int nq, int32_t* idx, float* zsel,
                                     const ScoreWs& ws, hipStream_t st) {
  int nsplit;
  hipError_t e;
  if (Dh % 8 == 0) {
    // x streamed once against A transposed: one partial set
    nsplit = 1;
    const int Dhp = dh_pad(Dh);
    hipLaunchKernelGGL((transpose_a_kernel<RP>), dim3((unsigned)(((long long)RP * Dhp + 255) / 256)), dim3(256), 0, st,
                       (const bf16_t*)A, Dh, r, Dhp, ws.at);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto uk = u_stream_kernel<RP>;
    e = hipFuncSetAttribute((const void*)uk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)u_stream_lds(RP));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(uk, dim3((nq + 63) / 64, dm.B), dim3(512), u_stream_lds(RP), st, (const bf16_t*)x, ws.at, Dh,
                       Dhp, ws.upart, dm.N, q0, nq);
  } else {
    nsplit = u_splits(dm, Dh, nq);
    const int nslices = (Dh + kUKc - 1) / kUKc;
    const int per = (nslices + nsplit - 1) / nsplit;
    hipLaunchKernelGGL((u_kernel<bf16_t, RP>), dim3((nq + 63) / 64, dm.B, nsplit), dim3(256), 0, st,
                       (const bf16_t*)x, (const bf16_t*)A, Dh, r, ws.upart, dm.N, q0, nq, per);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long heads = (long long)dm.B * dm.Hq;
  const long long groups8 = heads * ((dm.N + 15) / 16 * 16) * (D / 8);
  hipLaunchKernelGGL((split_frag_kernel<D>), dim3((unsigned)((groups8 + 255) / 256)), dim3(256), 0, st, s, ws.splanes,
                     dm.N, heads);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int HD = dm.Hq * D;
  hipLaunchKernelGGL((transpose_b_kernel<D, RP>), dim3((unsigned)(((long long)HD * RP + 255) / 256)), dim3(256), 0, st,
                     (const bf16_t*)Bm, r, HD, ws.bt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Past 1,024 chunks one sweep, the selection taken during it: 48 queries per block,
  // batches of 64 chunks (32 where those do not fit). Up to 1,024 the two-sweep kernel
  // below is faster (it selects once per query, from all keys; the one-sweep kernel
  // merges once per batch).
  if (dm.N > 1024) {
    const int tiles3 = (nq + 47) / 48 * dm.B * dm.Hkv;
    const int tb = stream_batch_tiles(dm, K);
    if (tb == 0) return hipErrorInvalidValue;   // excluded by fused_score_ok
    {
      const size_t lds = ss_lds(3, dm.Hq / dm.Hkv, tb, K);
      auto kern = tb == 4 ? route_score_stream_kernel<D, RP, 3, 4> : route_score_stream_kernel<D, RP, 3, 2>;
      e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(xcd_grid(tiles3)), dim3(64 * kRsWaves), lds, st, (const bf16_t*)q, ws.bt,
                         ws.upart, nsplit, ws.splanes, H, beta, scale, idx, zsel, dm.B, dm.Hq, dm.Hkv, dm.N, q0, nq,
                         K, radius, tile_order());
      return hipGetLastError();
    }
  }
  // Two sweeps: 48 queries per block up to N = 512 (the q~ of the wave's head for them
  // stays in registers as three 16-query tiles), 32 beyond, where 48 rows of keys would
  // pass the 160 KB of LDS.
  const int NT = dm.N <= 512 ? 3 : 2;
  // zsel staged in LDS when the rows fit
  const bool stage = rs3_lds(NT, dm.N, K, true) <= (size_t)(160 * 1024 - 512);
  const size_t lds = rs3_lds(NT, dm.N, K, stage);
  const int tiles = (nq + 16 * NT - 1) / (16 * NT) * dm.B * dm.Hkv;
#define LCR_RS(NTT, PP)                                                                                          \
  do {                                                                                                           \
    auto kern = stage ? route_score3_kernel<D, RP, NTT, PP, true> : route_score3_kernel<D, RP, NTT, PP, false>;                                                            \
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);          \
    if (e != hipSuccess) return e;                                                                               \
    hipLaunchKernelGGL(kern, dim3(xcd_grid(tiles)), dim3(64 * kRsWaves), lds, st, (const bf16_t*)q, ws.bt,      \
                       ws.upart, nsplit, ws.splanes, H, beta, scale, idx, zsel, dm.B, dm.Hq, dm.Hkv, dm.N, q0, nq, \
                       K, radius, tile_order());                                                                               \
  } while (0)
  if (dm.N <= 256) LCR_RS(3, 4);
  else if (dm.N <= 512) LCR_RS(3, 8);
  else LCR_RS(2, 16);
#undef LCR_RS
  return hipGetLastError();
}

template <int D, int RP>
static hipError_t launch_small_score(const RouteDims& dm, const void* q, const void* x, const void* A,
                                     const void* Bm, int Dh, int r, const float* s, const float* H, float beta,
                                     float scale, int K, int radius, int q0, int nq, int32_t* idx, float* zsel,
                                     const ScoreWs& ws, hipStream_t st) {
  const int nsplit = u_small_splits(Dh);
  hipLaunchKernelGGL((u_small_kernel<RP>), dim3(nsplit, dm.B), dim3(256), 0, st, (const bf16_t*)x,
                     (const bf16_t*)A, Dh, r, ws.upart, dm.N, q0, nq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((qtilde_dec_kernel<D, RP>), dim3(dm.Hq, dm.B), dim3(256), 0, st, (const bf16_t*)q,
                     (const bf16_t*)Bm, r, ws.upart, nsplit, ws.qplanes, dm.Hq, dm.N, q0, nq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)(dm.Hq / dm.Hkv) * 32 * D * 4 + 4 * 16 * 64 * 4;
  auto sk = score_small_kernel<D>;
  e = hipFuncSetAttribute((const void*)sk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sk, dim3((dm.N + 31) / 32, dm.B * dm.Hkv), dim3(256), lds, st, ws.qplanes, s, H, beta, scale,
                     ws.z, ws.zhat, dm.Hq, dm.Hkv, dm.N, nq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rows = (unsigned)(dm.B * dm.Hkv * nq);
  const int P = (dm.N + 255) / 256;
#define LCR_TK(PP)                                                                                           \
  hipLaunchKernelGGL((topk_small_kernel<PP>), dim3(rows), dim3(256), 0, st, ws.zhat, ws.z, idx, zsel, dm.Hq, \
                     dm.Hkv, dm.N, nq, q0, K, radius)
  if (P <= 1) LCR_TK(1);
  else if (P <= 2) LCR_TK(2);
  else if (P <= 4) LCR_TK(4);
  else if (P <= 8) LCR_TK(8);
  else if (P <= 16) LCR_TK(16);
  else LCR_TK(32);
#undef LCR_TK
  return hipGetLastError();
}

// q~ (float32 [B,Hq,nq,d]) and the partial sums of u = x A ([nsplit,B,nq,RP]) through
// the general two-kernel path, for the backward of the scoring.
template <typename T, int D, int RP>
static void launch_qtilde_uq(const RouteDims& dm, const void* q, const void* x, const void* A, const void* Bm,
                             int Dh, int r, float* qt, float* upart, int q0, int nq, hipStream_t st) {
  const int nsplit = u_splits(dm, Dh, nq);
  const int nslices = (Dh + kUKc - 1) / kUKc;
  const int per = (nslices + nsplit - 1) / nsplit;
  hipLaunchKernelGGL((u_kernel<T, RP>), dim3((nq + 63) / 64, dm.B, nsplit), dim3(256), 0, st, (const T*)x,
                     (const T*)A, Dh, r, upart, dm.N, q0, nq, per);
  hipLaunchKernelGGL((q_kernel<T, D, RP>), dim3((nq + 63) / 64, dm.Hq, dm.B), dim3(256), 0, st, (const T*)q,
                     (const T*)Bm, r, upart, nsplit, qt, dm.Hq, dm.N, q0, nq);
}

template <typename T, int D>
static void launch_qtilde_uq_r(const RouteDims& dm, const void* q, const void* x, const void* A, const void* Bm,
                               int Dh, int r, float* qt, float* upart, int q0, int nq, hipStream_t st) {
  if (r <= 32) launch_qtilde_uq<T, D, 32>(dm, q, x, A, Bm, Dh, r, qt, upart, q0, nq, st);
  else if (r <= 64) launch_qtilde_uq<T, D, 64>(dm, q, x, A, Bm, Dh, r, qt, upart, q0, nq, st);
  else launch_qtilde_uq<T, D, 128>(dm, q, x, A, Bm, Dh, r, qt, upart, q0, nq, st);
}

int qtilde_u_splits(const RouteDims& dm, int Dh, int nq) { return nq > 0 ? u_splits(dm, Dh, nq) : 1; }
int qtilde_rank_pad(int r) { return rank_pad(r); }

hipError_t launch_qtilde_with_u(const RouteDims& dm, const void* q, const void* x, const void* A, const void* Bm,
                                int Dh, int r, float* qt, float* upart, int q0, int nq, hipStream_t st) {
  if (dm.dtype == 1) {
    if (dm.d == 64) launch_qtilde_uq_r<bf16_t, 64>(dm, q, x, A, Bm, Dh, r, qt, upart, q0, nq, st);
    else launch_qtilde_uq_r<bf16_t, 128>(dm, q, x, A, Bm, Dh, r, qt, upart, q0, nq, st);
  } else {
    if (dm.d == 64) launch_qtilde_uq_r<float, 64>(dm, q, x, A, Bm, Dh, r, qt, upart, q0, nq, st);
    else launch_qtilde_uq_r<float, 128>(dm, q, x, A, Bm, Dh, r, qt, upart, q0, nq, st);
  }
  return hipGetLastError();
}

hipError_t launch_route_score_topk(const RouteDims& dm, const void* q, const void* x, const void* A,
                                   const void* Bm, int D, int r, const float* s, const float* H,
                                   float beta, float scale, int K, int radius, int q0, int nq,
                                   int32_t* idx, float* zsel, const ScoreWs& ws, hipStream_t st) {
  if (small_score_ok(dm, r, nq)) {
    if (dm.d == 64) return r <= 32 ? launch_small_score<64, 32>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st)
                                   : launch_small_score<64, 64>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st);
    return r <= 32 ? launch_small_score<128, 32>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st)
                   : launch_small_score<128, 64>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st);
  }
  if (fused_score_ok(dm, r, nq, K)) {
    if (dm.d == 64) return r <= 32 ? launch_fused_score<64, 32>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st)
                                   : launch_fused_score<64, 64>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st);
    return r <= 32 ? launch_fused_score<128, 32>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st)
                   : launch_fused_score<128, 64>(dm, q, x, A, Bm, D, r, s, H, beta, scale, K, radius, q0, nq, idx, zsel, ws, st);
  }
  if (dm.dtype == 1) {
    if (dm.d == 64) launch_qtilde_r<bf16_t, 64>(dm, q, x, A, Bm, D, r, ws, q0, nq, st);
    else launch_qtilde_r<bf16_t, 128>(dm, q, x, A, Bm, D, r, ws, q0, nq, st);
  } else {
    if (dm.d == 64) launch_qtilde_r<float, 64>(dm, q, x, A, Bm, D, r, ws, q0, nq, st);
    else launch_qtilde_r<float, 128>(dm, q, x, A, Bm, D, r, ws, q0, nq, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((dm.N + 63) / 64, (nq + 15) / 16, dm.B * dm.Hkv);
  const bool pipe = (long long)grid.x * grid.y * grid.z < 2048;
#define LCR_SCORE(DD, NS)                                                                                   \
  do {                                                                                                      \
    if (pipe)                                                                                               \
      hipLaunchKernelGGL((score_kernel<DD, NS, true>), grid, dim3(256), 0, st, ws.qt, s, H, beta, scale, ws.z, \
                         ws.zhat, dm.Hq, dm.Hkv, dm.N, nq);                                                   \
    else                                                                                                    \
      hipLaunchKernelGGL((score_kernel<DD, NS, false>), grid, dim3(256), 0, st, ws.qt, s, H, beta, scale,     \
                         ws.z, ws.zhat, dm.Hq, dm.Hkv, dm.N, nq);                                             \
  } while (0)
  if (dm.d == 64) {
    if (dm.dtype == 1) LCR_SCORE(64, 2);
    else LCR_SCORE(64, 3);
  } else {
    if (dm.dtype == 1) LCR_SCORE(128, 2);
    else LCR_SCORE(128, 3);
  }
#undef LCR_SCORE
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int P = (dm.N + 63) / 64;
  if (P <= 1) launch_topk<1>(dm, ws, idx, zsel, q0, nq, K, radius, st);
  else if (P <= 2) launch_topk<2>(dm, ws, idx, zsel, q0, nq, K, radius, st);
  else if (P <= 4) launch_topk<4>(dm, ws, idx, zsel, q0, nq, K, radius, st);
  else if (P <= 8) launch_topk<8>(dm, ws, idx, zsel, q0, nq, K, radius, st);
  else if (P <= 16) launch_topk<16>(dm, ws, idx, zsel, q0, nq, K, radius, st);
  else if (P <= 32) launch_topk<32>(dm, ws, idx, zsel, q0, nq, K, radius, st);
  else launch_topk<64>(dm, ws, idx, zsel, q0, nq, K, radius, st);
  return hipGetLastError();
}

}  // namespace lcr
