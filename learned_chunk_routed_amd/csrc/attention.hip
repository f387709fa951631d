// Routed attention and bidirectional sliding-window attention on gfx950.
//
// Routed attention: "Prefilling-dLLM v2: Learned Chunk Routing for Long-Context
// Diffusion Language Models", Figure 3 caption: the selected chunk scores and
// the local window's log-sum-exp share one softmax partition, then a second
// softmax spreads each chunk's mass over its content tokens. "The 172x Speedup
// Has an Evidence Budget": mass is allocated jointly between chosen remote
// chunks and the local window, then among content tokens inside each chunk.
//
// Algebra used here: the two-level softmax equals one softmax over a virtual
// key set in which window key u has logit a_u and content key j of selected
// chunk c has logit z_c + l_j - LSE_c (l_j its plain logit, LSE_c the chunk's
// log-sum-exp). Chunk c's keys then carry total mass e^{z_c}, exactly the
// partition weight of the chunk. So one online-softmax accumulator per row
// serves both kinds of key: a window chunk updates the running maximum with its
// key logits; a selected chunk updates it with z_c and adds its normalised
// intra-chunk distribution scaled by e^{z_c - m}.
//
// Work decomposition (gfx950, 64-wide waves, 16x16x32 bf16 MFMA):
//  - A tile is 16 MFMA columns = 2 consecutive queries x 8 head rows (the G
//    heads of one KV group; G <= 8). S^T = K_c Q^T puts the chunk's 64 slots on
//    the M side; the S^T output fragment is directly the B operand of
//    O^T += V^T P^T (same lane -> key assignment), so P never leaves registers.
//  - A block owns a run of consecutive queries of one (batch, KV group) and
//    walks the ascending union of every chunk its queries need (window chunks
//    and selected chunks). Each chunk's K and V (64 x d, contiguous in HBM) is
//    staged once into LDS and shared by every wave of the block; V stays
//    row-major and is read transposed with ds_read_b64_tr_b16.
//  - Decode-sized problems split a query block's chunk list across several
//    blocks; each writes an unnormalised partial (m, l, O) and a combine
//    kernel merges them.
// Sliding-window attention uses the same tile machinery with 16 consecutive
// slots of one head per tile and a band mask.
#include "device.h"
#include "launch.h"

namespace lcr {

__device__ __forceinline__ long long slot_of_i(long long i) { return (i / kContent) * kSlots + (i % kContent); }

template <int D> struct Strides {
  static constexpr int K = D + 8;    // K rows: 16-byte fragment reads, conflict-free
  static constexpr int V = D + 16;   // V rows: 8-byte transpose reads, conflict-free
};

// ---------------------------------------------------------------- operand planes
// bf16 inputs use one bf16 plane. float32 inputs are split into three bf16
// planes x = hi + mid + lo (24 significant bits) and every product keeps the
// six plane pairs whose order is at least 2^-16 (hi.hi, hi.mid, mid.hi,
// hi.lo, lo.hi, mid.mid), smallest first: near-float32 accuracy on MFMA.

template <typename T> struct NPlanes { static constexpr int value = sizeof(T) == 4 ? 3 : 1; };

template <int NP>
__device__ __forceinline__ void split_planes(float x, bf16_t* out) {
  if constexpr (NP == 1) {
    out[0] = f2bf(x);
  } else {
    const bf16_t h = f2bf(x);
    const float r = x - bf2f(h);
    const bf16_t m = f2bf(r);
    out[0] = h;
    out[1] = m;
    out[2] = f2bf(r - bf2f(m));
  }
}

template <int NP>
__device__ __forceinline__ f32x4 mfma_planes(const s16x8* a, const s16x8* b, f32x4 c) {
  if constexpr (NP == 3) {
    c = mfma16(a[0], b[2], c);
    c = mfma16(a[2], b[0], c);
    c = mfma16(a[1], b[1], c);
    c = mfma16(a[0], b[1], c);
    c = mfma16(a[1], b[0], c);
  }
  return mfma16(a[0], b[0], c);
}

// One buffer holds, per plane, 64 K rows (stride KS) then 64 V rows (stride VS).
template <int D> struct KV {
  static constexpr int KS = Strides<D>::K;
  static constexpr int VS = Strides<D>::V;
  static constexpr int PL = 64 * (KS + VS);     // elements per plane
};
template <int D, int NP>
__host__ __device__ constexpr int kv_buf_elems() { return NP * KV<D>::PL; }
// Two buffers (load of the next tile overlaps compute) unless they would not
// fit: three float32-derived planes at d = 128 use one.
template <int D, int NP>
__host__ __device__ constexpr int kv_nbuf() { return (NP == 3 && D == 128) ? 1 : 2; }

// ---------------------------------------------------------------- staging of one 64-slot K/V tile

template <typename T, int D, int NT>
struct KVStage {
  static constexpr int NP = NPlanes<T>::value;
  static constexpr int kElems = 16 / sizeof(T);          // elements per 16-byte piece
  static constexpr int kPerRow = D / kElems;
  static constexpr int kPieces = 64 * kPerRow;           // per tensor
  static constexpr int kPer = (kPieces + NT - 1) / NT;
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  u32x4 kr[kPer], vr[kPer];

  __device__ __forceinline__ void load(const T* kb, const T* vb, int tid, int rows_valid) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int pc = tid + j * NT;
      const int row = pc / kPerRow;
      if (pc < kPieces && row < rows_valid) {
        kr[j] = *reinterpret_cast<const u32x4*>(kb + (size_t)pc * kElems);
        vr[j] = *reinterpret_cast<const u32x4*>(vb + (size_t)pc * kElems);
      } else {
        kr[j] = u32x4{0u, 0u, 0u, 0u};
        vr[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* buf, int tid) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int pc = tid + j * NT;
      if (pc >= kPieces) continue;
      const int row = pc / kPerRow, col = (pc - row * kPerRow) * kElems;
      if constexpr (NP == 1) {
        *reinterpret_cast<u32x4*>(buf + row * KV<D>::KS + col) = kr[j];
        *reinterpret_cast<u32x4*>(buf + 64 * KV<D>::KS + row * KV<D>::VS + col) = vr[j];
      } else {
        s16x4 kp[NP], vp[NP];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16_t t[NP];
          split_planes<NP>(__uint_as_float(kr[j][e]), t);
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) kp[pl][e] = (short)t[pl];
          split_planes<NP>(__uint_as_float(vr[j][e]), t);
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) vp[pl][e] = (short)t[pl];
        }
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) {
          *reinterpret_cast<s16x4*>(buf + pl * KV<D>::PL + row * KV<D>::KS + col) = kp[pl];
          *reinterpret_cast<s16x4*>(buf + pl * KV<D>::PL + 64 * KV<D>::KS + row * KV<D>::VS + col) = vp[pl];
        }
      }
    }
  }
};

// ---------------------------------------------------------------- per-tile fragments and products

template <int D, int NP> struct QFrag {
  s16x8 f[D / 32][NP];
};

// B operand of S^T = K Q^T: lane l holds row (l%16) of Q, d = 32*ks + 8*(l/16) + j.
template <typename T, int D, int NP>
__device__ __forceinline__ void load_qfrag(QFrag<D, NP>& q, const T* row, int lane) {
  const int g16 = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    if (row == nullptr) {
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) q.f[ks][pl] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
      continue;
    }
    if constexpr (NP == 1) {
      q.f[ks][0] = load8(reinterpret_cast<const bf16_t*>(row) + 32 * ks + 8 * g16);
    } else {
      const float* rf = reinterpret_cast<const float*>(row) + 32 * ks + 8 * g16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16_t t[NP];
        split_planes<NP>(rf[j], t);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) q.f[ks][pl][j] = (short)t[pl];
      }
    }
  }
}

// S^T for 64 key slots x 16 rows: acc[mt] holds keys 16*mt + 4*(l/16) + i, row l%16.
template <int D, int NP>
__device__ __forceinline__ void s_tile(const bf16_t* buf, const QFrag<D, NP>& q, f32x4 acc[4], int lane) {
  const int L16 = lane & 15, g16 = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int off = (16 * mt + L16) * KV<D>::KS + 32 * ks + 8 * g16;
      s16x8 a[NP];
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) a[pl] = load8(buf + pl * KV<D>::PL + off);
      acc[mt] = mfma_planes<NP>(a, q.f[ks], acc[mt]);
    }
  }
}

// O^T[d][row] += sum_key V[key][d] p[row][key] with p in the S^T output layout.
template <int D, int NP>
__device__ __forceinline__ void pv_tile(const bf16_t* buf, const float p[4][4], f32x4 o[D / 16], int lane) {
  const int g16 = lane >> 4;
  s16x8 pf[2][NP];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pv = j < 4 ? p[2 * ks][j] : p[2 * ks + 1][j - 4];
      bf16_t t[NP];
      split_planes<NP>(pv, t);
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) pf[ks][pl][j] = (short)t[pl];
    }
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      s16x8 a[NP];
#pragma unroll
      for (int pl = 0; pl < NP; ++pl)
        a[pl] = lds_col_frag(buf + pl * KV<D>::PL + 64 * KV<D>::KS, KV<D>::VS, 32 * ks + 4 * g16,
                             32 * ks + 16 + 4 * g16, 16 * dm, lane);
      o[dm] = mfma_planes<NP>(a, pf[ks], o[dm]);
    }
  }
}

// Store 4 consecutive output values of a row.
template <typename T>
__device__ __forceinline__ void store4(T* dst, const float* v);
template <>
__device__ __forceinline__ void store4<float>(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* dst, const float* v) {
  *reinterpret_cast<s16x4*>(dst) = s16x4{(short)f2bf(v[0]), (short)f2bf(v[1]), (short)f2bf(v[2]), (short)f2bf(v[3])};
}

// ---------------------------------------------------------------- routed attention

struct RoutedParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  const float* zsel;
  void* o;
  float* lse;
  float* part;
  int B, Hq, Hkv, N, K, R, q0, nq, nsplit;
  float sl2;  // scale * log2(e)
};

template <typename T, int D, int WAVES, int TPW>
__global__ __launch_bounds__(WAVES * 64) void routed_attention_kernel(RoutedParams p) {
  constexpr int NP = NPlanes<T>::value;
  constexpr int NT = WAVES * 64;
  constexpr int QB = 2 * WAVES * TPW;
  constexpr int KVB = kv_buf_elems<D, NP>();
  constexpr int NBUF = kv_nbuf<D, NP>();
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* kvb = reinterpret_cast<bf16_t*>(smem);
  int* sel = reinterpret_cast<int*>(smem + NBUF * KVB * sizeof(bf16_t));
  int* list = sel + QB * p.K;
  unsigned char* flags = reinterpret_cast<unsigned char*>(list + p.N);
  __shared__ int s_nlist;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4;
  const int bg = blockIdx.y, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int tb0 = blockIdx.x * QB;
  const int split = blockIdx.z;
  const long long L = (long long)p.N * kSlots;
  const long long Tcont = (long long)p.N * kContent;
  const T* kg = reinterpret_cast<const T*>(p.k) + (size_t)bg * L * D;
  const T* vg = reinterpret_cast<const T*>(p.v) + (size_t)bg * L * D;

  // ---- the ascending union of chunks needed by this block's queries
  for (int c = tid; c < p.N; c += NT) flags[c] = 0;
  __syncthreads();
  for (int e = tid; e < QB * p.K; e += NT) {
    const int qi = e / p.K, kk = e - qi * p.K, t = tb0 + qi;
    int c = (t < p.nq) ? p.idx[((size_t)bg * p.nq + t) * p.K + kk] : -1;
    if (c >= p.N) c = -1;
    sel[e] = c;
    if (c >= 0) flags[c] = 1;
  }
  {
    const int t_last = min(tb0 + QB, p.nq) - 1;
    const long long i_first = (long long)p.q0 + tb0, i_last = (long long)p.q0 + t_last;
    const int cw0 = (int)(max(0LL, i_first - p.R) / kContent);
    const int cw1 = (int)(min(Tcont - 1, i_last + p.R) / kContent);
    for (int c = cw0 + tid; c <= cw1; c += NT) flags[c] = 1;
  }
  __syncthreads();
  if (w == 0) {
    int base = 0;
    for (int c0 = 0; c0 < p.N; c0 += 64) {
      const int c = c0 + lane;
      const bool f = c < p.N && flags[c];
      const unsigned long long m = __ballot(f);
      if (f) list[base + __popcll(m & ((1ull << lane) - 1ull))] = c;
      base += __popcll(m);
    }
    if (lane == 0) s_nlist = base;
  }
  __syncthreads();
  const int nlist = s_nlist;
  const int beg = (int)((long long)split * nlist / p.nsplit);
  const int end = (int)((long long)(split + 1) * nlist / p.nsplit);

  // ---- per-tile state
  const int qq = (lane & 15) >> 3, hh = lane & 7;
  const int h = g * G + hh;
  QFrag<D, NP> qf[TPW];
  f32x4 acc[TPW][D / 16];
  float mrow[TPW], lrow[TPW];
  int ptr[TPW], tq[TPW];
  bool rv[TPW];
  long long iq[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    tq[tt] = tb0 + 2 * (w * TPW + tt) + qq;
    iq[tt] = (long long)p.q0 + tq[tt];
    rv[tt] = tq[tt] < p.nq && hh < G;
    const T* qrow = rv[tt] ? reinterpret_cast<const T*>(p.q) + (((size_t)b * p.Hq + h) * L + slot_of_i(iq[tt])) * D
                           : nullptr;
    load_qfrag<T, D, NP>(qf[tt], qrow, lane);
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) acc[tt][dm] = zero4();
    mrow[tt] = kNegBig;
    lrow[tt] = 0.f;
    ptr[tt] = 0;
    if (tq[tt] < p.nq && beg < end) {
      const int cfirst = list[beg];
      const int* sq = sel + (tq[tt] - tb0) * p.K;
      while (ptr[tt] < p.K && sq[ptr[tt]] >= 0 && sq[ptr[tt]] < cfirst) ++ptr[tt];
    }
  }

  KVStage<T, D, NT> stg;
  if (beg < end) {
    const size_t off = (size_t)list[beg] * kSlots * D;
    stg.load(kg + off, vg + off, tid, 64);
  }
  for (int j = beg; j < end; ++j) {
    bf16_t* buf = kvb + (NBUF == 2 ? (j & 1) : 0) * KVB;
    if (NBUF == 1 && j > beg) __syncthreads();   // single buffer: wait for every reader
    stg.store(buf, tid);
    __syncthreads();
    if (j + 1 < end) {
      const size_t off = (size_t)list[j + 1] * kSlots * D;
      stg.load(kg + off, vg + off, tid, 64);
    }
    const int c = list[j];
    const long long cf = (long long)c * kContent, cl = cf + kContent - 1;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const bool qv = tq[tt] < p.nq;
      const bool win = qv && cf <= iq[tt] + p.R && cl >= iq[tt] - p.R;
      int slot = -1;
      if (qv && ptr[tt] < p.K) {
        if (sel[(tq[tt] - tb0) * p.K + ptr[tt]] == c) {
          slot = ptr[tt];
          ++ptr[tt];
        }
      }
      int mode = win ? 1 : (slot >= 0 ? 2 : 0);
      if (!rv[tt]) mode = 0;
      if (__ballot(mode != 0) == 0ull) continue;

      f32x4 sacc[4];
      s_tile<D, NP>(buf, qf[tt], sacc, lane);

      float x[4][4];
      float mloc = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * mt + 4 * g16 + i;
          bool ok = mode != 0 && key < kContent;
          if (mode == 1) {
            const long long u = cf + key;
            ok = ok && u >= iq[tt] - p.R && u <= iq[tt] + p.R;
          }
          const float xv = ok ? sacc[mt][i] * p.sl2 : -INFINITY;
          x[mt][i] = xv;
          mloc = fmaxf(mloc, xv);
        }
      const float mb = col_max(mloc);
      float zc = 0.f;
      if (mode == 2) zc = p.zsel[(((size_t)b * p.Hq + h) * p.nq + tq[tt]) * p.K + slot] * kLog2e;
      const float m_old = mrow[tt];
      float pbase;
      if (mode == 1) pbase = fmaxf(m_old, mb);
      else if (mode == 2) pbase = mb;
      else pbase = 0.f;
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(x[mt][i] - pbase);
          x[mt][i] = e;
          psum += e;
        }
      const float rs = col_sum(psum);
      float alpha = 1.f;
      if (mode == 1) {
        alpha = fast_exp2(m_old - pbase);
        lrow[tt] = lrow[tt] * alpha + rs;
        mrow[tt] = pbase;
      } else if (mode == 2) {
        const float m_new = fmaxf(m_old, zc);
        alpha = fast_exp2(m_old - m_new);
        const float wz = fast_exp2(zc - m_new);
        const float ws = wz / rs;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[mt][i] *= ws;
        lrow[tt] = lrow[tt] * alpha + wz;
        mrow[tt] = m_new;
      }
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tt][dm][i] *= alpha;
      pv_tile<D, NP>(buf, x, acc[tt], lane);
    }
  }

  // ---- results
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    if (!rv[tt]) continue;
    if (p.nsplit == 1) {
      const float inv = 1.f / lrow[tt];
      T* orow = reinterpret_cast<T*>(p.o) + (((size_t)b * p.Hq + h) * L + slot_of_i(iq[tt])) * D;
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm) {
        float v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = acc[tt][dm][i] * inv;
        store4<T>(orow + 16 * dm + 4 * g16, v4);
      }
      if (p.lse != nullptr && g16 == 0)
        p.lse[((size_t)b * p.Hq + h) * p.nq + tq[tt]] = (mrow[tt] + __log2f(lrow[tt])) * kLn2;
    } else {
      const size_t rows = (size_t)p.B * p.Hq * p.nq;
      float* pp = p.part + ((size_t)split * rows + ((size_t)b * p.Hq + h) * p.nq + tq[tt]) * (D + 4);
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm) {
        float v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = acc[tt][dm][i];
        store4<float>(pp + 16 * dm + 4 * g16, v4);
      }
      if (g16 == 0) {
        pp[D] = mrow[tt];
        pp[D + 1] = lrow[tt];
      }
    }
  }
}

// Merge the split partials of every query row (one wave per row).
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int nsplit, size_t rows,
                                                      void* o, float* lse, int nq, int N, int q0) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + w;
  if (row >= rows) return;
  float M = kNegBig;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part[((size_t)s * rows + row) * (D + 4) + D]);
  float lsum = 0.f, a[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) a[e] = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* pp = part + ((size_t)s * rows + row) * (D + 4);
    const float wgt = fast_exp2(pp[D] - M);
    lsum += pp[D + 1] * wgt;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) a[e] += pp[lane + 64 * e] * wgt;
  }
  const int t = (int)(row % nq);
  const size_t bh = row / nq;
  const long long L = (long long)N * kSlots;
  T* orow = reinterpret_cast<T*>(o) + (bh * L + slot_of_i((long long)q0 + t)) * D;
  const float inv = 1.f / lsum;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) orow[lane + 64 * e] = Elem<T>::from_f(a[e] * inv);
  if (lse != nullptr && lane == 0) lse[row] = (M + __log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------------- sliding-window attention

struct SwaParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, L, R;
  float sl2;
};

constexpr int kSwaTiles = 2;   // 16-slot row tiles per wave (one head per wave)

template <typename T, int D>
__global__ __launch_bounds__(512) void swa_kernel(SwaParams p) {
  constexpr int NP = NPlanes<T>::value;
  constexpr int KVB = kv_buf_elems<D, NP>();
  constexpr int NBUF = kv_nbuf<D, NP>();
  constexpr int QB = 16 * kSwaTiles;
  constexpr int NT = 512;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* kvb = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4;
  const int nthreads = blockDim.x;
  const int G = p.Hq / p.Hkv;
  const int bg = blockIdx.y, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int h = g * G + w;
  const int t0 = blockIdx.x * QB;
  const long long L = p.L;
  const T* kg = reinterpret_cast<const T*>(p.k) + (size_t)bg * L * D;
  const T* vg = reinterpret_cast<const T*>(p.v) + (size_t)bg * L * D;

  QFrag<D, NP> qf[kSwaTiles];
  f32x4 acc[kSwaTiles][D / 16];
  float mrow[kSwaTiles], lrow[kSwaTiles];
  long long trow[kSwaTiles];
#pragma unroll
  for (int tt = 0; tt < kSwaTiles; ++tt) {
    trow[tt] = t0 + 16 * tt + (lane & 15);
    const T* qrow = trow[tt] < L ? reinterpret_cast<const T*>(p.q) + (((size_t)b * p.Hq + h) * L + trow[tt]) * D
                                 : nullptr;
    load_qfrag<T, D, NP>(qf[tt], qrow, lane);
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) acc[tt][dm] = zero4();
    mrow[tt] = kNegBig;
    lrow[tt] = 0.f;
  }

  const long long lo = max(0LL, (long long)t0 - p.R);
  const long long hi = min(L - 1, (long long)t0 + QB - 1 + p.R);
  const long long kb0 = (lo / 64) * 64;
  const int ntile = (int)((hi - kb0) / 64) + 1;

  for (int j = 0; j < ntile; ++j) {
    const long long kb = kb0 + 64LL * j;
    bf16_t* buf = kvb + (NBUF == 2 ? (j & 1) : 0) * KVB;
    if (NBUF == 1 && j > 0) __syncthreads();   // single buffer: wait for every reader
    // Cooperative copy of the 64-slot K/V tile by the block's 64*G threads, in
    // rounds of NT virtual threads. Two buffers alternate, so the barrier at the
    // end of the previous tile is the only one needed before overwriting.
    const int rows_valid = (int)min(64LL, L - kb);
    for (int r0 = 0; r0 < NT; r0 += nthreads) {
      const int vt = r0 + tid;
      if (vt < NT) {
        KVStage<T, D, NT> s1;
        s1.load(kg + (size_t)kb * D, vg + (size_t)kb * D, vt, rows_valid);
        s1.store(buf, vt);
      }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < kSwaTiles; ++tt) {
      const long long ts = t0 + 16 * tt;
      if (kb > ts + 15 + p.R || kb + 63 < ts - p.R || ts >= L) continue;
      f32x4 sacc[4];
      s_tile<D, NP>(buf, qf[tt], sacc, lane);
      float x[4][4];
      float mloc = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long long u = kb + 16 * mt + 4 * g16 + i;
          const bool ok = trow[tt] < L && u < L && u >= trow[tt] - p.R && u <= trow[tt] + p.R;
          const float xv = ok ? sacc[mt][i] * p.sl2 : -INFINITY;
          x[mt][i] = xv;
          mloc = fmaxf(mloc, xv);
        }
      const float mb = col_max(mloc);
      const float m_new = fmaxf(mrow[tt], mb);
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(x[mt][i] - m_new);
          x[mt][i] = e;
          psum += e;
        }
      const float rs = col_sum(psum);
      const float alpha = fast_exp2(mrow[tt] - m_new);
      lrow[tt] = lrow[tt] * alpha + rs;
      mrow[tt] = m_new;
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tt][dm][i] *= alpha;
      pv_tile<D, NP>(buf, x, acc[tt], lane);
    }
  }

#pragma unroll
  for (int tt = 0; tt < kSwaTiles; ++tt) {
    if (trow[tt] >= L) continue;
    const float inv = 1.f / lrow[tt];
    T* orow = reinterpret_cast<T*>(p.o) + (((size_t)b * p.Hq + h) * L + trow[tt]) * D;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      float v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = acc[tt][dm][i] * inv;
      store4<T>(orow + 16 * dm + 4 * g16, v4);
    }
    if (p.lse != nullptr && g16 == 0)
      p.lse[((size_t)b * p.Hq + h) * L + trow[tt]] = (mrow[tt] + __log2f(lrow[tt])) * kLn2;
  }
}

// ---------------------------------------------------------------- host side

static size_t align256a(size_t x) { return (x + 255) & ~(size_t)255; }

// LDS bytes of the K/V staging buffers (all planes, all buffers).
static size_t kv_lds_bytes(int d, int dtype) {
  const int np = dtype == 0 ? 3 : 1;
  const size_t one = (size_t)np * 64 * ((d + 8) + (d + 16)) * 2;
  const int nbuf = (np == 3 && d == 128) ? 1 : 2;
  return nbuf * one;
}

size_t routed_lds_limit() { return 160 * 1024; }

AttnPlan plan_routed_attention(const RouteDims& dm, int K, int nq) {
  AttnPlan pl;
  const size_t kvb = kv_lds_bytes(dm.d, dm.dtype);
  // Prefill-sized problems: 8 waves x 2 tiles = 32 queries per block, no split.
  pl.waves = 8;
  pl.tiles = 2;
  pl.qblock = 2 * pl.waves * pl.tiles;
  pl.nsplit = 1;
  const long long blocks_prefill = (long long)((nq + pl.qblock - 1) / pl.qblock) * dm.B * dm.Hkv;
  if (blocks_prefill < 256) {
    // Decode-sized: one wave per 2-query tile and the chunk list split across blocks.
    pl.waves = 1;
    pl.tiles = 1;
    pl.qblock = 2;
    const long long blocks = (long long)((nq + 1) / 2) * dm.B * dm.Hkv;
    long long ns = (1024 + blocks - 1) / (blocks > 0 ? blocks : 1);
    pl.nsplit = (int)(ns < 1 ? 1 : (ns > 8 ? 8 : ns));
  }
  pl.lds = kvb + (size_t)pl.qblock * K * 4 + (size_t)dm.N * 4 + (size_t)dm.N;
  pl.lds = (pl.lds + 15) & ~(size_t)15;
  pl.ws = pl.nsplit > 1 ? align256a((size_t)pl.nsplit * dm.B * dm.Hq * nq * (dm.d + 4) * 4) : 0;
  return pl;
}

template <typename T, int D, int WAVES, int TPW>
static hipError_t launch_routed_t(const RouteDims& dm, const AttnPlan& pl, const RoutedParams& prm, hipStream_t st) {
  constexpr int QB = 2 * WAVES * TPW;
  auto kern = routed_attention_kernel<T, D, WAVES, TPW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds);
  if (e != hipSuccess) return e;
  dim3 grid((prm.nq + QB - 1) / QB, dm.B * dm.Hkv, pl.nsplit);
  hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), pl.lds, st, prm);
  e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  const size_t rows = (size_t)dm.B * dm.Hq * prm.nq;
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, prm.part,
                     pl.nsplit, rows, prm.o, prm.lse, prm.nq, dm.N, prm.q0);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_routed_d(const RouteDims& dm, const AttnPlan& pl, const RoutedParams& prm, hipStream_t st) {
  if (pl.waves == 8) return launch_routed_t<T, D, 8, 2>(dm, pl, prm, st);
  return launch_routed_t<T, D, 1, 1>(dm, pl, prm, st);
}

hipError_t launch_routed_attention(const RouteDims& dm, const AttnPlan& pl, const void* q, const void* k,
                                   const void* v, const int32_t* idx, const float* zsel, int K, int radius,
                                   float scale, int q0, int nq, void* o, float* lse, void* ws, hipStream_t st) {
  RoutedParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.idx = idx;
  prm.zsel = zsel;
  prm.o = o;
  prm.lse = lse;
  prm.part = reinterpret_cast<float*>(ws);
  prm.B = dm.B;
  prm.Hq = dm.Hq;
  prm.Hkv = dm.Hkv;
  prm.N = dm.N;
  prm.K = K;
  prm.R = radius;
  prm.q0 = q0;
  prm.nq = nq;
  prm.nsplit = pl.nsplit;
  prm.sl2 = scale * kLog2e;
  if (dm.dtype == 1) return dm.d == 64 ? launch_routed_d<bf16_t, 64>(dm, pl, prm, st)
                                       : launch_routed_d<bf16_t, 128>(dm, pl, prm, st);
  return dm.d == 64 ? launch_routed_d<float, 64>(dm, pl, prm, st) : launch_routed_d<float, 128>(dm, pl, prm, st);
}

size_t swa_lds_bytes(int d, int dtype) { return kv_lds_bytes(d, dtype); }

template <typename T, int D>
static hipError_t launch_swa_t(const SwaParams& prm, int G, hipStream_t st) {
  const size_t lds = swa_lds_bytes(D, sizeof(T) == 2 ? 1 : 0);
  auto kern = swa_kernel<T, D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((prm.L + 16 * kSwaTiles - 1) / (16 * kSwaTiles), prm.B * prm.Hkv);
  hipLaunchKernelGGL(kern, grid, dim3(64 * G), lds, st, prm);
  return hipGetLastError();
}

hipError_t launch_swa_attention(int B, int Hq, int Hkv, int L, int d, int dtype, const void* q, const void* k,
                                const void* v, int radius, float scale, void* o, float* lse, hipStream_t st) {
  SwaParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.lse = lse;
  prm.B = B;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.L = L;
  prm.R = radius;
  prm.sl2 = scale * kLog2e;
  const int G = Hq / Hkv;
  if (dtype == 1) return d == 64 ? launch_swa_t<bf16_t, 64>(prm, G, st) : launch_swa_t<bf16_t, 128>(prm, G, st);
  return d == 64 ? launch_swa_t<float, 64>(prm, G, st) : launch_swa_t<float, 128>(prm, G, st);
}

}  // namespace lcr
