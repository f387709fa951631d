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
#include <atomic>
#include <mutex>
#include <type_traits>

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

// ---------------------------------------------------------------- tile layouts in LDS
// Padded layout (register-staged tiles): K rows of D+8 and V rows of D+16
// elements. Swizzled layout (tiles written by direct-to-LDS loads, 1 KB of
// consecutive LDS per wave instruction, so rows cannot be padded): rows of D
// elements whose 16-byte blocks are permuted by an XOR of the row index, chosen
// so that the K fragment reads (16 rows, one block each) and the V transpose
// reads (8 rows, two blocks each, per 32 lanes) hit distinct banks.
template <int D, bool SWZ> struct TileLayout;

template <int D> struct TileLayout<D, false> {
  static constexpr int KE = 64 * (D + 8);
  static constexpr int VE = 64 * (D + 16);
  static constexpr int PL = KE + VE;
  __device__ static __forceinline__ int k_off(int row, int cb) { return row * (D + 8) + cb * 8; }
  __device__ static __forceinline__ int v_off(int row, int col) { return row * (D + 16) + col; }
};

template <int D> struct TileLayout<D, true> {
  static constexpr int KE = 64 * D;
  static constexpr int VE = 64 * D;
  static constexpr int PL = KE + VE;
  __device__ static __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static __forceinline__ int swz_v(int row) { return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3); }
  __device__ static __forceinline__ int k_off(int row, int cb) { return row * D + ((cb ^ swz_k(row)) << 3); }
  __device__ static __forceinline__ int v_off(int row, int col) {
    return row * D + (((col >> 3) ^ swz_v(row)) << 3) + (col & 7);
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
template <int D, int NP, bool SWZ>
__device__ __forceinline__ void s_tile(const bf16_t* buf, const QFrag<D, NP>& q, f32x4 acc[4], int lane) {
  typedef TileLayout<D, SWZ> TL;
  const int L16 = lane & 15, g16 = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int off = TL::k_off(16 * mt + L16, 4 * ks + g16);
      s16x8 a[NP];
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) a[pl] = load8(buf + pl * TL::PL + off);
      acc[mt] = mfma_planes<NP>(a, q.f[ks], acc[mt]);
    }
  }
}

// O^T[d][row] += sum_key V[key][d] p[row][key] with p in the S^T output layout.
// The V^T operand is read with ds_read_b64_tr_b16: lane L of each 16-lane group
// addresses row k0 + L/4, columns 16*dm + 4*(L%4) .. +3, and receives the column
// 16*dm + L over rows k0 .. k0+3.
template <int D, int NP, bool SWZ>
__device__ __forceinline__ void pv_tile(const bf16_t* buf, const float p[4][4], f32x4 o[D / 16], int lane) {
  typedef TileLayout<D, SWZ> TL;
  const int g16 = lane >> 4, L16 = lane & 15;
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
      const int r0 = 32 * ks + 4 * g16 + (L16 >> 2);
      const int col = 16 * dm + 4 * (L16 & 3);
      const int o0 = TL::KE + TL::v_off(r0, col);
      const int o1 = TL::KE + TL::v_off(r0 + 16, col);
      s16x8 a[NP];
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) {
        const s16x4 lo = ds_read_tr(buf + pl * TL::PL + o0);
        const s16x4 hi = ds_read_tr(buf + pl * TL::PL + o1);
        a[pl] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      o[dm] = mfma_planes<NP>(a, pf[ks], o[dm]);
    }
  }
}

// Online-softmax update of one 16-row tile for one chunk (or band tile).
// mode 1: window keys (logits of in-window content keys); mode 2: selected
// chunk (its 63 content keys normalised inside the chunk, then weighted by
// e^{zc}); mode 0: nothing. x holds the raw S^T scores on entry and the
// probabilities to multiply with V on exit; returns the factor that rescales
// the row's accumulator. Window membership of key j: lo <= j <= hi (chunk-local
// key indices, slot 63 excluded by the caller through hi).
__device__ __forceinline__ float tile_update(float x[4][4], int mode, int lo, int hi, float zc, float sl2,
                                             int g16, float& m, float& l) {
  float mloc = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * mt + 4 * g16 + i;
      const bool ok = mode != 0 && key >= lo && key <= hi;
      const float xv = ok ? x[mt][i] * sl2 : -INFINITY;
      x[mt][i] = xv;
      mloc = fmaxf(mloc, xv);
    }
  const float mb = col_max(mloc);
  const float m_old = m;
  const float pbase = mode == 1 ? fmaxf(m_old, mb) : (mode == 2 ? mb : 0.f);
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
    l = l * alpha + rs;
    m = pbase;
  } else if (mode == 2) {
    const float m_new = fmaxf(m_old, zc);
    alpha = fast_exp2(m_old - m_new);
    const float wz = fast_exp2(zc - m_new);
    const float ws = wz / rs;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[mt][i] *= ws;
    l = l * alpha + wz;
    m = m_new;
  }
  return alpha;
}

// Streamlined update for bf16 tiles (one operand plane). Same algebra as
// tile_update with fewer vector instructions per tile:
//  - without window rows in the wave (general = false) only the routing-mask
//    key (chunk slot 63) is masked; rows in mode 0 get P = 0 at the end;
//  - the row maximum is taken on raw scores, then scale and shift are fused
//    into one FMA before exp2;
//  - the running reference m moves only when the new maximum exceeds it by
//    more than 2^8 (values stay below 256 in float32), so the accumulator is
//    usually not rescaled (alpha == 1, the caller skips the multiply);
//  - P is packed with v_cvt_pk_bf16_f32 straight into the PV operand.
// Returns alpha; pf receives the two B-operand fragments of O^T += V^T P^T.
__device__ __forceinline__ float tile_update_bf16(f32x4 sacc[4], bool general, int mode, int lo, int hi, float zc,
                                                  float sl2, int g16, float& m, float& l, s16x8 pf[2]) {
  float mx = -INFINITY;
  if (general) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * mt + 4 * g16 + i;
        const bool ok = key >= lo && key <= hi;
        sacc[mt][i] = ok ? sacc[mt][i] : -INFINITY;
      }
  } else {
    if (g16 == 3) sacc[3][3] = -INFINITY;   // chunk slot 63: the routing mask, never a key
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) mx = fmaxf(mx, fmaxf(fmaxf(sacc[mt][0], sacc[mt][1]), fmaxf(sacc[mt][2], sacc[mt][3])));
  mx = col_max(mx);
  const float mb = mx * sl2;                               // scaled row maximum of this tile
  const float m_old = m;
  const float m_cand = mode == 1 ? fmaxf(m_old, mb) : (mode == 2 ? fmaxf(m_old, zc) : m_old);
  const float m_new = m_cand > m_old + 8.f ? m_cand : m_old;
  const float base = mode == 2 ? mb : (mode == 1 ? m_new : 0.f);
  float e[16];
  float rs = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[4 * mt + i] = fast_exp2(fmaf(sacc[mt][i], sl2, -base));
      rs += e[4 * mt + i];
    }
  rs = col_sum(rs);
  const float alpha = mode == 0 ? 1.f : fast_exp2(m_old - m_new);
  float scale;
  if (mode == 2) {
    const float wz = fast_exp2(zc - m_new);
    l = l * alpha + wz;
    scale = wz / rs;
  } else if (mode == 1) {
    l = l * alpha + rs;
    scale = 1.f;
  } else {
    scale = 0.f;
  }
  m = mode == 0 ? m_old : m_new;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
    u32x4 w;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      // slots j = 2h, 2h+1 of k-step ks: keys of m-tiles 2ks (j < 4) and 2ks+1 (j >= 4)
      const int mt = 2 * ks + (h >> 1), i0 = 2 * (h & 1);
      w[h] = pack2_bf16(e[4 * mt + i0] * scale, e[4 * mt + i0 + 1] * scale);
    }
    pf[ks] = __builtin_bit_cast(s16x8, w);
  }
  return alpha;
}

// O^T += V^T P^T with P already packed (bf16, swizzled V tile).
template <int D>
__device__ __forceinline__ void pv_tile_packed(const bf16_t* buf, const s16x8 pf[2], f32x4 o[D / 16], int lane) {
  typedef TileLayout<D, true> TL;
  const int g16 = lane >> 4, L16 = lane & 15;
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r0 = 32 * ks + 4 * g16 + (L16 >> 2);
      const int col = 16 * dm + 4 * (L16 & 3);
      const s16x4 lo = ds_read_tr(buf + TL::KE + TL::v_off(r0, col));
      const s16x4 hi = ds_read_tr(buf + TL::KE + TL::v_off(r0 + 16, col));
      o[dm] = mfma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf[ks], o[dm]);
    }
  }
}

// ---------------------------------------------------------------- direct-to-LDS chunk loads (bf16)

// One 16-byte-per-lane global_load_lds_dwordx4: lane i's 16 bytes land at LDS
// address m0 + 16*i. Issued from inline asm so that the compiler does not
// order later LDS reads behind it (it cannot tell the ring buffers apart);
// completion is awaited explicitly with wait_vm + a barrier before any wave
// reads the buffer. The asm has no output registers.
__device__ __forceinline__ void dma16(const void* gsrc, const bf16_t* lds_dst) {
  const uint32_t la = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(la)
               : "memory", "m0");
}

// 64 rows x D of K and of V (16 KB each at D = 128) land in the swizzled layout;
// each wave instruction moves 1 KB (64 lanes x 16 bytes). The 2 * D / 8
// instructions of a chunk (K first, then V) are dealt round-robin to the
// waves: wave w issues 2 * D / (8 * WAVES) of them.
template <int D, int WAVES>
__device__ __forceinline__ void dma_chunk(const bf16_t* kc, const bf16_t* vc, bf16_t* buf, int w, int lane) {
  typedef TileLayout<D, true> TL;
  constexpr int NI = D / 8;              // 1 KB instructions per tile
  constexpr int RPI = 512 / D;           // rows per instruction
  constexpr int BPR = D / 8;             // 16-byte blocks per row
  static_assert((2 * NI) % WAVES == 0, "instructions must divide evenly among waves");
#pragma unroll
  for (int jj = w; jj < 2 * NI; jj += WAVES) {
    const bool is_v = jj >= NI;
    const int ii = is_v ? jj - NI : jj;
    const int pr = ii * RPI + lane / BPR, pb = lane % BPR;
    if (!is_v) dma16(kc + pr * D + ((pb ^ TL::swz_k(pr)) << 3), buf + ii * 512);
    else dma16(vc + pr * D + ((pb ^ TL::swz_v(pr)) << 3), buf + TL::KE + ii * 512);
  }
}

// Compiler-only fence: keeps LDS accesses on their side of a raw barrier or flag.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Bounded wait until an LDS counter reaches target (wave-uniform). Returns false
// after `limit` polls (by default 2^22, a fraction of a second), so a logic error
// cannot hang the GPU. A wave whose wait gives up stops its walk and writes NaN to
// every output row it owns, so an incomplete result cannot pass for a valid one.
__device__ __forceinline__ bool spin_until_ge(int* ctr, int target, int limit) {
  for (int it = 0; it < limit; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
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
  int nent, epb;  // decode-sized plan: entries per 2-query tile, entries per block
  int spin;       // polls before a wait on an LDS counter gives up (>= 1)
  int rev;        // tiles in reversed order (results do not depend on it)
  int qb;         // pooled prefill kernel: queries per block (at most its compile-time count)
  float sl2;      // scale * log2(e)
};

// Chunk-staging policy: bf16 inputs go straight from HBM into LDS (swizzled
// layout, NBUF-deep ring, prefetch distance NBUF-1, one barrier per chunk);
// float32 inputs are split into three bf16 planes on the way, so they are
// staged through registers into the padded layout (double buffered when it
// fits).
template <typename T, int D> struct RoutedCfg {
  static constexpr int NP = NPlanes<T>::value;
  static constexpr bool SWZ = NP == 1;
  static constexpr int PLE = TileLayout<D, SWZ>::PL;           // elements per plane
  static constexpr int BUFE = NP * PLE;                         // elements per chunk buffer
};

template <typename T, int D, int WAVES, int TPW, int NBUF>
__global__ __launch_bounds__(WAVES * 64) void routed_attention_kernel(RoutedParams p) {
  typedef RoutedCfg<T, D> C;
  constexpr int NP = C::NP;
  constexpr bool SWZ = C::SWZ;
  constexpr int NT = WAVES * 64;
  constexpr int QB = 2 * WAVES * TPW;
  constexpr int PD = NBUF - 1;                                  // prefetch distance (DMA path)
  constexpr int NINST = 2 * (D / 8) / WAVES;                     // DMA instructions per wave per chunk
  static_assert(!SWZ || PD * NINST < 64, "in-flight loads must fit the vmcnt counter");
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* kvb = reinterpret_cast<bf16_t*>(smem);
  int* sel = reinterpret_cast<int*>(smem + (size_t)NBUF * C::BUFE * sizeof(bf16_t));
  float* zs = reinterpret_cast<float*>(sel + QB * p.K);          // [QB][G][K] chunk logits
  const int G = p.Hq / p.Hkv;
  int* list = reinterpret_cast<int*>(zs + QB * G * p.K);
  unsigned char* flags = reinterpret_cast<unsigned char*>(list + p.N);
  __shared__ int s_nlist;
  __shared__ int ctl_arr[NBUF];    // per ring slot: wave shares landed (monotonic)
  __shared__ int ctl_done[NBUF];   // per ring slot: waves finished with it (monotonic)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4;
  const int bg = blockIdx.y, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int tb0 = blockIdx.x * QB;
  if (tid < NBUF) {
    ctl_arr[tid] = 0;
    ctl_done[tid] = 0;
  }
  const int split = blockIdx.z;
  const long long L = (long long)p.N * kSlots;
  const long long Tcont = (long long)p.N * kContent;
  const T* kg = reinterpret_cast<const T*>(p.k) + (size_t)bg * L * D;
  const T* vg = reinterpret_cast<const T*>(p.v) + (size_t)bg * L * D;

  // ---- the ascending union of chunks needed by this block's queries, their
  //      selections and chunk logits (no global loads remain in the chunk loop)
  for (int c = tid; c < p.N; c += NT) flags[c] = 0;
  __syncthreads();
  for (int e = tid; e < QB * p.K; e += NT) {
    const int qi = e / p.K, kk = e - qi * p.K, t = tb0 + qi;
    int c = (t < p.nq) ? p.idx[((size_t)bg * p.nq + t) * p.K + kk] : -1;
    if (c >= p.N) c = -1;
    sel[e] = c;
    if (c >= 0) flags[c] = 1;
  }
  for (int e = tid; e < QB * G * p.K; e += NT) {
    const int qi = e / (G * p.K), rem = e - qi * G * p.K, hh2 = rem / p.K, kk = rem - hh2 * p.K;
    const int t = tb0 + qi;
    zs[e] = (t < p.nq) ? p.zsel[(((size_t)b * p.Hq + g * G + hh2) * p.nq + t) * p.K + kk] : 0.f;
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

  // ---- chunk loop
  // bf16 (SWZ): no block barrier. Every wave issues its share of each chunk's
  // direct-to-LDS loads PD positions ahead, publishes its share once its own
  // loads have landed (ctl_arr[slot] += 1), waits for all WAVES shares only when
  // it has work on that chunk, and reports the slot free afterwards
  // (ctl_done[slot] += 1). A slot is refilled only when every wave is done with
  // the chunk it held; PD <= NBUF - 1 keeps this free of deadlock. Every wait is
  // bounded: a wave that times out stops (its outputs are then wrong, but every
  // wave of the block still terminates).
  // float32 (register-staged planes): one block barrier per chunk.
  KVStage<T, D, NT> stg;
  bool failed = false;
  if constexpr (SWZ) {
    // Every earlier vector-memory load (query fragments, selections) completes
    // here, so the only ones in flight inside the loop are this wave's chunk
    // loads, which the loop waits for itself.
    wait_vm<0>();
#pragma unroll
    for (int jj = 0; jj < PD; ++jj)
      if (beg + jj < end) {
        const size_t off = (size_t)list[beg + jj] * kSlots * D;
        dma_chunk<D, WAVES>(reinterpret_cast<const bf16_t*>(kg + off), reinterpret_cast<const bf16_t*>(vg + off),
                            kvb + (jj % NBUF) * C::BUFE, w, lane);
      }
  } else {
    if (beg < end) {
      const size_t off = (size_t)list[beg] * kSlots * D;
      stg.load(kg + off, vg + off, tid, 64);
    }
  }
  for (int j = beg; j < end && !failed; ++j) {
    const int pos = j - beg;
    const int slot_buf = pos % NBUF;
    bf16_t* buf = kvb + slot_buf * C::BUFE;
    if constexpr (SWZ) {
      // (1) this wave's share of position pos + PD
      if (j + PD < end) {
        const int p2 = pos + PD, s2 = p2 % NBUF, use2 = p2 / NBUF;
        if (use2 > 0 && !spin_until_ge(&ctl_done[s2], WAVES * use2, p.spin)) {
          failed = true;
          break;
        }
        compiler_fence();
        const size_t off = (size_t)list[j + PD] * kSlots * D;
        dma_chunk<D, WAVES>(reinterpret_cast<const bf16_t*>(kg + off), reinterpret_cast<const bf16_t*>(vg + off),
                            kvb + s2 * C::BUFE, w, lane);
      }
      // (2) publish this wave's share of position pos once it has landed
      const int ahead = min(PD, end - 1 - j);   // positions issued after pos
      if (ahead >= 2) wait_vm<(PD >= 2 ? 2 * NINST : 0)>();
      else if (ahead == 1) wait_vm<NINST>();
      else wait_vm<0>();
      compiler_fence();
      if (lane == 0) __hip_atomic_fetch_add(&ctl_arr[slot_buf], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      if (NBUF == 1 && j > beg) __syncthreads();   // single buffer: wait for every reader
      stg.store(buf, tid);
      __syncthreads();
      if (j + 1 < end) {
        const size_t off = (size_t)list[j + 1] * kSlots * D;
        stg.load(kg + off, vg + off, tid, 64);
      }
    }
    const int c = list[j];
    const long long cf = (long long)c * kContent, cl = cf + kContent - 1;
    int mode[TPW], slot[TPW];
    bool any = false;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const bool qv = tq[tt] < p.nq;
      const bool win = qv && cf <= iq[tt] + p.R && cl >= iq[tt] - p.R;
      slot[tt] = -1;
      if (qv && ptr[tt] < p.K) {
        if (sel[(tq[tt] - tb0) * p.K + ptr[tt]] == c) {
          slot[tt] = ptr[tt];
          ++ptr[tt];
        }
      }
      mode[tt] = win ? 1 : (slot[tt] >= 0 ? 2 : 0);
      if (!rv[tt]) mode[tt] = 0;
      any = any || (__ballot(mode[tt] != 0) != 0ull);
    }
    if (any) {
      if constexpr (SWZ) {
        if (!spin_until_ge(&ctl_arr[slot_buf], WAVES * (pos / NBUF + 1), p.spin)) {
          failed = true;
          break;
        }
        compiler_fence();
      }
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        if (__ballot(mode[tt] != 0) == 0ull) continue;
        f32x4 sacc[4];
        s_tile<D, NP, SWZ>(buf, qf[tt], sacc, lane);
        if constexpr (NP == 1) {
          const bool general = __ballot(mode[tt] == 1) != 0ull;
          int lo = 0, hi = kContent - 1;
          if (mode[tt] == 1) {
            lo = (int)max(0LL, iq[tt] - p.R - cf);
            hi = (int)min((long long)kContent - 1, iq[tt] + p.R - cf);
          }
          const float zc = mode[tt] == 2 ? zs[((tq[tt] - tb0) * G + hh) * p.K + slot[tt]] * kLog2e : 0.f;
          s16x8 pf[2];
          const float alpha = tile_update_bf16(sacc, general, mode[tt], lo, hi, zc, p.sl2, g16, mrow[tt], lrow[tt], pf);
          if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
            for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[tt][dm][i] *= alpha;
          }
          pv_tile_packed<D>(buf, pf, acc[tt], lane);
          continue;
        }
        float x[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[mt][i] = sacc[mt][i];
        int lo = 0, hi = kContent - 1;
        if (mode[tt] == 1) {
          lo = (int)max(0LL, iq[tt] - p.R - cf);
          hi = (int)min((long long)kContent - 1, iq[tt] + p.R - cf);
        }
        float zc = 0.f;
        if (mode[tt] == 2) zc = zs[((tq[tt] - tb0) * G + hh) * p.K + slot[tt]] * kLog2e;
        const float alpha = tile_update(x, mode[tt], lo, hi, zc, p.sl2, g16, mrow[tt], lrow[tt]);
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tt][dm][i] *= alpha;
        pv_tile<D, NP, SWZ>(buf, x, acc[tt], lane);
      }
    }
    if constexpr (SWZ) {
      // every LDS read of this slot by this wave has returned (their values fed the MFMAs)
      wait_lgkm0();
      compiler_fence();
      if (lane == 0) __hip_atomic_fetch_add(&ctl_done[slot_buf], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  if constexpr (SWZ) wait_vm<0>();   // no load of this wave outlives the block

  // ---- results (NaN rows when this wave's walk was cut short by a wait that gave up)
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    if (!rv[tt]) continue;
    if (failed) {
      mrow[tt] = __builtin_nanf("");
      lrow[tt] = __builtin_nanf("");
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm) acc[tt][dm] = f32x4{mrow[tt], mrow[tt], mrow[tt], mrow[tt]};
    }
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

// ---------------------------------------------------------------- routed attention, prefill (bf16)
//
// Same tiles and algebra as routed_attention_kernel, with the work of a block
// split between one producer wave and kCons consumer waves so that no wave
// waits for another one's progress except through a pool of chunk halves:
//  - setup (all waves): the list of chunks the block's queries need (the window
//    range first, then the rest ascending), per list position a mask of the
//    block's queries active on it (window or selected), built with LDS atomics.
//  - producer: walks the list in order and moves the K and then the V of each
//    chunk into free entries of an NH-entry pool with direct-to-LDS loads (an
//    entry is free once its count of consumers still reading it is zero); it
//    publishes the entry of each half and the number of landed halves.
//  - consumer w (one 16-row tile: 2 queries x 8 head rows): visits only the
//    positions where one of its queries is active (found from the masks with
//    ballots, 64 positions at a time), forms S = K Q^T once the K half has
//    landed and releases that entry, then P V once V has landed and releases
//    V's entry. A consumer that is behind holds only the entries of positions
//    it still needs, and K is free again long before V. The chunk logit of a
//    lane's next selected chunk is loaded from zsel one visit ahead, so LDS
//    holds only the pool and the position tables.
// Chunks in the block's window range take the masked softmax only where some
// lane's window covers part of the chunk; every other visit takes the lean one.



// Softmax update of a bf16 tile (see tile_update_bf16); WINDOW selects at
// compile time whether per-key window bounds are applied.
template <bool WINDOW, bool MASK63 = true>
__device__ __forceinline__ float tile_softmax(f32x4 sacc[4], int mode, int lo, int hi, float zc, float sl2, int g16,
                                              float& m, float& l, s16x8 pf[2]) {
  if constexpr (WINDOW) {
    // key 16 mt + 4 g16 + i is kept when lo <= key <= hi: the constant 16 mt + i is
    // compared with bounds shifted by the lane's 4 g16 (no per-key registers)
    const int los = lo - 4 * g16, his = hi - 4 * g16;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[mt][i] = (16 * mt + i >= los && 16 * mt + i <= his) ? sacc[mt][i] : -INFINITY;
  } else if constexpr (MASK63) {
    if (g16 == 3) sacc[3][3] = -INFINITY;   // chunk slot 63: the routing mask, never a key
  }
  float mx = max3(sacc[0][0], sacc[0][1], max2(sacc[0][2], sacc[0][3]));
#pragma unroll
  for (int mt = 1; mt < 4; ++mt) mx = max3(mx, max3(sacc[mt][0], sacc[mt][1], sacc[mt][2]), sacc[mt][3]);
  mx = col_max(mx);
  const float mb = mx * sl2;
  const float m_old = m;
  const float m_cand = mode == 1 ? max2(m_old, mb) : (mode == 2 ? max2(m_old, zc) : m_old);
  const float m_new = m_cand > m_old + 8.f ? m_cand : m_old;
  const float base = mode == 2 ? mb : (mode == 1 ? m_new : 0.f);
  float rs = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sacc[mt][i] = fast_exp2(fmaf(sacc[mt][i], sl2, -base));   // in place: no second set of registers
      rs += sacc[mt][i];
    }
  rs = col_sum(rs);
  const float alpha = mode == 0 ? 1.f : fast_exp2(m_old - m_new);
  float scale;
  if (mode == 2) {
    const float wz = fast_exp2(zc - m_new);
    l = l * alpha + wz;
    scale = wz * __builtin_amdgcn_rcpf(rs);
  } else {
    l = mode == 1 ? l * alpha + rs : l;
    scale = mode == 1 ? 1.f : 0.f;
  }
  m = mode == 0 ? m_old : m_new;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
    u32x4 wv;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int mt = 2 * ks + (h >> 1), i0 = 2 * (h & 1);
      wv[h] = pack2_bf16(sacc[mt][i0] * scale, sacc[mt][i0 + 1] * scale);
    }
    pf[ks] = __builtin_bit_cast(s16x8, wv);
  }
  return alpha;
}

// The lean softmax of a remote visit on which only one query of the tile is active:
// the lanes of half ACT (lane % 16 / 8 == ACT) hold its head columns, the other half
// the idle query's. The lane pair (l, l ^ 8) of a 16-lane row shares the active
// column's 16 scores of that row group: the active lane keeps those of m-tiles 0 and
// 1, its partner takes those of m-tiles 2 and 3 through a DPP rotation by 8, so each
// lane exponentiates 8 scores instead of 16. Per score the arithmetic is that of
// tile_softmax in mode 2 (valid active lanes); the idle query keeps its state and
// gets P = 0.
template <int ACT>
__device__ __forceinline__ float tile_softmax_half(f32x4 sacc[4], bool valid, float zc, float sl2, int g16, int lane,
                                                   float& m, float& l, s16x8 pf[2]) {
  constexpr int kIdle = ACT == 0 ? 0xC : 0x3;   // DPP bank mask of the idle half (4 lanes per bank)
  constexpr int kAct = ACT == 0 ? 0x3 : 0xC;
  constexpr int kRor8 = 0x128;                   // row_ror:8
  // row_shl:8 (lane l reads l + 8) or row_shr:8 (l - 8): the active lane reads its partner,
  // the idle lane reads past its row and gets 0 (bound_ctrl)
  constexpr int kToAct = ACT == 0 ? 0x108 : 0x118;
  const bool act = ((lane >> 3) & 1) == ACT;
  if (g16 == 3) sacc[3][3] = -INFINITY;   // chunk slot 63: the routing mask, never a key
  float x[8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
    x[r] = __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp((int)__float_as_uint(sacc[r >> 2][r & 3]),
                                                                 (int)__float_as_uint(sacc[2 + (r >> 2)][r & 3]),
                                                                 kRor8, 0xF, kIdle, false));
  float mx = max3(x[0], x[1], max3(x[2], x[3], max3(x[4], x[5], max2(x[6], x[7]))));
  mx = max2(mx, __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(mx), kRor8, 0xF, 0xF, false)));
  mx = col_max(mx);
  const float mb = mx * sl2;
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    x[r] = fast_exp2(fmaf(x[r], sl2, -mb));
    rs += x[r];
  }
  rs += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(rs), kRor8, 0xF, 0xF, true));
  rs = col_sum(rs);
  const bool on = valid && act;
  const float m_old = m;
  const float m_cand = on ? max2(m_old, zc) : m_old;
  const float m_new = m_cand > m_old + 8.f ? m_cand : m_old;
  const float alpha = fast_exp2(m_old - m_new);
  const float wz = fast_exp2(zc - m_new);
  float scale = on ? wz * __builtin_amdgcn_rcpf(rs) : 0.f;
  l = on ? l * alpha + wz : l;
  m = m_new;
  // the partner lanes scale the active column's scores with its factor
  scale = __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp((int)__float_as_uint(scale), (int)__float_as_uint(scale),
                                                                kRor8, 0xF, kIdle, false));
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  u32x4 p0, p1;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t wv = pack2_bf16(x[2 * h] * scale, x[2 * h + 1] * scale);
    // m-tiles 0, 1: the active lane's own words; 2, 3: its partner's, rotated back
    p1[h] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wv, kToAct, 0xF, 0xF, true);
    p0[h] = act ? wv : 0u;
  }
  pf[0] = __builtin_bit_cast(s16x8, p0);
  pf[1] = __builtin_bit_cast(s16x8, p1);
  return alpha;
}

// S^T for NT tiles sharing every K fragment read.
template <int D, int NT>
__device__ __forceinline__ void s_tiles(const bf16_t* buf, const QFrag<D, 1>* q, f32x4 (*acc)[4], int lane) {
  typedef TileLayout<D, true> TL;
  const int L16 = lane & 15, g16 = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const s16x8 a = load8(buf + TL::k_off(16 * mt + L16, 4 * ks + g16));
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][mt] = mfma16(a, q[t].f[ks][0], acc[t][mt]);
    }
  }
}

// O^T += V^T P^T for NT tiles sharing every V^T fragment read (vbuf: a V half).
// The swizzle XORs an even key into the 16-byte block index, so the offset of
// rows r0 + 32 ks + 16 u and columns col + 16 dm is the unswizzled offset of
// (r0, col) plus (32 ks + 16 u) D plus 16 (dm ^ key): one XOR per column block,
// the rest immediate offsets. The lane index is formed here by an asm mbcnt that
// the compiler cannot merge with another, so that it derives the lane constants
// and the eight column offsets in place instead of keeping them live across the
// chunk loop, where registers are short.
template <int D, int NT>
__device__ __forceinline__ void pv_tiles(const bf16_t* vbuf, const s16x8 (*pf)[2], f32x4 (*o)[D / 16]) {
  typedef TileLayout<D, true> TL;
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const int r0 = ln >> 2;   // 4 (l / 16) + (l % 16) / 4
  const int lb0 = r0 * D + 4 * (ln & 3);
  const int key16 = 8 * TL::swz_v(r0);
  const bf16_t* base = vbuf + lb0;
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) {
    const bf16_t* bd = base + (key16 ^ (16 * dm));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const s16x4 lo = ds_read_tr(bd + 32 * ks * D);
      const s16x4 hi = ds_read_tr(bd + (32 * ks + 16) * D);
      const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t][dm] = mfma16(a, pf[t][ks], o[t][dm]);
    }
  }
}

// S^T and O^T += V^T P^T on LDS byte addresses, for the pooled prefill kernel (one
// tile) and the SWA kernel (NT tiles sharing every fragment read). A K or V half
// starts at a multiple of 8 KB (the pool or ring is the first thing in the block's
// LDS, and neither kernel declares static LDS), so the row swizzle and the fragment's
// k-step (S) or column block (P V) combine by one XOR of the 16-byte block bits:
// klane = row (l % 16) in bytes + ((l / 16) ^ that row's K swizzle) * 16, and vlane =
// the V^T fragment's byte offset of pv_tiles with its swizzle key; both are formed
// once per wave. The m-tiles and k-halves are immediate offsets.
typedef __attribute__((address_space(3))) const s16x8 lds_cs16x8;
__device__ __forceinline__ s16x8 lds_load8_at(uint32_t a) { return *(lds_cs16x8*)(size_t)a; }
__device__ __forceinline__ s16x4 lds_read_tr_at(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)a);
}
template <int D>
__device__ __forceinline__ void s_tile_x(uint32_t ebase, const QFrag<D, 1>& q, f32x4 acc[4], uint32_t klane) {
  const uint32_t a0 = ebase + klane;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = zero4();
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const uint32_t ak = a0 ^ (uint32_t)(ks << 6);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma16(lds_load8_at(ak + 16 * mt * D * 2), q.f[ks][0], acc[mt]);
  }
}
template <int D>
__device__ __forceinline__ void pv_tile_x(uint32_t ebase, const s16x8* pf, f32x4* o, uint32_t vlane) {
  const uint32_t a0 = ebase + vlane;
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) {
    const uint32_t ad = a0 ^ (uint32_t)(dm << 5);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const s16x4 lo = lds_read_tr_at(ad + 32 * ks * D * 2);
      const s16x4 hi = lds_read_tr_at(ad + (32 * ks + 16) * D * 2);
      o[dm] = mfma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf[ks], o[dm]);
    }
  }
}

template <int D, int NT>
__device__ __forceinline__ void s_tiles_x_acc(uint32_t ebase, const QFrag<D, 1>* q, f32x4 (*acc)[4], uint32_t klane) {
  const uint32_t a0 = ebase + klane;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const uint32_t ak = a0 ^ (uint32_t)(ks << 6);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const s16x8 a = lds_load8_at(ak + 16 * mt * D * 2);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][mt] = mfma16(a, q[t].f[ks][0], acc[t][mt]);
    }
  }
}
template <int D, int NT>
__device__ __forceinline__ void s_tiles_x(uint32_t ebase, const QFrag<D, 1>* q, f32x4 (*acc)[4], uint32_t klane) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[t][mt] = zero4();
  s_tiles_x_acc<D, NT>(ebase, q, acc, klane);
}
template <int D, int NT>
__device__ __forceinline__ void pv_tiles_x(uint32_t ebase, const s16x8 (*pf)[2], f32x4 (*o)[D / 16], uint32_t vlane) {
  const uint32_t a0 = ebase + vlane;
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) {
    const uint32_t ad = a0 ^ (uint32_t)(dm << 5);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const s16x4 lo = lds_read_tr_at(ad + 32 * ks * D * 2);
      const s16x4 hi = lds_read_tr_at(ad + (32 * ks + 16) * D * 2);
      const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int t = 0; t < NT; ++t) o[t][dm] = mfma16(a, pf[t][ks], o[t][dm]);
    }
  }
}

// One half (K or V) of a chunk, NI = D / 8 direct-to-LDS instructions of 1 KB,
// with the global address split into a uniform 64-bit base
// (SGPRs) and per-lane 32-bit offsets that depend only on the lane and on the
// instruction's position in a group of four (the swizzle repeats every 16 rows,
// one group spans 4 KB). voff[u] is precomputed once; per instruction only M0
// changes. No output registers: completion is awaited with wait_vm.
template <int D>
__device__ __forceinline__ int dma_voff(bool is_v, int u, int lane) {
  typedef TileLayout<D, true> TL;
  constexpr int RPI = 512 / D, BPR = D / 8;
  const int pr = u * RPI + lane / BPR, pb = lane % BPR;
  const int sw = is_v ? TL::swz_v(pr) : TL::swz_k(pr);
  return pr * D * 2 + ((pb ^ sw) << 4);
}

template <int D>
__device__ __forceinline__ void dma_half_fast(const bf16_t* src, uint32_t lds, const int* voff) {
  constexpr int NI = D / 8;
  static_assert(NI % 4 == 0, "groups of four instructions");
#pragma unroll
  for (int g = 0; g < NI / 4; ++g) {
    const bf16_t* sg = src + g * 2048;   // 4 KB per group
#pragma unroll
    for (int u = 0; u < 4; ++u)
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds + (4 * g + u) * 1024),
                   "v"(voff[u]), "s"(sg)
                   : "memory", "m0");
  }
}

__device__ __forceinline__ void lds_store_rel(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_load_rel(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Shape of the pooled prefill kernel: TPW 16-column tiles (2 queries x 8 head rows
// each) per consumer wave. One tile: 15 consumers under 128 VGPRs (16 waves, four per
// SIMD). Two tiles: 11 consumers under 168 VGPRs (12 waves, three per SIMD), 44
// queries per block, so each chunk the block loads serves more queries.
template <int TPW> struct PfCfg;
template <> struct PfCfg<1> {
  static constexpr int kProd = 1;
  static constexpr int kCons = 15;
  typedef unsigned Mask;
};
template <> struct PfCfg<2> {
  static constexpr int kProd = 1;
  static constexpr int kCons = 11;
  typedef unsigned long long Mask;
};
template <int TPW> constexpr int pf_waves() { return PfCfg<TPW>::kCons + PfCfg<TPW>::kProd; }
template <int TPW> constexpr int pf_qblock() { return 2 * TPW * PfCfg<TPW>::kCons; }

template <int D, int NH, int TPW>
__global__ __launch_bounds__(64 * pf_waves<TPW>()) void routed_prefill_kernel(RoutedParams p) {
  typedef TileLayout<D, true> TL;
  typedef typename PfCfg<TPW>::Mask MaskT;
  static_assert(TL::KE == TL::VE, "K and V halves share one pool");
  constexpr int kCons = PfCfg<TPW>::kCons;
  constexpr int kProd = PfCfg<TPW>::kProd;   // producer waves: producer r loads positions j = r (mod kProd)
  constexpr int kWaves = kCons + kProd;
  constexpr int NHP = NH / kProd;             // pool entries of each producer
  static_assert(NH % kProd == 0, "the pool splits evenly among the producers");
  constexpr int QB = pf_qblock<TPW>();        // queries per block
  constexpr int WB = 2 * TPW;                 // mask bits (queries) per consumer wave
  static_assert(QB <= 8 * (int)sizeof(MaskT), "one mask bit per query of the block");
  constexpr int HE = TL::KE;                   // elements per half (the K or the V of a chunk)
  constexpr int NI = D / 8;                    // DMA instructions per half
  constexpr int HF = (63 / NI) < NH ? (63 / NI) : NH;   // halves in flight
  static_assert(HF >= 2 && (HF - 1) * NI < 64, "in-flight loads must fit the vmcnt counter");
  static_assert(NH >= 2 && NH <= 32, "half pool size");
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = p.Hq / p.Hkv;
  bf16_t* kvb = reinterpret_cast<bf16_t*>(smem);
  MaskT* pos_mask = reinterpret_cast<MaskT*>(smem + (size_t)NH * HE * sizeof(bf16_t));   // [N]
  int* pos_chunk = reinterpret_cast<int*>(pos_mask + p.N);                              // [N]
  short* pos_of = reinterpret_cast<short*>(pos_chunk + p.N);                             // [N]
  // after setup, the same bytes hold per position the pool entries of its K (byte 2j) and V (2j + 1)
  unsigned char* pos_half = reinterpret_cast<unsigned char*>(pos_of);
  // the block's counters follow the tables (no static LDS: the pool starts at LDS address 0)
  int* tail = reinterpret_cast<int*>(smem + (((size_t)NH * HE * sizeof(bf16_t) +
                                                (size_t)p.N * (sizeof(MaskT) + 4 + 2) + 15) & ~(size_t)15));
  int& s_n = tail[0];
  int& s_fail = tail[1];
  // halves landed per producer: position j is producer j % kProd's (j / kProd)-th, its K the
  // producer's half 2 (j / kProd), its V half 2 (j / kProd) + 1
  int* s_landed = tail + 2;
  int* s_rem = tail + 2 + kProd;   // consumers still to finish the half held by a pool entry

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4;
  const int qb = p.qb;                         // this launch's queries per block (<= QB)
  const int nqb = (p.nq + qb - 1) / qb;
  const int tile = xcd_tile(nqb * p.B * p.Hkv, p.rev);   // (batch-head, query block), batch-head major
  if (tile < 0) return;
  const int bg = tile / nqb, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int tb0 = (tile - bg * nqb) * qb;
  const int qend = min(tb0 + qb, p.nq);        // the block's queries are tb0 .. qend - 1
  const long long L = (long long)p.N * kSlots;
  const long long Tcont = (long long)p.N * kContent;
  const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.k) + (size_t)bg * L * D;
  const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.v) + (size_t)bg * L * D;
  constexpr int NT = 64 * kWaves;

  // ---- setup: chunk list and per-position query masks
  if (tid == 0) s_fail = 0;
  if (tid < kProd) s_landed[tid] = 0;
  if (tid < NH) s_rem[tid] = 0;
  for (int c = tid; c < p.N; c += NT) pos_of[c] = 0;
  __syncthreads();
  const int t_last = qend - 1;
  // the block's window range: chunks in the window of any of its queries
  const int cw0 = (int)(max(0LL, (long long)p.q0 + tb0 - p.R) / kContent);
  const int cw1 = (int)(min(Tcont - 1, (long long)p.q0 + t_last + p.R) / kContent);
  for (int c = cw0 + tid; c <= cw1; c += NT) pos_of[c] = 1;
  for (int e = tid; e < QB * p.K; e += NT) {
    const int qi = e / p.K, kk = e - qi * p.K, t = tb0 + qi;
    const int c = (t < qend) ? p.idx[((size_t)bg * p.nq + t) * p.K + kk] : -1;
    if (c >= 0 && c < p.N) pos_of[c] = 1;
  }
  __syncthreads();
  if (w == 0) {
    // list order: ascending, so that concurrently running blocks walk the remote chunks
    // in step and share them in L2, and each query meets its selected chunks in the
    // order of its zsel row
    int base = 0;
    for (int c0 = 0; c0 < p.N; c0 += 64) {
      const int c = c0 + lane;
      const bool f = c < p.N && pos_of[c] != 0;
      const unsigned long long m = __ballot(f);
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (f) {
        pos_chunk[pos] = c;
        pos_mask[pos] = MaskT(0);
        pos_of[c] = (short)pos;
      }
      base += __popcll(m);
    }
    if (lane == 0) s_n = base;
  }
  __syncthreads();
  const int n = s_n;
  for (int e = tid; e < QB * p.K; e += NT) {
    const int qi = e / p.K, kk = e - qi * p.K, t = tb0 + qi;
    const int c = (t < qend) ? p.idx[((size_t)bg * p.nq + t) * p.K + kk] : -1;
    if (c >= 0 && c < p.N) atomicOr(&pos_mask[pos_of[c]], MaskT(1) << qi);
  }
  for (int qi = w; qi < QB; qi += kWaves) {
    const int t = tb0 + qi;
    if (t >= qend) continue;
    const long long i = (long long)p.q0 + t;
    const int c0 = (int)(max(0LL, i - p.R) / kContent), c1 = (int)(min(Tcont - 1, i + p.R) / kContent);
    for (int c = c0 + lane; c <= c1; c += 64) atomicOr(&pos_mask[pos_of[c]], MaskT(1) << qi);
  }
  __syncthreads();

  if (w >= kCons) {
    // ---------------- producer r = w - kCons: positions j = r, r + kProd, ... into its own
    // NHP entries of the pool (several producers keep more loads in flight than one
    // wave's vmcnt allows)
    // Its instructions go ahead of the consumers' on the shared SIMD: the whole block
    // runs at the pace of its loads, so their issue must not wait behind softmax work.
    __builtin_amdgcn_s_setprio(3);
    const int r = __builtin_amdgcn_readfirstlane(w - kCons);   // wave-uniform: entry numbers stay scalar
    const int e0 = r * NHP;
    int* landed = &s_landed[r];
    int told = 0;   // landed halves already published (monotonic)
    bool ok = true;
    int voffk[4], voffv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      voffk[u] = dma_voff<D>(false, u, lane);
      voffv[u] = dma_voff<D>(true, u, lane);
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)kvb);
    constexpr int HFP = HF < NHP ? HF : NHP;   // this producer's halves in flight
    // publish the halves below hh2 - HFP + 1 once at most HFP - 1 of this wave's loads are in flight
    auto publish_landed = [&](int hh2) {
      if (hh2 >= HFP && hh2 - HFP + 1 > told) {
        wait_vm<(HFP - 1) * NI>();
        compiler_fence();
        if (lane == 0) lds_store_rel(landed, hh2 - HFP + 1);
        told = hh2 - HFP + 1;
      }
    };
    // Any free entry of its own takes the next half. Entries seen free stay known (only
    // this wave fills them), so the counts are read again only when none is known free.
    // Before waiting for one, everything issued is awaited and published, so that the
    // consumers that hold the pool can finish. Returns -1 when the wait gives up or
    // another wave has failed.
    const unsigned mine_all = ((1u << NHP) - 1u) << e0;
    unsigned known_free = mine_all;
    auto free_entries = [&]() -> unsigned {
      const bool own = lane >= e0 && lane < e0 + NHP;
      return (unsigned)__ballot(own && lds_load_rel(&s_rem[own ? lane : e0]) == 0);
    };
    auto acquire = [&](int hx) -> int {
      if (known_free == 0u) {
        known_free = free_entries();
        if (known_free == 0u) {
          wait_vm<0>();
          compiler_fence();
          if (lane == 0) lds_store_rel(landed, hx);
          told = hx;
          int it = 0;
          for (; it < p.spin && known_free == 0u; ++it) {
            __builtin_amdgcn_s_sleep(1);
            known_free = free_entries();
          }
          if (known_free == 0u || lds_load_rel(&s_fail) != 0) return -1;
        }
      }
      const int e = __builtin_ctz(known_free);
      known_free &= known_free - 1u;
      return e;
    };
    // Chunks and consumer counts of 64 positions are read lane-parallel up front.
    int hl = 0;   // this producer's halves issued so far
    for (int base = 0; base < n && ok; base += 64) {
      const int pj = base + lane < n ? base + lane : n - 1;
      const int pcl = pos_chunk[pj];
      const MaskT pml = pos_mask[pj];
      int ul = 0;
#pragma unroll
      for (int cw = 0; cw < kCons; ++cw) ul += ((pml >> (WB * cw)) & ((MaskT(1) << WB) - 1)) != 0 ? 1 : 0;
      const int cnt = min(64, n - base);
      for (int jj = (r - base % kProd + kProd) % kProd; jj < cnt; jj += kProd) {
        const int hk = 2 * (base + jj);
        const int users = __builtin_amdgcn_readlane(ul, jj);
        const size_t off = (size_t)__builtin_amdgcn_readlane(pcl, jj) * kSlots * D;
        // K, then V, each into an entry of its own: K is released once its users have
        // formed S, well before they are done with V
        const int ek = acquire(hl);
        if (ek < 0) {
          ok = false;
          break;
        }
        if (lane == 0) {   // both written before the landed count covers the half
          lds_store_rel(&s_rem[ek], users);
          pos_half[hk] = (unsigned char)ek;
        }
        compiler_fence();
        publish_landed(hl);
        dma_half_fast<D>(kg + off, lds0 + (uint32_t)(ek * HE * 2), voffk);
        ++hl;
        const int ev = acquire(hl);
        if (ev < 0) {
          ok = false;
          break;
        }
        if (lane == 0) {
          lds_store_rel(&s_rem[ev], users);
          pos_half[hk + 1] = (unsigned char)ev;
        }
        compiler_fence();
        publish_landed(hl);
        dma_half_fast<D>(vg + off, lds0 + (uint32_t)(ev * HE * 2), voffv);
        ++hl;
      }
    }
    wait_vm<0>();
    compiler_fence();
    if (lane == 0) {
      if (ok) lds_store_rel(landed, hl);
      else lds_store_rel(&s_fail, 1);
    }
    return;
  }

  // ---------------- consumer w: queries WB w .. WB w + WB - 1 of the block; tile t holds
  // queries WB w + 2 t and WB w + 2 t + 1 (lane column: query qq of the tile, head hh)
  const int qq = (lane & 15) >> 3, hh = lane & 7;
  const int h = g * G + hh;
  const int R32 = (int)min((long long)p.R, Tcont);   // a wider radius selects the same keys
  // lane byte offsets of the K and V fragment reads within a pool entry, formed once
  const uint32_t klane = (uint32_t)((lane & 15) * D * 2 + ((g16 ^ TL::swz_k(lane & 15)) << 4));
  const uint32_t vlane = (uint32_t)(((lane >> 2) * D + 4 * (lane & 3) + 8 * TL::swz_v(lane >> 2)) * 2);
  const uint32_t kvb0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)kvb;
  QFrag<D, 1> qf[TPW];
  f32x4 acc[TPW][D / 16];
  float mrow[TPW], lrow[TPW], znext[TPW];
  int ptr[TPW];
  bool rv[TPW];
  // zsel row of this lane's query in tile 0; tile t's row is zoff0 + 2 K t (a lane whose
  // tile-t query is past nq never advances, so only its first read needs the clamp below)
  int zoff0 = 0;
  const int iq0 = p.q0 + tb0 + WB * w + qq;    // tile t's query is iq0 + 2 t (content indices fit in 32 bits)
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tq = iq0 + 2 * t - p.q0;
    rv[t] = tq < qend && hh < G;
    load_qfrag<bf16_t, D, 1>(qf[t], rv[t] ? reinterpret_cast<const bf16_t*>(p.q) +
                                                (((size_t)b * p.Hq + h) * L + slot_of_i(iq0 + 2 * t)) * D
                                          : nullptr, lane);
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) acc[t][dm] = zero4();
    mrow[t] = kNegBig;
    lrow[t] = 0.f;
    ptr[t] = 0;
    // the chunk logits of this lane's row stay in HBM / L2: the one for the next selected
    // chunk (the list is ascending, as is each zsel row) is loaded a visit ahead; rows
    // past the block's queries or heads read a valid row
    const int zo = (int)((((size_t)b * p.Hq + (hh < G ? h : g * G)) * p.nq + (tq < p.nq ? tq : p.nq - 1)) * p.K);
    if (t == 0) zoff0 = zo;
    znext[t] = p.K > 0 ? p.zsel[zo] : 0.f;
  }
  // landed halves of each producer known to this wave: a count is read again only when it
  // falls short. Half hv (0: K, 1: V) of position j is producer j % kProd's half
  // 2 (j / kProd) + hv.
  int seen[kProd];
#pragma unroll
  for (int r = 0; r < kProd; ++r) seen[r] = 0;
  auto await = [&](int j, int hv) -> bool {
    const int r = j % kProd, need = 2 * (j / kProd) + hv + 1;
    int it = 0;
    int sr = 0;
#pragma unroll
    for (int x = 0; x < kProd; ++x) sr = x == r ? seen[x] : sr;
    while (sr < need) {
      sr = lds_load_rel(&s_landed[r]);
      if (sr >= need) break;
      if (++it >= p.spin || lds_load_rel(&s_fail) != 0) return false;
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int x = 0; x < kProd; ++x) seen[x] = x == r ? sr : seen[x];
    compiler_fence();
    return true;
  };
  // every LDS read of entry e has returned: release it
  auto release = [&](int e) {
    wait_lgkm0();
    compiler_fence();
    if (lane == 0) __hip_atomic_fetch_add(&s_rem[e], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  bool failed = false;
  for (int base = 0; base < n && !failed; base += 64) {
    const int pl = base + lane < n ? base + lane : n - 1;
    const unsigned wbl = base + lane < n ? (unsigned)((pos_mask[pl] >> (WB * w)) & ((MaskT(1) << WB) - 1)) : 0u;
    const int pc = pos_chunk[pl];
    unsigned long long mine = __ballot(wbl != 0u);
    while (mine != 0ull) {
      const int bit = __builtin_ctzll(mine);
      mine &= mine - 1ull;
      const int j = base + bit;
      const int c = __builtin_amdgcn_readlane(pc, bit);
      const unsigned wb = (unsigned)__builtin_amdgcn_readlane((int)wbl, bit);   // this wave's queries on c
      const bool inr = c >= cw0 && c <= cw1;     // inside the block's window range (uniform)
      const int last = (TPW == 2 && (wb & 12u) != 0u) ? 1 : 0;   // last active tile (uniform)
      if (!await(j, 0)) {
        failed = true;
        break;
      }
      const int ek = pos_half[2 * j];   // written by the producer before the landed count covered it
      int ev = -1;
      // tile by tile: S, softmax, then P V, so that only one tile's P is live; K is released
      // after the last tile's S, V after its P V
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const unsigned tb = (wb >> (2 * t)) & 3u;
        if (tb == 0u) continue;                  // uniform: neither query of the tile uses c
        // per lane: window keys (mode 1), selected chunk (2) or nothing (0); a window lane
        // whose window covers only part of the chunk needs per-key bounds (partial)
        const bool qa = ((tb >> qq) & 1u) != 0u;
        bool win = false;
        int lo = 0, hi = kContent - 1;
        if (inr) {
          const int rel = iq0 + 2 * t - c * kContent;   // query index relative to the chunk's first key
          win = rel + R32 >= 0 && rel - R32 <= kContent - 1;
          if (win && qa && rv[t]) {
            lo = max(0, rel - R32);
            hi = min(kContent - 1, rel + R32);
          }
        }
        const int mode = (!qa || !rv[t]) ? 0 : (win ? 1 : 2);
        const bool partial = inr && __ballot(lo > 0 || hi < kContent - 1) != 0ull;
        const float zc = znext[t] * kLog2e;
        if (qa && !win) {
          ++ptr[t];
          znext[t] = p.zsel[zoff0 + 2 * p.K * t + min(ptr[t], p.K - 1)];   // lands while this chunk is processed
        }
        f32x4 sacc[4];
        s_tile_x<D>(kvb0 + (uint32_t)(ek * HE * 2), qf[t], sacc, klane);
        if (t == last) release(ek);
        s16x8 pf[2];
        float alpha;
        if (!inr && tb != 3u) {   // uniform: a remote chunk that one query of the tile selected
          alpha = tb == 1u ? tile_softmax_half<0>(sacc, rv[t], zc, p.sl2, g16, lane, mrow[t], lrow[t], pf)
                           : tile_softmax_half<1>(sacc, rv[t], zc, p.sl2, g16, lane, mrow[t], lrow[t], pf);
        } else {
          alpha = partial ? tile_softmax<true>(sacc, mode, lo, hi, zc, p.sl2, g16, mrow[t], lrow[t], pf)
                          : tile_softmax<false>(sacc, mode, lo, hi, zc, p.sl2, g16, mrow[t], lrow[t], pf);
        }
        if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
          for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][dm][i] *= alpha;
        }
        if (ev < 0) {
          if (!await(j, 1)) {
            failed = true;
            break;
          }
          ev = pos_half[2 * j + 1];
        }
        pv_tile_x<D>(kvb0 + (uint32_t)(ev * HE * 2), pf, acc[t], vlane);
        if (t == last) release(ev);
      }
      if (failed) break;
    }
  }
  if (failed && lane == 0) lds_store_rel(&s_fail, 1);

  // ---- results (NaN rows when this wave's walk was cut short by a wait that gave up)
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (failed) {
      mrow[t] = __builtin_nanf("");
      lrow[t] = mrow[t];
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm) acc[t][dm] = f32x4{mrow[t], mrow[t], mrow[t], mrow[t]};
    }
    if (rv[t]) {
      const float inv = 1.f / lrow[t];
      bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (((size_t)b * p.Hq + h) * L + slot_of_i(iq0 + 2 * t)) * D;
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm) {
        float v4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = acc[t][dm][i] * inv;
        store4<bf16_t>(orow + 16 * dm + 4 * g16, v4);
      }
      if (p.lse != nullptr && g16 == 0)
        p.lse[((size_t)b * p.Hq + h) * p.nq + (iq0 + 2 * t - p.q0)] = (mrow[t] + __log2f(lrow[t])) * kLn2;
    }
  }
}

// ---------------------------------------------------------------- routed attention backward, query side
// The forward's producer / consumer pool with a backward consumer: the block's 14
// queries (7 consumer waves, one 16-column tile each) share one ascending stream of
// the chunks any of them needs, so each chunk's K and V are fetched once per block.
// Per visit a consumer forms S^T = K Q^T and dP^T = V dO^T, the intra-chunk softmax
// statistics, ds, and dQ^T += K^T dS^T (K^T by transposing reads of the K half, which
// it holds until then). It writes dq, dzsel, D = dO . o and, per (row, selected chunk),
// the probability bias and U_c that the key-side kernel needs.
constexpr int kBqCons = 11;
constexpr int kBqWaves = kBqCons + 1;
constexpr int kBqQB = 2 * kBqCons;

struct BwdQueryParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const int32_t* idx;
  const float* zsel;
  const float* lse;
  float* dq;
  float* dzsel;
  float* dsum;
  float* cbias;
  float* cu;
  int B, Hq, Hkv, N, K, R, q0, nq;
  int spin;       // polls before a wait on an LDS counter gives up (>= 1)
  int rev;        // tiles in reversed order (results do not depend on it)
  float scale;
};

template <int D, int NH>
__global__ __launch_bounds__(64 * kBqWaves) void bwd_query_pool_kernel(BwdQueryParams p) {
  typedef TileLayout<D, true> TL;
  static_assert(TL::KE == TL::VE, "K and V halves share one pool");
  constexpr int HE = TL::KE;                   // elements per half (the K or the V of a chunk)
  constexpr int NI = D / 8;                    // DMA instructions per half
  constexpr int HF = (63 / NI) < NH ? (63 / NI) : NH;   // halves in flight
  static_assert(HF >= 2 && (HF - 1) * NI < 64, "in-flight loads must fit the vmcnt counter");
  static_assert(NH >= 2 && NH <= 32, "half pool size");
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = p.Hq / p.Hkv;
  bf16_t* kvb = reinterpret_cast<bf16_t*>(smem);
  int* pos_chunk = reinterpret_cast<int*>(smem + (size_t)NH * HE * sizeof(bf16_t));   // [N]
  unsigned* pos_mask = reinterpret_cast<unsigned*>(pos_chunk + p.N);                  // [N]
  short* pos_of = reinterpret_cast<short*>(pos_mask + p.N);                           // [N]
  // after setup, the same bytes hold per position the pool entries of its K (byte 2j) and V (2j + 1)
  unsigned char* pos_half = reinterpret_cast<unsigned char*>(pos_of);
  __shared__ int s_n;
  __shared__ int s_landed;           // halves landed: K of position j is half 2j, V half 2j + 1
  __shared__ int s_rem[NH];          // consumers still to finish the half held by a pool entry
  __shared__ int s_fail;
  __shared__ int s_nlo[kBqQB];       // per query: selected chunks below the block's window range
  __shared__ int s_nin[kBqQB];       // ... and inside it

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g16 = lane >> 4;
  const int nqb = (p.nq + kBqQB - 1) / kBqQB;
  const int tile = xcd_tile(nqb * p.B * p.Hkv, p.rev);   // (batch-head, query block), batch-head major
  if (tile < 0) return;
  const int bg = tile / nqb, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int tb0 = (tile - bg * nqb) * kBqQB;
  const long long L = (long long)p.N * kSlots;
  const long long Tcont = (long long)p.N * kContent;
  const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.k) + (size_t)bg * L * D;
  const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.v) + (size_t)bg * L * D;
  constexpr int NT = 64 * kBqWaves;

  // ---- setup: chunk list and per-position query masks
  if (tid == 0) {
    s_landed = 0;
    s_fail = 0;
  }
  if (tid < NH) s_rem[tid] = 0;
  if (tid < kBqQB) {
    s_nlo[tid] = 0;
    s_nin[tid] = 0;
  }
  for (int c = tid; c < p.N; c += NT) pos_of[c] = 0;
  __syncthreads();
  const int t_last = min(tb0 + kBqQB, p.nq) - 1;
  // the block's window range: chunks in the window of any of its queries
  const int cw0 = (int)(max(0LL, (long long)p.q0 + tb0 - p.R) / kContent);
  const int cw1 = (int)(min(Tcont - 1, (long long)p.q0 + t_last + p.R) / kContent);
  for (int c = cw0 + tid; c <= cw1; c += NT) pos_of[c] = 1;
  for (int e = tid; e < kBqQB * p.K; e += NT) {
    const int qi = e / p.K, kk = e - qi * p.K, t = tb0 + qi;
    const int c = (t < p.nq) ? p.idx[((size_t)bg * p.nq + t) * p.K + kk] : -1;
    if (c >= 0 && c < p.N) {
      pos_of[c] = 1;
      if (c < cw0) atomicAdd(&s_nlo[qi], 1);
      else if (c <= cw1) atomicAdd(&s_nin[qi], 1);
    }
  }
  __syncthreads();
  if (w == 0) {
    // list order: the window range first (every block's heavy positions up front), then
    // the other chunks ascending, so that concurrently running blocks walk the remote
    // chunks in step and share them in L2
    int base = 0;
    auto append = [&](int c, bool f) {
      const unsigned long long m = __ballot(f);
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (f) {
        pos_chunk[pos] = c;
        pos_mask[pos] = 0u;
        pos_of[c] = (short)pos;
      }
      base += __popcll(m);
    };
    for (int c0 = cw0; c0 <= cw1; c0 += 64) {
      const int c = c0 + lane;
      append(c, c <= cw1 && pos_of[c] != 0);
    }
    for (int c0 = 0; c0 < p.N; c0 += 64) {
      const int c = c0 + lane;
      append(c, c < p.N && (c < cw0 || c > cw1) && pos_of[c] != 0);
    }
    if (lane == 0) s_n = base;
  }
  __syncthreads();
  const int n = s_n;
  for (int e = tid; e < kBqQB * p.K; e += NT) {
    const int qi = e / p.K, kk = e - qi * p.K, t = tb0 + qi;
    const int c = (t < p.nq) ? p.idx[((size_t)bg * p.nq + t) * p.K + kk] : -1;
    if (c >= 0 && c < p.N) atomicOr(&pos_mask[pos_of[c]], 1u << qi);
  }
  for (int qi = w; qi < kBqQB; qi += kBqWaves) {
    const int t = tb0 + qi;
    if (t >= p.nq) continue;
    const long long i = (long long)p.q0 + t;
    const int c0 = (int)(max(0LL, i - p.R) / kContent), c1 = (int)(min(Tcont - 1, i + p.R) / kContent);
    for (int c = c0 + lane; c <= c1; c += 64) atomicOr(&pos_mask[pos_of[c]], 1u << qi);
  }
  __syncthreads();

  if (w == kBqCons) {
    // ---------------- producer
    // Its instructions go ahead of the consumers' on the shared SIMD: the whole block
    // runs at the pace of its loads, so their issue must not wait behind softmax work.
    __builtin_amdgcn_s_setprio(3);
    int told = 0;   // landed halves already published (monotonic)
    bool ok = true;
    int voffk[4], voffv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      voffk[u] = dma_voff<D>(false, u, lane);
      voffv[u] = dma_voff<D>(true, u, lane);
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)kvb);
    // publish the halves below hh2 - HF + 1 once at most HF - 1 of this wave's loads are in flight
    auto publish_landed = [&](int hh2) {
      if (hh2 >= HF && hh2 - HF + 1 > told) {
        wait_vm<(HF - 1) * NI>();
        compiler_fence();
        if (lane == 0) lds_store_rel(&s_landed, hh2 - HF + 1);
        told = hh2 - HF + 1;
      }
    };
    // Any free entry takes the next half. Entries seen free stay known (only this wave
    // fills them), so the counts are read again only when none is known free. Before
    // waiting for one, everything issued is awaited and published, so that the
    // consumers that hold the pool can finish. Returns -1 when the wait gives up or
    // another wave has failed.
    unsigned known_free = NH == 32 ? ~0u : (1u << NH) - 1u;
    auto acquire = [&](int hx) -> int {
      if (known_free == 0u) {
        known_free = (unsigned)__ballot(lane < NH && lds_load_rel(&s_rem[lane < NH ? lane : 0]) == 0);
        if (known_free == 0u) {
          wait_vm<0>();
          compiler_fence();
          if (lane == 0) lds_store_rel(&s_landed, hx);
          told = hx;
          int it = 0;
          for (; it < p.spin && known_free == 0u; ++it) {
            __builtin_amdgcn_s_sleep(1);
            known_free = (unsigned)__ballot(lane < NH && lds_load_rel(&s_rem[lane < NH ? lane : 0]) == 0);
          }
          if (known_free == 0u || lds_load_rel(&s_fail) != 0) return -1;
        }
      }
      const int e = __builtin_ctz(known_free);
      known_free &= known_free - 1u;
      return e;
    };
    // Chunks and consumer counts of 64 positions are read lane-parallel up front.
    for (int base = 0; base < n && ok; base += 64) {
      const int pj = base + lane < n ? base + lane : n - 1;
      const int pcl = pos_chunk[pj];
      const unsigned pml = pos_mask[pj];
      int ul = 0;
#pragma unroll
      for (int cw = 0; cw < kBqCons; ++cw) ul += ((pml >> (2 * cw)) & 3u) != 0u ? 1 : 0;
      const int cnt = min(64, n - base);
      for (int jj = 0; jj < cnt; ++jj) {
        const int hk = 2 * (base + jj);
        const int users = __builtin_amdgcn_readlane(ul, jj);
        const size_t off = (size_t)__builtin_amdgcn_readlane(pcl, jj) * kSlots * D;
        // K, then V, each into an entry of its own: K is released once its users have
        // formed S, well before they are done with V
        const int ek = acquire(hk);
        if (ek < 0) {
          ok = false;
          break;
        }
        if (lane == 0) {   // both written before the landed count covers the half
          lds_store_rel(&s_rem[ek], users);
          pos_half[hk] = (unsigned char)ek;
        }
        compiler_fence();
        publish_landed(hk);
        dma_half_fast<D>(kg + off, lds0 + (uint32_t)(ek * HE * 2), voffk);
        const int ev = acquire(hk + 1);
        if (ev < 0) {
          ok = false;
          break;
        }
        if (lane == 0) {
          lds_store_rel(&s_rem[ev], users);
          pos_half[hk + 1] = (unsigned char)ev;
        }
        compiler_fence();
        publish_landed(hk + 1);
        dma_half_fast<D>(vg + off, lds0 + (uint32_t)(ev * HE * 2), voffv);
      }
    }
    wait_vm<0>();
    compiler_fence();
    if (lane == 0) {
      if (ok) lds_store_rel(&s_landed, 2 * n);
      else lds_store_rel(&s_fail, 1);
    }
    return;
  }

  // ---------------- consumer w: queries 2w and 2w + 1 of the block, one 16-row tile
  const int qq = (lane & 15) >> 3, hh = lane & 7, L16 = lane & 15;
  const int h = g * G + (hh < G ? hh : 0);
  const int qb = 2 * w + qq;                 // this lane's query in the block
  const int tq = tb0 + qb;
  const int iq = p.q0 + (tq < p.nq ? tq : p.nq - 1);
  const bool rv = tq < p.nq && hh < G;
  const int R32 = (int)min((long long)p.R, Tcont);
  const size_t row = (((size_t)b * p.Hq + h) * L + slot_of_i(iq)) * D;
  const size_t rq = ((size_t)b * p.Hq + h) * p.nq + (tq < p.nq ? tq : p.nq - 1);
  // per-row offsets into zsel, dzsel, cbias and cu as 32-bit indices (fewer live registers
  // than 64-bit row pointers; the host checks that B*Hq*nq*K fits)
  const int rqk = (int)(rq * (size_t)p.K);
  // B operands of this lane's column: q and dO (d = 32 ks + 8 g16 + j); D = dO . o
  s16x8 qf2[D / 32], dof[D / 32];
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    if (rv) {
      qf2[ks] = load8(reinterpret_cast<const bf16_t*>(p.q) + row + 32 * ks + 8 * g16);
      dof[ks] = load8(reinterpret_cast<const bf16_t*>(p.dO) + row + 32 * ks + 8 * g16);
      const s16x8 of = load8(reinterpret_cast<const bf16_t*>(p.o) + row + 32 * ks + 8 * g16);
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += bf2f((bf16_t)dof[ks][j]) * bf2f((bf16_t)of[j]);
    } else {
      qf2[ks] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
      dof[ks] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  QFrag<D, 1> qf;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qf.f[ks][0] = qf2[ks];
  dsum = col_sum(dsum);
  const float lse = rv ? p.lse[rq] : 0.f;
  if (rv && g16 == 0) {
    p.dsum[rq] = dsum;
    for (int kk = 0; kk < p.K; ++kk) p.dzsel[rqk + kk] = 0.f;
  }
  const float sl2 = p.scale * kLog2e;   // the only live copy of the scale: dQ is scaled by sl2 * ln 2
  f32x4 dqa[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) dqa[dm] = zero4();
  int ptr = 0;   // selected chunks of this lane's query visited so far
  const int nlo = s_nlo[qb], nin = s_nin[qb];

  // the v-th selected chunk visited: the list walks the window range, then the chunks
  // below it, then those above, each ascending, while zsel is ascending
  auto zsel_slot = [&](int v) {
    const int ks = v < nin ? nlo + v : (v < nin + nlo ? v - nin : v);
    return ks < p.K ? ks : p.K - 1;
  };
  float znext = p.K > 0 ? p.zsel[rqk + zsel_slot(0)] : 0.f;
  int seen = 0;
  auto await = [&](int need) -> bool {
    int it = 0;
    while (seen < need) {
      seen = lds_load_rel(&s_landed);
      if (seen >= need) break;
      if (++it >= p.spin || lds_load_rel(&s_fail) != 0) return false;
      __builtin_amdgcn_s_sleep(1);
    }
    compiler_fence();
    return true;
  };
  auto release = [&](int e) {
    wait_lgkm0();
    compiler_fence();
    if (lane == 0) __hip_atomic_fetch_add(&s_rem[e], -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  typedef TileLayout<D, true> TL;
  bool failed = false;
  for (int base = 0; base < n && !failed; base += 64) {
    const int pl = base + lane < n ? base + lane : n - 1;
    const unsigned pm = base + lane < n ? pos_mask[pl] : 0u;
    const int pc = pos_chunk[pl];
    unsigned long long mine = __ballot(((pm >> (2 * w)) & 3u) != 0u);
    while (mine != 0ull) {
      const int bit = __builtin_ctzll(mine);
      mine &= mine - 1ull;
      const int j = base + bit;
      const int c = __builtin_amdgcn_readlane(pc, bit);
      const unsigned bits = (unsigned)__builtin_amdgcn_readlane((int)pm, bit) >> (2 * w);
      const bool qa = ((bits >> qq) & 1u) != 0u;
      const int rel = iq - c * kContent;
      const bool win = rel + R32 >= 0 && rel - R32 <= kContent - 1;
      const int mode = (!qa || !rv) ? 0 : (win ? 1 : 2);
      const int lo = mode == 1 ? max(0, rel - R32) : 0;
      const int hi = mode == 1 ? min(kContent - 1, rel + R32) : (mode == 2 ? kContent - 1 : -1);
      int slot = 0;
      float z = 0.f;
      if (qa && !win) {
        slot = zsel_slot(ptr);
        z = znext;
        ++ptr;
        znext = p.zsel[rqk + zsel_slot(ptr)];
      }
      if (!await(2 * j + 1)) {
        failed = true;
        break;
      }
      const int ek = pos_half[2 * j];
      const bf16_t* kb = kvb + ek * HE;
      f32x4 sacc[1][4];
      s_tiles<D, 1>(kb, &qf, sacc, lane);
      if (!await(2 * j + 2)) {
        failed = true;
        break;
      }
      const int ev = pos_half[2 * j + 1];
      const bf16_t* vb = kvb + ev * HE;
      // dP^T = V dO^T: V rows (swizzled V layout) as the A operand
      f32x4 pacc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        pacc[mt] = zero4();
        const int vr = 16 * mt + L16;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          pacc[mt] = mfma16(load8(vb + vr * D + (((4 * ks + g16) ^ TL::swz_v(vr)) << 3)), dof[ks], pacc[mt]);
      }
      release(ev);
      // intra-chunk softmax statistics of every column (used where the chunk is selected)
      // in base-2 units: every exponent below is one FMA and one exp2
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * mt + 4 * g16 + e < kContent) mx = fmaxf(mx, sl2 * sacc[0][mt][e]);
      mx = col_max(mx);
      float l = 0.f, tu = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 16 * mt + 4 * g16 + e;
          const float ex = jj < kContent ? fast_exp2(fmaf(sacc[0][mt][e], sl2, -mx)) : 0.f;
          l += ex;
          tu += ex * pacc[mt][e];
        }
      l = col_sum(l);
      tu = col_sum(tu);
      const float U = tu / l;
      // The weight of a key is exp2(s sl2 - b): b = lse log2 e inside the window; for a
      // selected chunk b = mx + log2 l - (z - lse) log2 e = -cbias log2 e folds the chunk
      // weight exp(z - lse) and the intra-chunk normalisation into the exponent.
      float b = lse * kLog2e, sub = dsum;
      if (mode == 2) {
        const float lc = mx + fast_log2(l);
        b = lc - (z - lse) * kLog2e;
        sub = U;
        if (g16 == 0) {
          p.dzsel[rqk + slot] = __expf(z - lse) * (U - dsum);
          p.cbias[rqk + slot] = (z - lse) - lc * kLn2;
          p.cu[rqk + slot] = U;
        }
      }
      float ds[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 16 * mt + 4 * g16 + e;
          ds[mt][e] = (jj >= lo && jj <= hi) ? fast_exp2(fmaf(sacc[0][mt][e], sl2, -b)) * (pacc[mt][e] - sub) : 0.f;
        }
      s16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pf[ks] = pack8_bf16(ds[2 * ks], ds[2 * ks + 1]);
      // dQ^T += K^T dS^T: K^T read transposed from the swizzled K half. Rows r0 + 32 ks + 16 u
      // share the swizzle of r0 (period 16), so each column block is one XOR per lane.
      {
        const int r0 = lane >> 2;
        const int sw = TL::swz_k(r0);
        const int ab = (lane & 3) >> 1, b4 = 4 * (lane & 1);
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm) {
          const int off = (((2 * dm + ab) ^ sw) << 3) + b4;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const s16x4 lo4 = ds_read_tr(kb + (r0 + 32 * ks) * D + off);
            const s16x4 hi4 = ds_read_tr(kb + (r0 + 32 * ks + 16) * D + off);
            dqa[dm] = mfma16(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), pf[ks], dqa[dm]);
          }
        }
      }
      release(ek);
    }
  }
  if (failed && lane == 0) lds_store_rel(&s_fail, 1);

  // ---- results (NaN rows when this wave's walk was cut short by a wait that gave up)
  if (failed) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) dqa[dm] = f32x4{nan, nan, nan, nan};
    if (rv && g16 == 0)
      for (int kk = 0; kk < p.K; ++kk) p.dzsel[rqk + kk] = nan;
  }
  if (rv) {
    float* dqr = p.dq + row;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) *reinterpret_cast<f32x4*>(dqr + 16 * dm + 4 * g16) = dqa[dm] * (sl2 * kLn2);
  }
}

// Merge the split partials of every query row (one wave per row). Partial s of
// a row holds (O, m, l) at part[(s * rows + row) * (D + 4)]; a partial with
// l = 0 saw no key of the row and its O is not read (it may not be written).
constexpr int kCombineRegs = 4;                       // up to 64 * 4 partials per row
constexpr int kMaxPartials = 64 * kCombineRegs;

template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, int nsplit, size_t rows,
                                                      void* o, float* lse, int nq, int N, int q0) {
  constexpr int DE = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + w;
  if (row >= rows) return;
  const size_t rs = rows * (D + 4);                   // stride between partials
  const float* pr = part + row * (D + 4);
  float mv[kCombineRegs], lv[kCombineRegs], wv[kCombineRegs];
  float M = kNegBig;
#pragma unroll
  for (int j = 0; j < kCombineRegs; ++j) {
    const int s = lane + 64 * j;
    const int sc = s < nsplit ? s : nsplit - 1;          // in bounds: loads need no branch
    const float m_s = pr[(size_t)sc * rs + D], l_s = pr[(size_t)sc * rs + D + 1];
    mv[j] = s < nsplit ? m_s : kNegBig;
    lv[j] = s < nsplit ? l_s : 0.f;
    if (lv[j] > 0.f) M = fmaxf(M, mv[j]);
  }
  M = wave_max(M);
  float lsum = 0.f;
  unsigned long long act[kCombineRegs];
#pragma unroll
  for (int j = 0; j < kCombineRegs; ++j) {
    wv[j] = lv[j] > 0.f ? fast_exp2(mv[j] - M) : 0.f;
    lsum += lv[j] * wv[j];
    act[j] = __ballot(lv[j] > 0.f);
  }
  lsum = wave_sum(lsum);
  float a[DE];
#pragma unroll
  for (int e = 0; e < DE; ++e) a[e] = 0.f;
#pragma unroll
  for (int j = 0; j < kCombineRegs; ++j) {
    unsigned long long m = act[j];
    while (m != 0ull) {
      // up to 8 active partials at once (their loads are in flight together);
      // unused slots repeat the first one with weight 0
      int sl[8];
      float ww[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (m != 0ull) {
          const int bit = __builtin_ctzll(m);
          m &= m - 1ull;
          sl[u] = 64 * j + bit;
          ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv[j]), bit));
        } else {
          sl[u] = sl[0];
          ww[u] = 0.f;
        }
      }
      float v[8][DE];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < DE; ++e) v[u][e] = pr[(size_t)sl[u] * rs + lane + 64 * e];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < DE; ++e) a[e] += v[u][e] * ww[u];
    }
  }
  const int t = (int)(row % nq);
  const size_t bh = row / nq;
  const long long L = (long long)N * kSlots;
  T* orow = reinterpret_cast<T*>(o) + (bh * L + slot_of_i((long long)q0 + t)) * D;
  const float inv = 1.f / lsum;
#pragma unroll
  for (int e = 0; e < DE; ++e) orow[lane + 64 * e] = Elem<T>::from_f(a[e] * inv);
  if (lse != nullptr && lane == 0) lse[row] = (M + __log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------------- routed attention, decode-sized problems
//
// Few queries: the work of a 2-query tile is a list of entries. Entries 0..K-1
// are the first query's selected chunks, K..2K-1 the second query's, and 2K..
// the chunks of the tile's window range. A chunk that occurs in more than one
// place is handled once: a selected chunk inside the window range belongs to
// its window entry, and a chunk chosen by both queries belongs to the first
// query's entry. The list is cut into runs of p.epb entries, one single-wave
// block per (tile, run). A block walks the chunks of its run (bf16: the next
// chunk is loaded into the second LDS buffer while the current one is
// multiplied), keeps the online-softmax state of both queries across them and
// writes one unnormalised partial (O, m, l) per row; combine_kernel merges the
// runs of a row.
template <typename T, int D>
__global__ __launch_bounds__(64) void routed_decode_kernel(RoutedParams p) {
  typedef RoutedCfg<T, D> C;
  constexpr int NP = C::NP;
  constexpr bool SWZ = C::SWZ;
  constexpr int NI2 = 2 * (D / 8);   // direct-to-LDS loads per chunk (bf16)
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* bufs = reinterpret_cast<bf16_t*>(smem);
  const int G = p.Hq / p.Hkv;
  float* zs = reinterpret_cast<float*>(smem + (size_t)(SWZ ? 2 : 1) * C::BUFE * sizeof(bf16_t));   // [2][G][K]
  const int lane = threadIdx.x, g16 = lane >> 4;
  const int bg = blockIdx.y, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int tb0 = 2 * blockIdx.x;
  const long long L = (long long)p.N * kSlots;
  const long long Tcont = (long long)p.N * kContent;

  // selections of the two queries: lane k holds entry k
  int s0 = -1, s1 = -1;
  if (p.K > 0) {   // uniform; idx may be NULL when K = 0
    const int kl = lane < p.K ? lane : p.K - 1, t1 = tb0 + 1 < p.nq ? tb0 + 1 : tb0;
    s0 = p.idx[((size_t)bg * p.nq + tb0) * p.K + kl];        // in bounds for every lane: no branch
    s1 = p.idx[((size_t)bg * p.nq + t1) * p.K + kl];
    if (lane >= p.K || s0 >= p.N) s0 = -1;
    if (lane >= p.K || tb0 + 1 >= p.nq || s1 >= p.N) s1 = -1;
  }
  const int t_last = min(tb0 + 2, p.nq) - 1;
  const long long i_first = (long long)p.q0 + tb0, i_last = (long long)p.q0 + t_last;
  const int cw0 = (int)(max(0LL, i_first - p.R) / kContent);
  const int cw1 = (int)(min(Tcont - 1, i_last + p.R) / kContent);
  const int e_end = min(p.nent, (int)blockIdx.z * p.epb + p.epb);
  // chunk of entry e, or -1 (wave-uniform)
  auto chunk_of = [&](int e) -> int {
    int c;
    if (e < p.K) {
      c = __builtin_amdgcn_readlane(s0, e);
      if (c >= cw0 && c <= cw1) c = -1;
    } else if (e < 2 * p.K) {
      c = __builtin_amdgcn_readlane(s1, e - p.K);
      if (c >= 0 && ((c >= cw0 && c <= cw1) || __ballot(s0 == c) != 0ull)) c = -1;
    } else {
      c = cw0 + (e - 2 * p.K);
      if (c > cw1) c = -1;
    }
    return c;
  };
  // first entry at or after e that has a chunk (e_end if none); its chunk in c
  auto next_entry = [&](int e, int& c) -> int {
    c = -1;
    for (; e < e_end; ++e) {
      c = chunk_of(e);
      if (c >= 0) return e;
    }
    return e_end;
  };

  // this lane's row: query qq of the tile, head hh of the group
  const int qq = (lane & 15) >> 3, hh = lane & 7;
  const int h = g * G + hh;
  const int t = tb0 + qq;
  const bool rv = t < p.nq && hh < G;
  const long long iq = (long long)p.q0 + t;
  const size_t rows = (size_t)p.B * p.Hq * p.nq;
  float* pp = p.part + ((size_t)blockIdx.z * rows + ((size_t)b * p.Hq + h) * p.nq + t) * (D + 4);
  int c;
  int e = next_entry((int)blockIdx.z * p.epb, c);
  if (c < 0) {
    if (rv && g16 == 0) {
      pp[D] = kNegBig;
      pp[D + 1] = 0.f;
    }
    return;
  }
  auto kv_of = [&](int cc, const T*& kc, const T*& vc) {
    kc = reinterpret_cast<const T*>(p.k) + ((size_t)bg * L + (size_t)cc * kSlots) * D;
    vc = reinterpret_cast<const T*>(p.v) + ((size_t)bg * L + (size_t)cc * kSlots) * D;
  };
  const T* kc;
  const T* vc;
  kv_of(c, kc, vc);
  if constexpr (SWZ) dma_chunk<D, 1>(reinterpret_cast<const bf16_t*>(kc), reinterpret_cast<const bf16_t*>(vc), bufs, 0, lane);

  // the two queries' chunk logits into LDS and the query fragments, all awaited
  // before the next chunk load is issued (the compiler does not count those loads)
  if (p.K > 0) {   // uniform; zsel may be NULL when K = 0
    constexpr int kZPer = 16;   // 2 queries x G <= 8 heads x K <= 64 values over 64 lanes
    const int nz = 2 * G * p.K;
    float zv[kZPer];
#pragma unroll
    for (int j = 0; j < kZPer; ++j) {
      if (64 * j < nz) {   // uniform
        const int x = lane + 64 * j < nz ? lane + 64 * j : nz - 1;
        const int xq = x / (G * p.K), rem = x - xq * G * p.K, xh = rem / p.K, xk = rem - xh * p.K;
        const int tt = tb0 + xq < p.nq ? tb0 + xq : tb0;
        zv[j] = p.zsel[(((size_t)b * p.Hq + g * G + xh) * p.nq + tt) * p.K + xk];
      }
    }
#pragma unroll
    for (int j = 0; j < kZPer; ++j)
      if (lane + 64 * j < nz) zs[lane + 64 * j] = zv[j] * kLog2e;
  }
  QFrag<D, NP> qf;
  const T* qrow = rv ? reinterpret_cast<const T*>(p.q) + (((size_t)b * p.Hq + h) * L + slot_of_i(iq)) * D : nullptr;
  load_qfrag<T, D, NP>(qf, qrow, lane);
  wait_vm<0>();
  wait_lgkm0();
  compiler_fence();

  f32x4 acc[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) acc[dm] = zero4();
  float m = kNegBig, l = 0.f;
  int cur = 0;
  for (;;) {
    int cn;
    const int en = next_entry(e + 1, cn);
    bf16_t* buf = bufs + cur * C::BUFE;
    if constexpr (SWZ) {
      if (cn >= 0) {
        kv_of(cn, kc, vc);
        dma_chunk<D, 1>(reinterpret_cast<const bf16_t*>(kc), reinterpret_cast<const bf16_t*>(vc),
                        bufs + (cur ^ 1) * C::BUFE, 0, lane);
        wait_vm<NI2>();   // chunk c has landed; chunk cn stays in flight
      } else {
        wait_vm<0>();
      }
      compiler_fence();
    } else {
      KVStage<T, D, 64> stg;
      stg.load(kc, vc, lane, 64);
      __syncthreads();   // the previous chunk's reads are done
      stg.store(buf, lane);
      __syncthreads();
      if (cn >= 0) kv_of(cn, kc, vc);
    }
    // per lane: window keys, selected-chunk keys or nothing
    const long long cf = (long long)c * kContent, cl = cf + kContent - 1;
    const bool win = cf <= iq + p.R && cl >= iq - p.R;
    const unsigned long long m0 = __ballot(s0 == c), m1 = __ballot(s1 == c);   // full-wave ballots
    const unsigned long long mq = qq ? m1 : m0;
    const int ksel = mq != 0ull ? __builtin_ctzll(mq) : -1;
    int mode = win ? 1 : (ksel >= 0 ? 2 : 0);
    if (!rv) mode = 0;
    int lo = 0, hi = kContent - 1;
    if (mode == 1) {
      lo = (int)max(0LL, iq - p.R - cf);
      hi = (int)min((long long)kContent - 1, iq + p.R - cf);
    }
    const float zc = mode == 2 ? zs[(qq * G + hh) * p.K + ksel] : 0.f;
    f32x4 sacc[4];
    s_tile<D, NP, SWZ>(buf, qf, sacc, lane);
    float alpha;
    if constexpr (NP == 1) {
      const bool general = __ballot(mode == 1) != 0ull;
      s16x8 pf[2];
      alpha = tile_update_bf16(sacc, general, mode, lo, hi, zc, p.sl2, g16, m, l, pf);
      if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[dm][i] *= alpha;
      }
      pv_tile_packed<D>(buf, pf, acc, lane);
    } else {
      float x[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[mt][i] = sacc[mt][i];
      alpha = tile_update(x, mode, lo, hi, zc, p.sl2, g16, m, l);
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[dm][i] *= alpha;
      pv_tile<D, NP, SWZ>(buf, x, acc, lane);
    }
    if (cn < 0) break;
    wait_lgkm0();   // every LDS read of this buffer has returned before it is loaded again
    compiler_fence();
    e = en;
    c = cn;
    if constexpr (SWZ) cur ^= 1;
  }
  if (!rv) return;
  if (l > 0.f) {
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      float v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = acc[dm][i];
      store4<float>(pp + 16 * dm + 4 * g16, v4);
    }
  }
  if (g16 == 0) {
    pp[D] = m;
    pp[D + 1] = l;
  }
}

// bf16 variant of routed_decode_kernel with the same entries, runs and partials:
// a chunk's K fragments (the A operand of S^T = K Q^T, row-major in HBM like the
// operand) go straight into registers and only its V passes through LDS (for the
// transposing reads), so a block holds 2 x 16 KB of LDS instead of 2 x 32 KB. The
// next chunk's V is loaded into the other LDS buffer when a chunk starts, its K
// right after S has consumed the current K registers: both are in flight during the
// softmax and P V. (Blocks of four waves with short runs merged in LDS, to keep
// more chunks in flight per CU, measured slower: the gather of scattered 16 KB
// chunks from a cache larger than the 256 MB MALL is bound by HBM, not by loads in
// flight.)
template <int D>
__global__ __launch_bounds__(64) void routed_decode_kv_kernel(RoutedParams p) {
  typedef TileLayout<D, true> TL;
  constexpr int KS = D / 32;
  constexpr int HE = TL::VE;                 // elements of one V half
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* vbufs = reinterpret_cast<bf16_t*>(smem);                                  // [2][64][D] swizzled V
  const int G = p.Hq / p.Hkv;
  float* zs = reinterpret_cast<float*>(smem + (size_t)2 * HE * sizeof(bf16_t));     // [2][G][K]
  const int lane = threadIdx.x, g16 = lane >> 4, L16 = lane & 15;
  const int bg = blockIdx.y, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int tb0 = 2 * blockIdx.x;
  const long long L = (long long)p.N * kSlots;
  const long long Tcont = (long long)p.N * kContent;
  const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.k) + (size_t)bg * L * D;
  const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.v) + (size_t)bg * L * D;

  // selections of the two queries: lane k holds entry k
  int s0 = -1, s1 = -1;
  if (p.K > 0) {   // uniform; idx may be NULL when K = 0
    const int kl = lane < p.K ? lane : p.K - 1, t1 = tb0 + 1 < p.nq ? tb0 + 1 : tb0;
    s0 = p.idx[((size_t)bg * p.nq + tb0) * p.K + kl];        // in bounds for every lane: no branch
    s1 = p.idx[((size_t)bg * p.nq + t1) * p.K + kl];
    if (lane >= p.K || s0 >= p.N) s0 = -1;
    if (lane >= p.K || tb0 + 1 >= p.nq || s1 >= p.N) s1 = -1;
  }
  const int t_last = min(tb0 + 2, p.nq) - 1;
  const long long i_first = (long long)p.q0 + tb0, i_last = (long long)p.q0 + t_last;
  const int cw0 = (int)(max(0LL, i_first - p.R) / kContent);
  const int cw1 = (int)(min(Tcont - 1, i_last + p.R) / kContent);
  const int e_end = min(p.nent, (int)blockIdx.z * p.epb + p.epb);
  // chunk of entry e, or -1 (wave-uniform); a chunk in several places belongs to one entry
  auto chunk_of = [&](int e) -> int {
    int c;
    if (e < p.K) {
      c = __builtin_amdgcn_readlane(s0, e);
      if (c >= cw0 && c <= cw1) c = -1;
    } else if (e < 2 * p.K) {
      c = __builtin_amdgcn_readlane(s1, e - p.K);
      if (c >= 0 && ((c >= cw0 && c <= cw1) || __ballot(s0 == c) != 0ull)) c = -1;
    } else {
      c = cw0 + (e - 2 * p.K);
      if (c > cw1) c = -1;
    }
    return c;
  };
  auto next_entry = [&](int e, int& c) -> int {
    c = -1;
    for (; e < e_end; ++e) {
      c = chunk_of(e);
      if (c >= 0) return e;
    }
    return e_end;
  };

  // this lane's row: query qq of the tile, head hh of the group
  const int qq = (lane & 15) >> 3, hh = lane & 7;
  const int h = g * G + hh;
  const int t = tb0 + qq;
  const bool rv = t < p.nq && hh < G;
  const long long iq = (long long)p.q0 + t;
  const size_t rows = (size_t)p.B * p.Hq * p.nq;
  float* pp = p.part + ((size_t)blockIdx.z * rows + ((size_t)b * p.Hq + h) * p.nq + t) * (D + 4);
  int c;
  int e = next_entry((int)blockIdx.z * p.epb, c);
  if (c < 0) {
    if (rv && g16 == 0) {
      pp[D] = kNegBig;
      pp[D + 1] = 0.f;
    }
    return;
  }
  int voffv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) voffv[u] = dma_voff<D>(true, u, lane);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)vbufs);
  // K fragments of chunk cc: lane holds key 16 mt + l % 16, d = 32 ks + 8 (l / 16) + {0..7}
  s16x8 kf[4][KS];
  auto load_k = [&](int cc) {
    const bf16_t* kc = kg + ((size_t)cc * kSlots + L16) * D + 8 * g16;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[mt][ks] = load8(kc + 16 * mt * D + 32 * ks);
  };
  dma_half_fast<D>(vg + (size_t)c * kSlots * D, lds0, voffv);
  load_k(c);

  // the two queries' chunk logits into LDS and the query fragments
  if (p.K > 0) {   // uniform; zsel may be NULL when K = 0
    constexpr int kZPer = 16;   // 2 queries x G <= 8 heads x K <= 64 values over 64 lanes
    const int nz = 2 * G * p.K;
    float zv[kZPer];
#pragma unroll
    for (int j = 0; j < kZPer; ++j) {
      if (64 * j < nz) {   // uniform
        const int x = lane + 64 * j < nz ? lane + 64 * j : nz - 1;
        const int xq = x / (G * p.K), rem = x - xq * G * p.K, xh = rem / p.K, xk = rem - xh * p.K;
        const int tt = tb0 + xq < p.nq ? tb0 + xq : tb0;
        zv[j] = p.zsel[(((size_t)b * p.Hq + g * G + xh) * p.nq + tt) * p.K + xk];
      }
    }
#pragma unroll
    for (int j = 0; j < kZPer; ++j)
      if (lane + 64 * j < nz) zs[lane + 64 * j] = zv[j] * kLog2e;
  }
  QFrag<D, 1> qf;
  load_qfrag<bf16_t, D, 1>(qf, rv ? reinterpret_cast<const bf16_t*>(p.q) + (((size_t)b * p.Hq + h) * L + slot_of_i(iq)) * D
                                  : nullptr, lane);

  f32x4 acc[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) acc[dm] = zero4();
  float m = kNegBig, l = 0.f;
  int cur = 0;
  for (;;) {
    int cn;
    const int en = next_entry(e + 1, cn);
    wait_vm<0>();   // chunk c's K (registers) and V (LDS buffer cur) have landed
    wait_lgkm0();   // and every read of the other V buffer (the previous chunk's) has returned
    compiler_fence();
    if (cn >= 0) dma_half_fast<D>(vg + (size_t)cn * kSlots * D, lds0 + (uint32_t)((cur ^ 1) * HE * 2), voffv);
    // per lane: window keys, selected-chunk keys or nothing
    const long long cf = (long long)c * kContent, cl = cf + kContent - 1;
    const bool win = cf <= iq + p.R && cl >= iq - p.R;
    const unsigned long long m0 = __ballot(s0 == c), m1 = __ballot(s1 == c);   // full-wave ballots
    const unsigned long long mq = qq ? m1 : m0;
    const int ksel = mq != 0ull ? __builtin_ctzll(mq) : -1;
    int mode = win ? 1 : (ksel >= 0 ? 2 : 0);
    if (!rv) mode = 0;
    int lo = 0, hi = kContent - 1;
    if (mode == 1) {
      lo = (int)max(0LL, iq - p.R - cf);
      hi = (int)min((long long)kContent - 1, iq + p.R - cf);
    }
    const bool partial = __ballot(lo > 0 || hi < kContent - 1) != 0ull;
    const float zc = mode == 2 ? zs[(qq * G + hh) * p.K + ksel] : 0.f;
    f32x4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[mt] = mfma16(kf[mt][ks], qf.f[ks][0], sacc[mt]);
    }
    if (cn >= 0) load_k(cn);   // the K registers are free once the MFMAs above have read them
    s16x8 pf[2];
    const float alpha = partial ? tile_softmax<true>(sacc, mode, lo, hi, zc, p.sl2, g16, m, l, pf)
                                : tile_softmax<false>(sacc, mode, lo, hi, zc, p.sl2, g16, m, l, pf);
    if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[dm][i] *= alpha;
    }
    pv_tiles<D, 1>(vbufs + cur * HE, &pf, &acc);
    if (cn < 0) break;
    e = en;
    c = cn;
    cur ^= 1;
  }
  wait_vm<0>();
  if (!rv) return;
  if (l > 0.f) {
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      float v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = acc[dm][i];
      store4<float>(pp + 16 * dm + 4 * g16, v4);
    }
  }
  if (g16 == 0) {
    pp[D] = m;
    pp[D + 1] = l;
  }
}

// ---------------------------------------------------------------- sliding-window attention
//
// swa_kernel serves float32 inputs (three bf16 planes staged through registers);
// swa_bf16_kernel below serves bf16 inputs.

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
      s_tile<D, NP, false>(buf, qf[tt], sacc, lane);
      const int mode = trow[tt] < L ? 1 : 0;
      const int lo = (int)max(0LL, trow[tt] - p.R - kb);
      const int hi = (int)min(63LL, min(L - 1, trow[tt] + p.R) - kb);
      float x[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[mt][i] = sacc[mt][i];
      const float alpha = tile_update(x, mode, lo, hi, 0.f, p.sl2, g16, mrow[tt], lrow[tt]);
#pragma unroll
      for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tt][dm][i] *= alpha;
      pv_tile<D, NP, false>(buf, x, acc[tt], lane);
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

// Sliding-window attention, bf16 inputs. A block of G waves (one head each, the
// heads of one KV group) covers 32 consecutive slots: two 16-row tiles per wave,
// so every K fragment of S^T = K Q^T and every V^T fragment of O^T += V^T P^T
// read from LDS serves both tiles. The 64-slot K/V tiles of the band come into a
// RING-deep LDS ring with direct-to-LDS loads (swizzled layout), issued by the
// first DW waves; a raw s_barrier per tile, after each issuing wave has seen its
// own loads of that tile land, makes the tile visible and frees the slot of the
// tile before the previous one (no register staging, and no barrier that would
// wait for the loads still in flight). The loop is software-pipelined by one
// tile: while the softmax of tile j runs on the VALU, the MFMAs form S of tile
// j + 1, interleaved with it instruction by instruction where both query tiles
// are fully inside the window; then P V of tile j. Rows of a partial last tile
// are read from the sequence's last row and masked out.
template <int D, int DW, int RING>
__global__ __launch_bounds__(512) void swa_bf16_kernel(SwaParams p) {
  typedef TileLayout<D, true> TL;
  constexpr int BUFE = TL::PL;              // K then V of one 64-slot tile
  constexpr int NI = D / 8;                 // 1 KB instructions per half
  constexpr int RPI = 512 / D, BPR = D / 8;
  constexpr int PER = 2 * NI / DW;          // instructions per issuing wave per tile
  // at most RING - 2 tiles of loads are in flight per issuing wave
  static_assert(RING >= 3 && (2 * NI) % DW == 0 && (RING - 2) * PER < 64, "in-flight loads must fit the vmcnt counter");
  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* kvb = reinterpret_cast<bf16_t*>(smem);
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g16 = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const int bg = blockIdx.y, b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int h = g * G + w;
  const int t0 = blockIdx.x * 32;   // slot indices fit in 32 bits (L < 2^31 - 2^16)
  const int L = p.L;
  const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.k) + (size_t)bg * L * D;
  const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.v) + (size_t)bg * L * D;

  QFrag<D, 1> qf[2];
  f32x4 acc[2][D / 16];
  float mrow[2], lrow[2];
  int trow[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    trow[tt] = t0 + 16 * tt + (lane & 15);
    load_qfrag<bf16_t, D, 1>(
        qf[tt], trow[tt] < L ? reinterpret_cast<const bf16_t*>(p.q) + (((size_t)b * p.Hq + h) * L + trow[tt]) * D : nullptr,
        lane);
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) acc[tt][dm] = zero4();
    mrow[tt] = kNegBig;
    lrow[tt] = 0.f;
  }
  const uint32_t klane = (uint32_t)((lane & 15) * D * 2 + ((g16 ^ TL::swz_k(lane & 15)) << 4));
  const uint32_t vlane = (uint32_t)(((lane >> 2) * D + 4 * (lane & 3) + 8 * TL::swz_v(lane >> 2)) * 2);
  const int R = min(p.R, L);   // a wider radius covers the same slots
  const int lo_all = max(0, t0 - R);
  const int hi_all = min(L - 1, t0 + 31 + R);
  const int kb0 = (lo_all / 64) * 64;
  const int ntile = (hi_all - kb0) / 64 + 1;

  // the query fragments have landed: from here on this wave's vector loads are its
  // share of the ring, which the loop waits for itself
  wait_vm<0>();
  // Full tiles: groups of four 1 KB loads with a uniform base (SGPRs) and per-lane
  // offsets that repeat every group (the swizzle period); the rare partial last
  // tile reads its missing rows from the sequence's last row. The lane index is
  // formed in place so that no address is kept live across the loop.
  static_assert(PER % 4 == 0, "whole groups of four loads per wave");
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)kvb);
  auto issue = [&](int j) {
    if (w >= DW) return;
    const int kb = kb0 + 64 * j;
    const uint32_t lbuf = lds0 + (uint32_t)((j % RING) * BUFE * 2);
    int ln;   // the lane index formed in place: no per-lane offsets live across the loop
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    if (kb + 64 <= L) {
#pragma unroll
      for (int gi = 0; gi < PER / 4; ++gi) {
        const int i0 = w * PER + 4 * gi;   // first load of the group (wave-uniform)
        const bool is_v = i0 >= NI;
        const int ii0 = is_v ? i0 - NI : i0;
        const bf16_t* sg = (is_v ? vg : kg) + (size_t)kb * D + (size_t)ii0 * 512;
        const uint32_t lg = lbuf + (uint32_t)((is_v ? TL::KE : 0) + ii0 * 512) * 2;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lg + u * 1024),
                       "v"(dma_voff<D>(is_v, u, ln)), "s"(sg)
                       : "memory", "m0");
      }
    } else {
      const int rows_valid = L - kb;
      bf16_t* buf = kvb + (j % RING) * BUFE;
      for (int u = 0; u < PER; ++u) {
        const int jj = w * PER + u;
        const bool is_v = jj >= NI;
        const int ii = is_v ? jj - NI : jj;
        const int pr = ii * RPI + ln / BPR, pb = ln % BPR;
        const int sr = pr < rows_valid ? pr : rows_valid - 1;
        const int sw = is_v ? TL::swz_v(pr) : TL::swz_k(pr);
        dma16((is_v ? vg : kg) + (size_t)(kb + sr) * D + ((pb ^ sw) << 3), buf + (is_v ? TL::KE : 0) + ii * 512);
      }
    }
  };
  // Tile t is made visible by arrive(t): this wave's loads of it have landed
  // (tiles up to t + RING - 3 being issued), every wave's LDS reads before the
  // barrier have returned, and tile t + RING - 2 goes into the slot of tile t - 2,
  // which no wave reads any more (in the pipelined run below a wave reads tile
  // t - 1 after arrive(t), so the slot of t - 1 is not yet free).
  auto arrive = [&](int t) {
    if (w < DW) {
      const int ahead = min(t + RING - 3, ntile - 1) - t;
      static_assert(RING <= 4, "at most one tile in flight beside the one awaited");
      if (ahead >= 1) wait_vm<(RING >= 4 ? PER : 0)>();
      else wait_vm<0>();
    }
    wait_lgkm0();
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    if (t + RING - 2 < ntile) issue(t + RING - 2);
  };
  // Tile jt lies inside the window of all 32 rows (and of the sequence): the run
  // between the band's edges, whose products start from zero accumulators.
  auto inside = [&](int jt) {
    const int kb = kb0 + 64 * jt;
    return kb >= t0 + 31 - R && kb + 63 <= t0 + R && kb + 63 < L && t0 + 31 < L;   // wave-uniform
  };
  // Accumulators of S^T for a band-edge tile jt before the products: 0, or -inf for
  // each key outside a row's window or past the sequence (rows past the sequence mask
  // all keys), so the softmax needs no bounds.
  auto s_init = [&](int jt, f32x4 (&s)[2][4]) {
    const int kb = kb0 + 64 * jt;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int lo = 1, hi = 0;
      if (trow[tt] < L) {
        lo = max(0, trow[tt] - R - kb);
        hi = min(63, min(L - 1, trow[tt] + R) - kb);
      }
      // key 16 mt + 4 g16 + i is kept when lo <= key <= hi
      const int los = lo - 4 * g16, his = hi - 4 * g16;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[tt][mt][i] = (16 * mt + i >= los && 16 * mt + i <= his) ? 0.f : -INFINITY;
    }
  };

  for (int jj = 0; jj < RING - 2 && jj < ntile; ++jj) issue(jj);
  // Pipelined walk over the band: S of tile j + 1 (every K fragment read serving both
  // query tiles) is formed ahead of the softmax of tile j, whose VALU work runs beside
  // those MFMAs; then P V of tile j for both query tiles (a query tile that does not
  // reach a band-edge tile gets P = 0 there).
  f32x4 sc[2][4], sn[2][4];
  arrive(0);
  if (inside(0)) {
    s_tiles_x<D, 2>(lds0, qf, sc, klane);
  } else {
    s_init(0, sc);
    s_tiles_x_acc<D, 2>(lds0, qf, sc, klane);
  }
  for (int j = 0; j < ntile; ++j) {
    s16x8 pf[2][2];
    float alpha[2];
    const bool nx = j + 1 < ntile;
    if (nx) arrive(j + 1);
    // (after the last tile the products are formed once more on that tile and
    // dropped, which keeps them and the softmax in one scheduling region)
    const int jn = nx ? j + 1 : j;
    // the products and the softmax in one region, one MFMA then a few softmax VALU
    // instructions in turn; the region is written twice so that the run between
    // the edges keeps zero-initialised products
    if (inside(jn)) {
      s_tiles_x<D, 2>(lds0 + (uint32_t)((jn % RING) * BUFE * 2), qf, sn, klane);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        alpha[tt] = tile_softmax<false, false>(sc[tt], 1, 0, 63, 0.f, p.sl2, g16, mrow[tt], lrow[tt], pf[tt]);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    } else {
      s_init(jn, sn);
      s_tiles_x_acc<D, 2>(lds0 + (uint32_t)((jn % RING) * BUFE * 2), qf, sn, klane);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        alpha[tt] = tile_softmax<false, false>(sc[tt], 1, 0, 63, 0.f, p.sl2, g16, mrow[tt], lrow[tt], pf[tt]);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (__ballot(alpha[tt] != 1.f) != 0ull) {
#pragma unroll
        for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tt][dm][i] *= alpha[tt];
      }
    }
    pv_tiles_x<D, 2>(lds0 + (uint32_t)(((j % RING) * BUFE + TL::KE) * 2), pf, acc, vlane);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) sc[tt][mt] = sn[tt][mt];
  }

#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    if (trow[tt] >= L) continue;
    const float inv = 1.f / lrow[tt];
    bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (((size_t)b * p.Hq + h) * L + trow[tt]) * D;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      float v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = acc[tt][dm][i] * inv;
      store4<bf16_t>(orow + 16 * dm + 4 * g16, v4);
    }
    if (p.lse != nullptr && g16 == 0)
      p.lse[((size_t)b * p.Hq + h) * L + trow[tt]] = (mrow[tt] + __log2f(lrow[tt])) * kLn2;
  }
}

// ---------------------------------------------------------------- host side

static size_t align256a(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- static scratch
// For lcr_routed_attention_noalloc (callers that cannot allocate device memory):
// the partial results of decode-sized plans go to this file-scope device array
// instead of a caller workspace. Each GPU the library runs on holds its own copy
// until the process ends. Host code must not pass the array's name to a kernel
// (on the host it is only a stand-in): its device address is looked up once per
// device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

size_t routed_scratch_bytes() { return kScratchBytes; }

hipError_t routed_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {   // first call on this device, which is current
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

// Polls before a wait on an LDS counter gives up, read at every launch.
static constexpr int kDefaultWaitLimit = 1 << 22;
static std::atomic<int> g_wait_limit{kDefaultWaitLimit};
int set_wait_limit(int polls) { return g_wait_limit.exchange(polls >= 1 ? polls : kDefaultWaitLimit); }
static int wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }

static std::atomic<int> g_tile_order{0};
int set_tile_order(int reversed) { return g_tile_order.exchange(reversed != 0 ? 1 : 0); }
int tile_order() { return g_tile_order.load(std::memory_order_relaxed); }

// LDS bytes of the K/V staging buffers (all planes, all buffers).
static size_t kv_lds_bytes(int d, int dtype) {
  const int np = dtype == 0 ? 3 : 1;
  const size_t one = (size_t)np * 64 * ((d + 8) + (d + 16)) * 2;
  const int nbuf = (np == 3 && d == 128) ? 1 : 2;
  return nbuf * one;
}

size_t routed_lds_limit() { return 160 * 1024 - 512; }  // room for the static LDS variables

static int routed_nbuf(int d, int dtype, int waves) {
  if (dtype == 1) return waves == 1 ? 2 : 3;        // direct-to-LDS ring, prefetch distance NBUF - 1
  return (d == 128) ? 1 : 2;                        // three float32-derived planes
}

static size_t routed_buf_bytes(int d, int dtype) {
  if (dtype == 1) return (size_t)2 * 64 * d * 2;    // swizzled K + V, one plane
  return (size_t)3 * 64 * ((d + 8) + (d + 16)) * 2;  // padded K + V, three planes
}

static size_t routed_lds(const RouteDims& dm, int K, int qblock, int waves) {
  const int G = dm.Hq / dm.Hkv;
  size_t b = (size_t)routed_nbuf(dm.d, dm.dtype, waves) * routed_buf_bytes(dm.d, dm.dtype) + (size_t)qblock * K * 4 +
             (size_t)qblock * G * K * 4 + (size_t)dm.N * 4 + (size_t)dm.N;
  return (b + 15) & ~(size_t)15;
}

// LDS of routed_prefill_kernel: the pool of nh K-or-V halves and the per-position
// tables (chunk, query mask, position of each chunk).
static size_t prefill_lds(const RouteDims& dm, int nh, int tpw) {
  const size_t mask = tpw == 1 ? sizeof(PfCfg<1>::Mask) : sizeof(PfCfg<2>::Mask);
  const size_t b = (size_t)nh * 64 * dm.d * 2 + (size_t)dm.N * (mask + 4 + 2);
  return ((b + 15) & ~(size_t)15) + 4 * (2 + 1 + 32);   // + the block's counters
}

// tiles per consumer wave of the pooled prefill kernel
static constexpr int kPfTiles = 2;

// single-wave blocks the decode-sized plan aims at (about two per CU: 1,024 and
// 2,048 measured slower, the combine then reads more partials)
static constexpr long long kDecodeBlocks = 512;

// Queries per block of the pooled prefill kernel (at most qmax, one block per CU at a
// time). A launch of a few rounds of blocks leaves most CUs idle while its last,
// partial round runs; where the full-size blocks take at most kBalanceRounds rounds,
// the count that minimises rounds x queries per block is taken instead (the block
// time scales with its queries), ties to the larger count. On 256 CUs the 16K prefill
// (4 x 16,128 queries) goes from 1,468 blocks of 44 (5.7 rounds, six block times)
// to 1,536 blocks of 42 (six rounds of 42/44 of a block time).
constexpr int kCus = 256;            // compute units of an MI355X
constexpr int kBalanceRounds = 8;
static int balanced_qblock(long long nq, long long groups, int qmax) {
  auto rounds = [&](int qb) { return ((nq + qb - 1) / qb * groups + kCus - 1) / kCus; };
  if (nq <= 0 || rounds(qmax) > kBalanceRounds) return qmax;
  int best = qmax;
  long long best_cost = rounds(qmax) * qmax;
  for (int qb = qmax - 1; qb >= (qmax + 1) / 2; --qb) {
    const long long cost = rounds(qb) * qb;
    if (cost < best_cost) {
      best_cost = cost;
      best = qb;
    }
  }
  return best;
}

AttnPlan plan_routed_attention(const RouteDims& dm, int K, int radius, int nq) {
  AttnPlan pl;
  pl.nent = 0;
  pl.epb = 0;
  // Prefill-sized problems: 8 waves x 2 tiles = 32 queries per block, no split;
  // 8 waves x 1 tile when the selections of 32 queries do not fit in LDS.
  pl.waves = 8;
  pl.tiles = 2;
  pl.qblock = 2 * pl.waves * pl.tiles;
  pl.nsplit = 1;
  if (routed_lds(dm, K, pl.qblock, pl.waves) > routed_lds_limit()) {
    pl.waves = 8;
    pl.tiles = 1;
    pl.qblock = 2 * pl.waves * pl.tiles;
  }
  const long long blocks_prefill = (long long)((nq + pl.qblock - 1) / pl.qblock) * dm.B * dm.Hkv;
  pl.kind = 0;
  if (blocks_prefill < 256) {
    // Decode-sized. With a narrow window: one single-wave block per (2-query
    // tile, entry), entries = 2K selected chunks + the tile's window chunks.
    const long long wmax = (2LL * radius + 2) / kContent + 3;       // window chunks of a 2-query tile
    const long long nent = 2LL * K + (wmax < dm.N ? wmax : dm.N);
    pl.waves = 1;
    pl.tiles = 1;
    pl.qblock = 2;
    if (nent <= kMaxPartials) {
      // runs of epb entries per block: enough blocks to fill the chip (about two
      // single-wave blocks per CU), at least two chunks per block
      pl.kind = 1;
      const long long tiles = (long long)((nq + 1) / 2) * dm.B * dm.Hkv;
      long long runs = (kDecodeBlocks + tiles - 1) / (tiles > 0 ? tiles : 1);
      if (runs > nent / 2) runs = nent / 2;
      if (runs < 1) runs = 1;
      pl.epb = (int)((nent + runs - 1) / runs);
      pl.nsplit = (int)((nent + pl.epb - 1) / pl.epb);
      pl.nent = (int)nent;
    } else {
      // Wide window: the tile's chunk list is split across blocks instead.
      const long long blocks = (long long)((nq + 1) / 2) * dm.B * dm.Hkv;
      long long ns = (1024 + blocks - 1) / (blocks > 0 ? blocks : 1);
      pl.nsplit = (int)(ns < 1 ? 1 : (ns > 8 ? 8 : ns));
    }
  }
  if (pl.kind == 1) {
    // bf16: two V halves (K goes to registers); float32: one staged K + V buffer of three planes
    pl.lds = (dm.dtype == 1 ? (size_t)2 * 64 * dm.d * 2 : routed_buf_bytes(dm.d, dm.dtype)) +
             (size_t)2 * (dm.Hq / dm.Hkv) * K * 4;
  } else {
    pl.lds = routed_lds(dm, K, pl.qblock, pl.waves);
  }
  pl.nbuf = 0;
  if (pl.kind == 0 && pl.nsplit == 1 && dm.dtype == 1 && dm.N < 32768) {
    // bf16 prefill: producer / consumer kernel with the largest pool of halves that fits
    for (int nh : {9, 8, 6, 4}) {
      const size_t lds = prefill_lds(dm, nh, kPfTiles);
      if (lds <= routed_lds_limit()) {
        pl.kind = 2;
        pl.nbuf = nh;
        pl.tiles = kPfTiles;
        pl.waves = kPfTiles == 1 ? pf_waves<1>() : pf_waves<2>();
        pl.qblock = balanced_qblock(nq, (long long)dm.B * dm.Hkv, kPfTiles == 1 ? pf_qblock<1>() : pf_qblock<2>());
        pl.lds = lds;
        break;
      }
    }
  }
  // kind 1 always writes its partials (one per run, merged by combine_kernel), even for a single run
  pl.ws = (pl.nsplit > 1 || pl.kind == 1) ? align256a((size_t)pl.nsplit * dm.B * dm.Hq * nq * (dm.d + 4) * 4) : 0;
  return pl;
}

template <typename T, int D, int WAVES, int TPW, int NBUF>
static hipError_t launch_routed_t(const RouteDims& dm, const AttnPlan& pl, const RoutedParams& prm, hipStream_t st) {
  constexpr int QB = 2 * WAVES * TPW;
  auto kern = routed_attention_kernel<T, D, WAVES, TPW, NBUF>;
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
  constexpr int NB = sizeof(T) == 2 ? 3 : (D == 128 ? 1 : 2);
  constexpr int NB1 = sizeof(T) == 2 ? 2 : NB;
  if (pl.waves == 8 && pl.tiles == 2) return launch_routed_t<T, D, 8, 2, NB>(dm, pl, prm, st);
  if (pl.waves == 8) return launch_routed_t<T, D, 8, 1, NB>(dm, pl, prm, st);
  return launch_routed_t<T, D, 1, 1, NB1>(dm, pl, prm, st);
}

template <typename T, int D>
static hipError_t launch_decode_t(const RouteDims& dm, const AttnPlan& pl, const RoutedParams& prm, hipStream_t st) {
  auto kern = std::is_same<T, bf16_t>::value ? routed_decode_kv_kernel<D> : routed_decode_kernel<T, D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds);
  if (e != hipSuccess) return e;
  dim3 grid((prm.nq + 1) / 2, dm.B * dm.Hkv, pl.nsplit);
  hipLaunchKernelGGL(kern, grid, dim3(64), pl.lds, st, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t rows = (size_t)dm.B * dm.Hq * prm.nq;
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, prm.part,
                     pl.nsplit, rows, prm.o, prm.lse, prm.nq, dm.N, prm.q0);
  return hipGetLastError();
}

template <int D, int NH>
static hipError_t launch_prefill_t(const RouteDims& dm, const AttnPlan& pl, const RoutedParams& prm, hipStream_t st) {
  constexpr int TPW = kPfTiles;
  auto kern = routed_prefill_kernel<D, NH, TPW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds);
  if (e != hipSuccess) return e;
  const int tiles = (prm.nq + prm.qb - 1) / prm.qb * dm.B * dm.Hkv;
  hipLaunchKernelGGL(kern, dim3(xcd_grid(tiles)), dim3(64 * pf_waves<TPW>()), pl.lds, st, prm);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const RouteDims& dm, const AttnPlan& pl, const RoutedParams& prm, hipStream_t st) {
  if (pl.nbuf >= 9) return launch_prefill_t<D, 9>(dm, pl, prm, st);
  if (pl.nbuf >= 8) return launch_prefill_t<D, 8>(dm, pl, prm, st);
  if (pl.nbuf >= 6) return launch_prefill_t<D, 6>(dm, pl, prm, st);
  return launch_prefill_t<D, 4>(dm, pl, prm, st);
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
  prm.nent = pl.nent;
  prm.epb = pl.epb;
  prm.spin = wait_limit();
  prm.rev = tile_order();
  prm.qb = pl.qblock;
  prm.sl2 = scale * kLog2e;
  if (pl.kind == 2) return dm.d == 64 ? launch_prefill_d<64>(dm, pl, prm, st) : launch_prefill_d<128>(dm, pl, prm, st);
  if (pl.kind == 1) {
    if (dm.dtype == 1) return dm.d == 64 ? launch_decode_t<bf16_t, 64>(dm, pl, prm, st)
                                         : launch_decode_t<bf16_t, 128>(dm, pl, prm, st);
    return dm.d == 64 ? launch_decode_t<float, 64>(dm, pl, prm, st) : launch_decode_t<float, 128>(dm, pl, prm, st);
  }
  if (dm.dtype == 1) return dm.d == 64 ? launch_routed_d<bf16_t, 64>(dm, pl, prm, st)
                                       : launch_routed_d<bf16_t, 128>(dm, pl, prm, st);
  return dm.d == 64 ? launch_routed_d<float, 64>(dm, pl, prm, st) : launch_routed_d<float, 128>(dm, pl, prm, st);
}

// bf16: a ring of at most 4 swizzled 64-slot K/V tiles (2 for a one-wave block at
// d = 128, where 32 loads per tile leave room for one tile in flight); float32: the
// register-staged padded planes of swa_kernel.

size_t bwd_query_pool_lds(int d, int N) { return (size_t)9 * 64 * d * 2 + (size_t)N * 10; }

template <int D>
static hipError_t launch_bwd_query_pool_d(const BwdQueryParams& prm, hipStream_t st) {
  const size_t lds = bwd_query_pool_lds(D, prm.N);
  hipError_t e = hipFuncSetAttribute((const void*)bwd_query_pool_kernel<D, 9>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int nqb = (prm.nq + kBqQB - 1) / kBqQB;
  hipLaunchKernelGGL((bwd_query_pool_kernel<D, 9>), dim3(xcd_grid(nqb * prm.B * prm.Hkv)), dim3(64 * kBqWaves), lds,
                     st, prm);
  return hipGetLastError();
}

hipError_t launch_bwd_query_pool(const RouteDims& dm, const void* q, const void* k, const void* v, const void* o,
                                 const void* dO, const int32_t* idx, const float* zsel, const float* lse, int K,
                                 int radius, float scale, int q0, int nq, float* dq, float* dzsel, float* dsum,
                                 float* cbias, float* cu, hipStream_t st) {
  BwdQueryParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.o = o;
  prm.dO = dO;
  prm.idx = idx;
  prm.zsel = zsel;
  prm.lse = lse;
  prm.dq = dq;
  prm.dzsel = dzsel;
  prm.dsum = dsum;
  prm.cbias = cbias;
  prm.cu = cu;
  prm.B = dm.B;
  prm.Hq = dm.Hq;
  prm.Hkv = dm.Hkv;
  prm.N = dm.N;
  prm.K = K;
  prm.R = radius;
  prm.q0 = q0;
  prm.nq = nq;
  prm.spin = wait_limit();
  prm.rev = tile_order();
  prm.scale = scale;
  return dm.d == 128 ? launch_bwd_query_pool_d<128>(prm, st) : launch_bwd_query_pool_d<64>(prm, st);
}

size_t swa_lds_bytes(int d, int dtype) {
  return dtype == 1 ? (size_t)4 * 2 * 64 * d * 2 : kv_lds_bytes(d, dtype);
}

template <int D, int DW, int RING>
static hipError_t launch_swa_bf16_t(const SwaParams& prm, int G, hipStream_t st) {
  const size_t lds = (size_t)RING * 2 * 64 * D * 2;
  auto kern = swa_bf16_kernel<D, DW, RING>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((prm.L + 31) / 32), prm.B * prm.Hkv);
  hipLaunchKernelGGL(kern, grid, dim3(64 * G), lds, st, prm);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_swa_bf16(const SwaParams& prm, int G, hipStream_t st) {
  if (G >= 4) return launch_swa_bf16_t<D, 4, 4>(prm, G, st);
  if (G >= 2) return launch_swa_bf16_t<D, 2, 4>(prm, G, st);
  if constexpr (D == 128) return launch_swa_bf16_t<D, 1, 3>(prm, G, st);
  else return launch_swa_bf16_t<D, 1, 4>(prm, G, st);
}

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
  if (dtype == 1) return d == 64 ? launch_swa_bf16<64>(prm, G, st) : launch_swa_bf16<128>(prm, G, st);
  return d == 64 ? launch_swa_t<float, 64>(prm, G, st) : launch_swa_t<float, 128>(prm, G, st);
}

}  // namespace lcr
