// Backward of routed attention on gfx950 (bf16 inputs, float32 gradients).
//
// "The 172x Speedup Has an Evidence Budget" (section "How learned routing
// controls what the model can read"): which chunks are chosen is not
// differentiable, and the router learns through the masses the selected chunks
// receive. So idx is a constant here; gradients flow into q, k, v and into the
// chunk logits zsel. "Prefilling-dLLM v2", Figure 3 caption fixes the forward:
// one partition P over window logits a_u = scale q.k_u and chunk logits z_c,
// and inside chunk c a softmax pi over its 63 content keys.
//
// Gradients, per (query row, head), with D = dO . o (the forward's output):
//   window key u:  p_u = exp(a_u - lse);            ds_u = p_u (dO.v_u - D)
//   chunk c:       P_c = exp(z_c - lse), U_c = sum_j pi_j dO.v_cj
//                  dz_c = P_c (U_c - D)
//   chunk key j:   p_cj = P_c pi_j;                  ds_cj = p_cj (dO.v_cj - U_c)
//   dq = scale sum ds k,   dk += scale ds q,   dv += p dO
// Every probability above is exp(scale q.k + bias) with a per-(row, source)
// bias: -lse for window keys, z_c - lse - LSE_c for chunk keys (LSE_c the
// chunk's own log-sum-exp), so the key-side pass needs only two floats per
// (row, selected chunk), written by the query-side pass.
//
// Kernels (one call, in stream order):
//  1. bwd_query_kernel: one wave per 2 consecutive queries x 8 head rows (the
//     16 MFMA columns of a tile, as in the forward). The wave walks the union of
//     its window chunks and selected chunks in ascending order; per chunk it
//     recomputes S^T = K Q^T and dP^T = V dO^T, forms ds, and accumulates
//     dQ^T += K^T dS^T (K^T read from LDS with the transposing read). Writes dq,
//     dzsel, D and, per (row, selected chunk), the bias and U_c.
//  2. inverse index: per (batch, KV group, chunk) the list of (query, slot)
//     entries that selected it, in ascending query order (per-tile counts,
//     a scan over chunks and tiles, placement row by row).
//  3. bwd_key_kernel: one block per (batch, KV group, chunk), wave w owning keys
//     16w .. 16w+15. Rows (query, head) are staged 32 at a time in LDS: first
//     the queries whose window reaches the chunk, then the chunk's entries from
//     the inverse index. Per step S = Q K^T and dP = dO V^T (K, V fragments in
//     registers), then dV += P^T dO and dK += dS^T Q with P and dS straight from
//     the S output layout as the A operand (no LDS round trip). Each key row of
//     dk and dv is written once, by the block that owns its chunk.
#include <limits.h>

#include <algorithm>

#include "device.h"
#include "launch.h"

namespace lcr {

struct BwdParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* o;
  const bf16_t* dO;
  const int32_t* idx;   // [B,Hkv,nq,K]
  const float* zsel;    // [B,Hq,nq,K]
  const float* lse;     // [B,Hq,nq]
  float* dq;            // [B,Hq,L,d]  rows slot(i)
  float* dk;            // [B,Hkv,L,d] every row
  float* dv;            // [B,Hkv,L,d] every row
  float* dzsel;         // [B,Hq,nq,K]
  float* dsum;          // ws [B,Hq,nq]
  float* cbias;         // ws [B,Hq,nq,K]
  float* cu;            // ws [B,Hq,nq,K]
  int* cnt;             // ws [B*Hkv*N]
  int* th;              // ws [B*Hkv*ntile*N]  per-tile chunk counts, then first positions
  int* off;             // ws [B*Hkv*(N+1)]
  int* list;            // ws [B*Hkv*nq*K]  entries t*K + slot
  int B, Hq, Hkv, N, G, K, R, q0, nq;
  float scale;
};

__device__ __forceinline__ int slot_of_c(int i) { return (i / kContent) * kSlots + (i % kContent); }

__device__ __forceinline__ void store8(bf16_t* p, s16x8 v) { *reinterpret_cast<s16x8*>(p) = v; }

__device__ __forceinline__ s16x8 zero8() { return s16x8{0, 0, 0, 0, 0, 0, 0, 0}; }

// ---------------------------------------------------------------- 1. query side

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_query_kernel(BwdParams p) {
  constexpr int LDK = D + 8;   // padded K rows in LDS
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  bf16_t* kl = reinterpret_cast<bf16_t*>(smem) + w * 64 * LDK;
  const int tiles_bg = (p.nq + 1) >> 1;
  const int tile = blockIdx.x * 4 + w;
  if (tile >= p.B * p.Hkv * tiles_bg) return;   // whole wave; this kernel has no block barrier
  const int bg = tile / tiles_bg, b = bg / p.Hkv, g = bg % p.Hkv;
  const int t0 = 2 * (tile % tiles_bg);
  const int L16 = lane & 15, g16 = lane >> 4;
  const int qi = L16 >> 3, hh = L16 & 7;
  const int t = t0 + qi;
  const bool valid = t < p.nq && hh < p.G;
  const int T = p.N * kContent;
  const int i = p.q0 + min(t, p.nq - 1);
  const int hq = g * p.G + min(hh, p.G - 1);
  const size_t L = (size_t)p.N * kSlots;
  const size_t row = (((size_t)b * p.Hq + hq) * L + slot_of_c(i)) * D;
  const size_t rq = ((size_t)b * p.Hq + hq) * p.nq + min(t, p.nq - 1);

  // B operands (column = this lane's row): q and dO, d = 32 ks + 8 g16 + j
  s16x8 qf[D / 32], df[D / 32];
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    if (valid) {
      qf[ks] = load8(p.q + row + 32 * ks + 8 * g16);
      df[ks] = load8(p.dO + row + 32 * ks + 8 * g16);
      const s16x8 of = load8(p.o + row + 32 * ks + 8 * g16);
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += bf2f((bf16_t)df[ks][j]) * bf2f((bf16_t)of[j]);
    } else {
      qf[ks] = zero8();
      df[ks] = zero8();
    }
  }
  dsum = col_sum(dsum);
  const float lse = valid ? p.lse[rq] : 0.f;
  if (valid && g16 == 0) {
    p.dsum[rq] = dsum;
    for (int kk = 0; kk < p.K; ++kk) p.dzsel[rq * p.K + kk] = 0.f;
  }
  const int lo = max(0, i - p.R), hi = min(T - 1, i + p.R);    // this column's window (content indices)
  const int tl = min(t0 + 1, p.nq - 1);
  const int wc_lo = max(0, p.q0 + t0 - p.R) / kContent;        // union of the wave's window chunks
  const int wc_hi = min(T - 1, p.q0 + tl + p.R) / kContent;
  const int32_t* id0 = p.idx + (((size_t)b * p.Hkv + g) * p.nq + t0) * p.K;
  const bool has1 = t0 + 1 < p.nq;
  auto sel_at = [&](int which, int pos) -> int {
    if (pos >= p.K || (which == 1 && !has1)) return INT_MAX;
    const int c = __builtin_amdgcn_readfirstlane(id0[which * p.K + pos]);
    return c < 0 ? INT_MAX : c;
  };
  int p0 = 0, p1 = 0;
  int nx0 = sel_at(0, 0), nx1 = sel_at(1, 0);
  int nw = wc_lo;
  const float sc = p.scale;

  f32x4 dqa[D / 16];
#pragma unroll
  for (int dm = 0; dm < D / 16; ++dm) dqa[dm] = zero4();

  const bf16_t* kbase = p.k + (size_t)bg * L * D;
  const bf16_t* vbase = p.v + (size_t)bg * L * D;
  while (true) {
    const int cw = nw <= wc_hi ? nw : INT_MAX;
    const int c = min(cw, min(nx0, nx1));
    if (c == INT_MAX) break;
    const int mypos = qi ? p1 : p0;
    const bool is_sel = (qi ? nx1 : nx0) == c;
    const bool in_w = c * kContent <= hi && c * kContent + kContent - 1 >= lo;

    // K of chunk c -> this wave's LDS tile (64 rows x D, padded)
    const bf16_t* kc = kbase + (size_t)c * kSlots * D;
    wait_lgkm0();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {
      const int piece = u * 64 + lane;
      const int r = piece / (D / 8), cb = piece % (D / 8);
      store8(kl + r * LDK + cb * 8, load8(kc + r * D + cb * 8));
    }
    wait_lgkm0();
    asm volatile("" ::: "memory");

    // S^T = K Q^T and dP^T = V dO^T: keys 16 mt + 4 g16 + i, column L16
    f32x4 sacc[4], pacc[4];
    const bf16_t* vc = vbase + (size_t)c * kSlots * D;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = zero4();
      pacc[mt] = zero4();
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const s16x8 a = load8(kl + (16 * mt + L16) * LDK + 32 * ks + 8 * g16);
        sacc[mt] = mfma16(a, qf[ks], sacc[mt]);
        const s16x8 av = load8(vc + (size_t)(16 * mt + L16) * D + 32 * ks + 8 * g16);
        pacc[mt] = mfma16(av, df[ks], pacc[mt]);
      }
    }

    // intra-chunk softmax statistics of every column (used where c is selected)
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * mt + 4 * g16 + e;
        if (j < kContent) mx = fmaxf(mx, sc * sacc[mt][e]);
      }
    mx = col_max(mx);
    float l = 0.f, tu = 0.f;
    float ex[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * mt + 4 * g16 + e;
        ex[mt][e] = j < kContent ? __expf(sc * sacc[mt][e] - mx) : 0.f;
        l += ex[mt][e];
        tu += ex[mt][e] * pacc[mt][e];
      }
    l = col_sum(l);
    tu = col_sum(tu);
    const float il = 1.f / l;
    const float U = tu * il;
    float Pc = 0.f;
    if (is_sel && valid) {
      const float z = p.zsel[rq * p.K + mypos];
      Pc = __expf(z - lse);
      if (g16 == 0) {
        p.dzsel[rq * p.K + mypos] = Pc * (U - dsum);
        p.cbias[rq * p.K + mypos] = z - lse - (mx + __logf(l));
        p.cu[rq * p.K + mypos] = U;
      }
    }

    // ds^T in the S^T layout
    float ds[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * mt + 4 * g16 + e;
        const int u = c * kContent + j;
        float v = 0.f;
        if (in_w) {
          const bool inwin = j < kContent && u >= lo && u <= hi;
          const float pw = inwin ? __expf(sc * sacc[mt][e] - lse) : 0.f;
          v = pw * (pacc[mt][e] - dsum);
        } else if (is_sel) {
          v = Pc * ex[mt][e] * il * (pacc[mt][e] - U);
        }
        ds[mt][e] = valid ? v : 0.f;
      }

    // dQ^T += K^T dS^T: B operand = dS^T (keys as k, permuted as the S^T output)
    s16x8 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[ks][j] = (short)f2bf(j < 4 ? ds[2 * ks][j] : ds[2 * ks + 1][j - 4]);
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const s16x8 a = lds_col_frag(kl, LDK, 32 * ks + 4 * g16, 32 * ks + 16 + 4 * g16, 16 * dm, lane);
        dqa[dm] = mfma16(a, pf[ks], dqa[dm]);
      }

    if (cw == c) ++nw;
    if (nx0 == c) nx0 = sel_at(0, ++p0);
    if (nx1 == c) nx1 = sel_at(1, ++p1);
  }

  if (valid) {
    float* dqr = p.dq + row;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      f32x4 r = dqa[dm] * sc;
      *reinterpret_cast<f32x4*>(dqr + 16 * dm + 4 * g16) = r;
    }
  }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(int* a, size_t n) {
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) a[x] = 0;
}

// ---------------------------------------------------------------- 2. inverse index
// Rows t of one (batch, KV group) are cut into tiles of kIdxTile. The list of
// chunk c holds its entries (t, slot) in ascending t: tile by tile, and inside
// a tile row by row. Per tile an LDS histogram of the chunks it selects; a scan
// over (chunk, tile) gives every tile its first position in each chunk's list;
// one wave per tile then walks its rows in order. The result does not depend on
// scheduling, so dk and dv are reproducible bit for bit.
constexpr int kIdxTile = 256;

__global__ __launch_bounds__(256) void bwd_hist_kernel(BwdParams p) {
  extern __shared__ int hist[];   // [N]
  const int tile = blockIdx.x, bg = blockIdx.y, ntile = gridDim.x;
  for (int c = threadIdx.x; c < p.N; c += 256) hist[c] = 0;
  __syncthreads();
  const int t0 = tile * kIdxTile, t1 = min(p.nq, t0 + kIdxTile);
  const int32_t* id = p.idx + ((size_t)bg * p.nq + t0) * p.K;
  const int n = (t1 - t0) * p.K;
  for (int x = threadIdx.x; x < n; x += 256) {
    const int c = id[x];
    if (c >= 0) atomicAdd(&hist[c], 1);
  }
  __syncthreads();
  int* th = p.th + ((size_t)bg * ntile + tile) * p.N;
  for (int c = threadIdx.x; c < p.N; c += 256) th[c] = hist[c];
}

// One block per (batch, KV group): th[tile][c] becomes the number of entries of
// chunk c in earlier tiles; cnt[c] the chunk's total; off[c] the exclusive
// prefix of cnt (off[N] = all entries of the group).
__global__ __launch_bounds__(256) void bwd_scan_kernel(BwdParams p, int ntile) {
  __shared__ int part[256];
  const int bg = blockIdx.x, tid = threadIdx.x;
  int* th = p.th + (size_t)bg * ntile * p.N;
  int* cnt = p.cnt + (size_t)bg * p.N;
  for (int c = tid; c < p.N; c += 256) {
    int run = 0;
    for (int tl = 0; tl < ntile; ++tl) {
      const int v = th[(size_t)tl * p.N + c];
      th[(size_t)tl * p.N + c] = run;
      run += v;
    }
    cnt[c] = run;
  }
  __syncthreads();
  int* off = p.off + (size_t)bg * (p.N + 1);
  int base = 0;
  for (int c0 = 0; c0 < p.N; c0 += 256) {
    const int v = c0 + tid < p.N ? cnt[c0 + tid] : 0;
    part[tid] = v;
    __syncthreads();
    for (int s = 1; s < 256; s <<= 1) {
      const int a = tid >= s ? part[tid - s] : 0;
      __syncthreads();
      part[tid] += a;
      __syncthreads();
    }
    if (c0 + tid < p.N) off[c0 + tid] = base + part[tid] - v;
    base += part[255];
    __syncthreads();
  }
  if (tid == 0) off[p.N] = base;
}

// One wave per (tile, batch and KV group): rows in order, lane k places entry (t, k).
// Chunks within a row are distinct, so the LDS cursors see no two lanes of one row
// on the same chunk; the atomic keeps positions distinct even if they were not.
__global__ __launch_bounds__(64) void bwd_fill_kernel(BwdParams p) {
  extern __shared__ int curs[];   // [N]
  const int tile = blockIdx.x, bg = blockIdx.y, ntile = gridDim.x, lane = threadIdx.x;
  const int* th = p.th + ((size_t)bg * ntile + tile) * p.N;
  const int* off = p.off + (size_t)bg * (p.N + 1);
  for (int c = lane; c < p.N; c += 64) curs[c] = off[c] + th[c];
  __syncthreads();
  const int t0 = tile * kIdxTile, t1 = min(p.nq, t0 + kIdxTile);
  const size_t per = (size_t)p.nq * p.K;
  int* list = p.list + (size_t)bg * per;
  for (int t = t0; t < t1; ++t) {
    for (int k0 = 0; k0 < p.K; k0 += 64) {
      const int k = k0 + lane;
      const int c = k < p.K ? p.idx[((size_t)bg * p.nq + t) * p.K + k] : -1;
      if (c >= 0) {
        const int pos = atomicAdd(&curs[c], 1);
        list[pos] = t * p.K + k;
      }
    }
  }
}

// ---------------------------------------------------------------- 3. key side

template <int D>
__global__ __launch_bounds__(256) void bwd_key_kernel(BwdParams p) {
  constexpr int LDR = D + 8;
  constexpr int PPT = D / 64;   // 16-byte pieces per thread per staged tensor (32 rows x D/8 pieces / 256)
  __shared__ __align__(16) bf16_t qs[32 * LDR];
  __shared__ __align__(16) bf16_t dos[32 * LDR];
  __shared__ float sbias[32], ssub[32];
  __shared__ int squery[32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L16 = lane & 15, g16 = lane >> 4;
  const int c = blockIdx.x % p.N, bg = blockIdx.x / p.N, b = bg / p.Hkv, g = bg % p.Hkv;
  const size_t L = (size_t)p.N * kSlots;
  const int key = 16 * w + L16;                 // this lane's key (chunk-local slot) in S = Q K^T
  const int iw_lo = max(p.q0, c * kContent - p.R);
  const int iw_hi = min(p.q0 + p.nq - 1, c * kContent + kContent - 1 + p.R);
  const int nwq = max(0, iw_hi - iw_lo + 1);
  const int ncnt = p.cnt[(size_t)bg * p.N + c];
  if (nwq == 0 && ncnt == 0) {   // no queried row reaches this chunk: zero gradients (block-uniform exit)
    float* dkb = p.dk + ((size_t)bg * L + (size_t)c * kSlots) * D;
    float* dvb = p.dv + ((size_t)bg * L + (size_t)c * kSlots) * D;
    for (int x = tid; x < kSlots * D; x += 256) {
      dkb[x] = 0.f;
      dvb[x] = 0.f;
    }
    return;
  }
  const bf16_t* krow = p.k + ((size_t)bg * L + (size_t)c * kSlots + key) * D;
  const bf16_t* vrow = p.v + ((size_t)bg * L + (size_t)c * kSlots + key) * D;
  s16x8 kf[D / 32], vf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    kf[ks] = load8(krow + 32 * ks + 8 * g16);
    vf[ks] = load8(vrow + 32 * ks + 8 * g16);
  }
  f32x4 dka[D / 16], dva[D / 16];
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) {
    dka[nt] = zero4();
    dva[nt] = zero4();
  }
  const float sc = p.scale;
  const int u_key = c * kContent + key;         // content index of this lane's key (key < 63)
  const size_t per = (size_t)p.nq * p.K;
  const int* lst = p.list + (size_t)bg * per + p.off[(size_t)bg * (p.N + 1) + c];

  // staging role of this thread: row sr of the 32, pieces sp*PPT .. +PPT-1 of D/8
  const int sr = tid >> 3, sp = tid & 7;

  for (int pass = 0; pass < 2; ++pass) {
    const int nrows = (pass == 0 ? nwq : ncnt) * p.G;
    const int nsteps = (nrows + 31) / 32;
    s16x8 rq[PPT], rd[PPT];
    float rb = -INFINITY, ru = 0.f;
    int rqi = INT_MIN / 2;
    auto fetch = [&](int step) {
      const int r = step * 32 + sr;
      const int e = r / p.G, h = r % p.G;
      bool ok = r < nrows;
      int t = 0, slotk = 0;
      if (ok) {
        if (pass == 0) {
          t = iw_lo + e - p.q0;
        } else {
          const int ent = lst[e];
          t = ent / p.K;
          slotk = ent % p.K;
        }
      }
      const int hq = g * p.G + h;
      const size_t rowq = ((size_t)b * p.Hq + hq) * p.nq + t;
      const size_t base = (((size_t)b * p.Hq + hq) * L + slot_of_c(p.q0 + t)) * D;
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        rq[u] = ok ? load8(p.q + base + (sp * PPT + u) * 8) : zero8();
        rd[u] = ok ? load8(p.dO + base + (sp * PPT + u) * 8) : zero8();
      }
      if (sp == 0) {
        if (!ok) {
          rb = -INFINITY;
          ru = 0.f;
          rqi = INT_MIN / 2;
        } else if (pass == 0) {
          rb = -p.lse[rowq];
          ru = p.dsum[rowq];
          rqi = p.q0 + t;
        } else {
          rb = p.cbias[rowq * p.K + slotk];
          ru = p.cu[rowq * p.K + slotk];
          rqi = 0;
        }
      }
    };
    if (nsteps > 0) fetch(0);
    for (int step = 0; step < nsteps; ++step) {
      __syncthreads();   // the previous step's readers are done with qs / dos
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        store8(qs + sr * LDR + (sp * PPT + u) * 8, rq[u]);
        store8(dos + sr * LDR + (sp * PPT + u) * 8, rd[u]);
      }
      if (sp == 0) {
        sbias[sr] = rb;
        ssub[sr] = ru;
        squery[sr] = rqi;
      }
      __syncthreads();
      if (step + 1 < nsteps) fetch(step + 1);

      // S = Q K^T, dP = dO V^T: rows 16 mt + 4 g16 + e, key column L16 of this wave
      f32x4 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = zero4();
        pacc[mt] = zero4();
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const s16x8 a = load8(qs + (16 * mt + L16) * LDR + 32 * ks + 8 * g16);
          sacc[mt] = mfma16(a, kf[ks], sacc[mt]);
          const s16x8 ad = load8(dos + (16 * mt + L16) * LDR + 32 * ks + 8 * g16);
          pacc[mt] = mfma16(ad, vf[ks], pacc[mt]);
        }
      }
      float pv[2][4], dsv[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mt + 4 * g16 + e;
          bool ok = key < kContent;
          if (pass == 0) ok = ok && abs(u_key - squery[r]) <= p.R;
          const float pr = ok ? __expf(sc * sacc[mt][e] + sbias[r]) : 0.f;
          pv[mt][e] = pr;
          dsv[mt][e] = pr * (pacc[mt][e] - ssub[r]);
        }
      s16x8 pa, da;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pa[j] = (short)f2bf(j < 4 ? pv[0][j] : pv[1][j - 4]);
        da[j] = (short)f2bf(j < 4 ? dsv[0][j] : dsv[1][j - 4]);
      }
      // dV += P^T dO, dK += dS^T Q: M = this wave's 16 keys, k = the 32 rows (same permutation)
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        const s16x8 bo = lds_col_frag(dos, LDR, 4 * g16, 16 + 4 * g16, 16 * nt, lane);
        dva[nt] = mfma16(pa, bo, dva[nt]);
        const s16x8 bq = lds_col_frag(qs, LDR, 4 * g16, 16 + 4 * g16, 16 * nt, lane);
        dka[nt] = mfma16(da, bq, dka[nt]);
      }
    }
  }

  // lane holds rows key 16 w + 4 g16 + e, column 16 nt + L16
  float* dkb = p.dk + ((size_t)bg * L + (size_t)c * kSlots) * D;
  float* dvb = p.dv + ((size_t)bg * L + (size_t)c * kSlots) * D;
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kr = 16 * w + 4 * g16 + e;
      dkb[(size_t)kr * D + 16 * nt + L16] = sc * dka[nt][e];
      dvb[(size_t)kr * D + 16 * nt + L16] = dva[nt][e];
    }
}

// ---------------------------------------------------------------- host side

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static int bwd_ntile(int nq) { return (nq + kIdxTile - 1) / kIdxTile; }

size_t routed_bwd_ws_bytes(const RouteDims& dm, int K, int nq) {
  const size_t rows = (size_t)dm.B * dm.Hq * nq;
  const size_t bg = (size_t)dm.B * dm.Hkv;
  return al256(rows * 4) + 2 * al256(rows * K * 4) + al256(bg * dm.N * 4) + al256(bg * (dm.N + 1) * 4) +
         al256(bg * bwd_ntile(nq) * dm.N * 4) + al256(bg * nq * K * 4);
}

size_t routed_bwd_lds_bytes(int d) { return (size_t)4 * 64 * (d + 8) * 2; }

template <int D>
static hipError_t launch_bwd_d(const BwdParams& prm, hipStream_t st) {
  const size_t bgn = (size_t)prm.B * prm.Hkv * prm.N;
  const int ntile = bwd_ntile(prm.nq);
  const size_t idx_lds = (size_t)prm.N * 4;
  hipError_t e = hipFuncSetAttribute((const void*)bwd_hist_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)idx_lds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)bwd_fill_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)idx_lds);
  if (e != hipSuccess) return e;
  if (prm.nq > 0) {
    hipLaunchKernelGGL(bwd_hist_kernel, dim3(ntile, prm.B * prm.Hkv), dim3(256), idx_lds, st, prm);
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(prm.B * prm.Hkv), dim3(256), 0, st, prm, ntile);
    if (prm.K > 0) hipLaunchKernelGGL(bwd_fill_kernel, dim3(ntile, prm.B * prm.Hkv), dim3(64), idx_lds, st, prm);
  } else {
    // nothing selects anything: zero counts and offsets, the key side then writes zero gradients
    const size_t no = (size_t)prm.B * prm.Hkv * (prm.N + 1);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)std::min<size_t>((bgn + 255) / 256, 65535)), dim3(256), 0,
                       st, prm.cnt, bgn);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)std::min<size_t>((no + 255) / 256, 65535)), dim3(256), 0,
                       st, prm.off, no);
  }
  const int tiles = prm.B * prm.Hkv * ((prm.nq + 1) / 2);
  const size_t lds = routed_bwd_lds_bytes(D);
  e = hipFuncSetAttribute((const void*)bwd_query_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (tiles > 0) hipLaunchKernelGGL(bwd_query_kernel<D>, dim3((tiles + 3) / 4), dim3(256), lds, st, prm);
  hipLaunchKernelGGL(bwd_key_kernel<D>, dim3((unsigned)bgn), dim3(256), 0, st, prm);
  return hipGetLastError();
}

hipError_t launch_routed_attention_backward(const RouteDims& dm, const void* q, const void* k, const void* v,
                                            const int32_t* idx, const float* zsel, int K, int radius,
                                            float scale, int q0, int nq, const void* o, const float* lse,
                                            const void* dO, float* dq, float* dk, float* dv, float* dzsel,
                                            void* ws, hipStream_t st) {
  BwdParams prm;
  prm.q = (const bf16_t*)q;
  prm.k = (const bf16_t*)k;
  prm.v = (const bf16_t*)v;
  prm.o = (const bf16_t*)o;
  prm.dO = (const bf16_t*)dO;
  prm.idx = idx;
  prm.zsel = zsel;
  prm.lse = lse;
  prm.dq = dq;
  prm.dk = dk;
  prm.dv = dv;
  prm.dzsel = dzsel;
  const size_t rows = (size_t)dm.B * dm.Hq * nq;
  const size_t bgn = (size_t)dm.B * dm.Hkv * dm.N;
  char* w = (char*)ws;
  prm.dsum = (float*)w;
  w += al256(rows * 4);
  prm.cbias = (float*)w;
  w += al256(rows * K * 4);
  prm.cu = (float*)w;
  w += al256(rows * K * 4);
  prm.cnt = (int*)w;
  w += al256(bgn * 4);
  prm.off = (int*)w;
  w += al256(((size_t)dm.B * dm.Hkv * (dm.N + 1)) * 4);
  prm.th = (int*)w;
  w += al256((size_t)dm.B * dm.Hkv * bwd_ntile(nq) * dm.N * 4);
  prm.list = (int*)w;
  prm.B = dm.B;
  prm.Hq = dm.Hq;
  prm.Hkv = dm.Hkv;
  prm.N = dm.N;
  prm.G = dm.Hq / dm.Hkv;
  prm.K = K;
  prm.R = radius;
  prm.q0 = q0;
  prm.nq = nq;
  prm.scale = scale;
  return dm.d == 128 ? launch_bwd_d<128>(prm, st) : launch_bwd_d<64>(prm, st);
}

}  // namespace lcr
