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
//  1. query side: bwd_query_pool_kernel (attention.hip, beside the forward whose
//     chunk pool it shares) walks one ascending stream of the chunks any of a
//     block's 22 queries needs; where that pool does not fit in LDS,
//     bwd_query_kernel here gives each wave of 2 queries its own walk. Per
//     (tile, chunk) both recompute S^T = K Q^T and dP^T = V dO^T, form ds, and
//     accumulate dQ^T += K^T dS^T (K^T read from LDS with the transposing read).
//     They write dq, dzsel, D and, per (row, selected chunk), the bias and U_c.
//  2. inverse index: per (batch, KV group, chunk) the list of (query, slot)
//     entries that selected it, in ascending query order (per-tile counts,
//     a scan over chunks and tiles, placement row by row).
//  3. bwd_key_kernel: one block per (batch, KV group, chunk), wave w owning keys
//     16w .. 16w+15. Rows (query, head) are staged 64 at a time in LDS: first
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
    for (int ks = 0; ks < 2; ++ks) pf[ks] = pack8_bf16(ds[2 * ks], ds[2 * ks + 1]);
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
constexpr int kMaxTopK = 64;   // largest K
constexpr int kKeyRows = 64;   // (query, head) rows the key-side kernel stages per step

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
__global__ __launch_bounds__(256, 2) void bwd_key_kernel(BwdParams p) {
  constexpr int LDR = D + 16;   // staged row stride in elements (288 bytes at d = 128: rows 8 banks apart)
  constexpr int RS = kKeyRows;   // rows staged per step
  constexpr int TPR = 256 / RS;  // staging threads per row
  constexpr int PPT = D / 8 / TPR;   // 16-byte pieces per thread per staged tensor
  __shared__ __align__(16) bf16_t qs[RS * LDR];
  __shared__ __align__(16) bf16_t dos[RS * LDR];
  __shared__ float sbias[RS], ssub[RS];
  __shared__ int squery[RS];
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

  // staging role of this thread: row sr of the RS, pieces sp*PPT .. +PPT-1 of D/8
  const int sr = tid / TPR, sp = tid % TPR;

  for (int pass = 0; pass < 2; ++pass) {
    const int nrows = (pass == 0 ? nwq : ncnt) * p.G;
    const int nsteps = (nrows + RS - 1) / RS;
    s16x8 rq[PPT], rd[PPT];
    float rb = -INFINITY, ru = 0.f;
    int rqi = INT_MIN / 2;
    // entry word of this thread's row in a step (pass 1), read two steps ahead of its use
    auto entry = [&](int step) -> int {
      const int r = step * RS + sr;
      if (pass == 0 || r >= nrows) return 0;
      return lst[r / p.G];
    };
    auto fetch = [&](int step, int ent) {
      const int r = step * RS + sr;
      const int e = r / p.G, h = r % p.G;
      const bool ok = r < nrows;
      int t = 0, slotk = 0;
      if (ok) {
        if (pass == 0) {
          t = iw_lo + e - p.q0;
        } else {
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
        // bias: lse (pass 0, used negated) or the chunk bias (pass 1); rows past the end
        // get a bias that makes their probability exactly 0. Loaded values are stored as
        // they are, so no wait on them is needed before the next step.
        if (!ok) {
          rb = pass == 0 ? INFINITY : -INFINITY;
          ru = 0.f;
          rqi = INT_MIN / 2;
        } else if (pass == 0) {
          rb = p.lse[rowq];
          ru = p.dsum[rowq];
          rqi = p.q0 + t;
        } else {
          rb = p.cbias[rowq * p.K + slotk];
          ru = p.cu[rowq * p.K + slotk];
          rqi = 0;
        }
      }
    };
    int ent_next = 0;
    if (nsteps > 0) {
      fetch(0, entry(0));
      ent_next = entry(1);
    }
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
      if (step + 1 < nsteps) {
        fetch(step + 1, ent_next);
        ent_next = entry(step + 2);
      }

      // S = Q K^T, dP = dO V^T: rows 16 mt + 4 g16 + e, key column L16 of this wave
      constexpr int MT = RS / 16;
      f32x4 sacc[MT], pacc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
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
      float pv[MT][4], dsv[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mt + 4 * g16 + e;
          bool ok = key < kContent;
          if (pass == 0) ok = ok && abs(u_key - squery[r]) <= p.R;
          const float bias = pass == 0 ? -sbias[r] : sbias[r];
          const float pr = ok ? __expf(sc * sacc[mt][e] + bias) : 0.f;
          pv[mt][e] = pr;
          dsv[mt][e] = pr * (pacc[mt][e] - ssub[r]);
        }
      // dV += P^T dO, dK += dS^T Q: M = this wave's 16 keys, k = the RS rows in 32-row
      // steps (rows 32 kq + 4 g16 + j and 32 kq + 16 + 4 g16 + j, as the S output holds them)
#pragma unroll
      for (int kq = 0; kq < RS / 32; ++kq) {
        const s16x8 pa = pack8_bf16(pv[2 * kq], pv[2 * kq + 1]);
        const s16x8 da = pack8_bf16(dsv[2 * kq], dsv[2 * kq + 1]);
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) {
          const s16x8 bo = lds_col_frag(dos, LDR, 32 * kq + 4 * g16, 32 * kq + 16 + 4 * g16, 16 * nt, lane);
          dva[nt] = mfma16(pa, bo, dva[nt]);
          const s16x8 bq = lds_col_frag(qs, LDR, 32 * kq + 4 * g16, 32 * kq + 16 + 4 * g16, 16 * nt, lane);
          dka[nt] = mfma16(da, bq, dka[nt]);
        }
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


// ---------------------------------------------------------------- float32 inputs
// The same gradients for float32 q, k, v, o, dO, in plain float32 VALU arithmetic
// (every product and sum in float32, a fixed order: reproducible bit for bit). The
// float32 entry point serves parity-sized problems, so these kernels favour a plain
// structure over speed; the inverse index is the bf16 path's.
//  bwd32_query_kernel: one block per (batch, head, query row); a wave takes one key
//    at a time (lanes own D/64 dimensions each, dot products by wave sums). Window
//    keys: p = exp(scale q.k - lse), ds = p (dO.v - D). Selected chunk c (waves
//    take chunk slots in turn): the chunk's logits and dO.v per key (lane j holds
//    key j), its own log-sum-exp LSE_c, pi_j, U_c = sum pi_j dO.v_j, dz_c =
//    P_c (U_c - D), ds_j = P_c pi_j (dO.v_j - U_c). dq = scale sum ds k (the four
//    waves' partial sums added in wave order). Writes dq, dzsel and, for the key
//    side, D, the chunk bias z_c - lse - LSE_c and U_c.
//  bwd32_key_kernel: one block per (batch, KV group, chunk); lane l of wave w owns
//    key 16 w + l / 4 and a quarter of the dimensions. Rows (query, head) are
//    staged 16 at a time: the window's queries, then the chunk's inverse-index
//    entries; per row p = exp(scale q.k + bias) (window: bias -lse, keys outside
//    the row's window excluded; chunk: bias z_c - lse - LSE_c), ds = p (dO.v - sub)
//    (sub: D or U_c); dk = scale sum ds q, dv = sum p dO.
constexpr int kBwd32Rows = 16;

template <int D>
__global__ __launch_bounds__(256) void bwd32_query_kernel(BwdParams p) {
  constexpr int DPL = D / 64;   // dimensions per lane
  __shared__ float part[4][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / p.G;
  const size_t L = (size_t)p.N * kSlots;
  const float* q = reinterpret_cast<const float*>(p.q);
  const float* kk = reinterpret_cast<const float*>(p.k);
  const float* vv = reinterpret_cast<const float*>(p.v);
  const float* o = reinterpret_cast<const float*>(p.o);
  const float* dO = reinterpret_cast<const float*>(p.dO);
  const int i = p.q0 + t;
  const size_t rq = ((size_t)b * p.Hq + h) * p.nq + t;   // (batch, head, row) of lse, dsum, zsel
  const size_t qoff = (((size_t)b * p.Hq + h) * L + slot_of_c(i)) * D;
  const float* kg = kk + ((size_t)b * p.Hkv + g) * L * D;
  const float* vg = vv + ((size_t)b * p.Hkv + g) * L * D;
  float qv[DPL], dv[DPL], acc[DPL];
  float dsum = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int dd = DPL * lane + e;
    qv[e] = q[qoff + dd];
    dv[e] = dO[qoff + dd];
    dsum += dv[e] * o[qoff + dd];
    acc[e] = 0.f;
  }
  dsum = wave_sum(dsum);
  const float lse = p.lse[rq];
  auto dots = [&](size_t koff, float& sq, float& sd) {
    float a = 0.f, c = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      a += qv[e] * kg[koff + DPL * lane + e];
      c += dv[e] * vg[koff + DPL * lane + e];
    }
    sq = wave_sum(a);
    sd = wave_sum(c);
  };
  // window keys, wave w taking every fourth
  const int T = p.N * kContent;
  const int lo = max(0, i - p.R), hi = min(T - 1, i + p.R);
  for (int u = lo + w; u <= hi; u += 4) {
    const size_t koff = (size_t)slot_of_c(u) * D;
    float sq, sd;
    dots(koff, sq, sd);
    const float ds = expf(p.scale * sq - lse) * (sd - dsum);
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += ds * kg[koff + DPL * lane + e];
  }
  // selected chunks, wave w taking slots w, w + 4, ...
  for (int ks = w; ks < p.K; ks += 4) {
    const int c = p.idx[(((size_t)b * p.Hkv + g) * p.nq + t) * p.K + ks];
    if (c < 0) {
      if (lane == 0) {
        p.dzsel[rq * p.K + ks] = 0.f;
        p.cbias[rq * p.K + ks] = -INFINITY;
        p.cu[rq * p.K + ks] = 0.f;
      }
      continue;
    }
    float lj = -INFINITY, ej = 0.f;   // lane j: key j's logit and dO.v
    for (int j = 0; j < kContent; ++j) {
      float sq, sd;
      dots((size_t)(c * kSlots + j) * D, sq, sd);
      if (lane == j) {
        lj = p.scale * sq;
        ej = sd;
      }
    }
    const float m = wave_max(lj);
    const float lsec = m + logf(wave_sum(lane < kContent ? expf(lj - m) : 0.f));
    const float pij = lane < kContent ? expf(lj - lsec) : 0.f;
    const float U = wave_sum(pij * ej);
    const float z = p.zsel[rq * p.K + ks];
    const float Pc = expf(z - lse);
    const float dsj = Pc * pij * (ej - U);
    for (int j = 0; j < kContent; ++j) {
      const float dj = __shfl(dsj, j);
      const size_t koff = (size_t)(c * kSlots + j) * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += dj * kg[koff + DPL * lane + e];
    }
    if (lane == 0) {
      p.dzsel[rq * p.K + ks] = Pc * (U - dsum);
      p.cbias[rq * p.K + ks] = z - lse - lsec;
      p.cu[rq * p.K + ks] = U;
    }
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) part[w][DPL * lane + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int dd = threadIdx.x;
    reinterpret_cast<float*>(p.dq)[qoff + dd] = p.scale * (((part[0][dd] + part[1][dd]) + part[2][dd]) + part[3][dd]);
  }
  if (threadIdx.x == 0) p.dsum[rq] = dsum;
}

template <int D>
__global__ __launch_bounds__(256) void bwd32_key_kernel(BwdParams p) {
  constexpr int DQ = D / 4;          // dimensions per lane
  constexpr int RB = kBwd32Rows;     // rows staged per round
  __shared__ float sq[RB][D], sdo[RB][D];
  __shared__ float sbias[RB], ssub[RB];
  __shared__ int squery[RB];         // content index of a window row, INT_MIN / 2 for chunk rows and padding
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x % p.N, bg = blockIdx.x / p.N, b = bg / p.Hkv, g = bg % p.Hkv;
  const size_t L = (size_t)p.N * kSlots;
  const int key = 16 * w + lane / 4, d0 = DQ * (lane & 3);
  const float* q = reinterpret_cast<const float*>(p.q);
  const float* dO = reinterpret_cast<const float*>(p.dO);
  const size_t krow = ((size_t)bg * L + (size_t)c * kSlots + key) * D;
  float kf[DQ], vf[DQ], dka[DQ], dva[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    kf[e] = reinterpret_cast<const float*>(p.k)[krow + d0 + e];
    vf[e] = reinterpret_cast<const float*>(p.v)[krow + d0 + e];
    dka[e] = 0.f;
    dva[e] = 0.f;
  }
  const int u_key = c * kContent + key;   // content index of this lane's key (key < 63)
  const int iw_lo = max(p.q0, c * kContent - p.R);
  const int iw_hi = min(p.q0 + p.nq - 1, c * kContent + kContent - 1 + p.R);
  const int nwq = max(0, iw_hi - iw_lo + 1);
  const int ncnt = p.nq > 0 ? p.cnt[(size_t)bg * p.N + c] : 0;
  const size_t per = (size_t)p.nq * p.K;
  const int* lst = p.list + (size_t)bg * per + (p.nq > 0 ? p.off[(size_t)bg * (p.N + 1) + c] : 0);
  const int nrow = (nwq + ncnt) * p.G;   // window rows first, then the chunk's entries, G heads each
  for (int r0 = 0; r0 < nrow; r0 += RB) {
    __syncthreads();   // the previous round's readers are done
    // stage the round's q and dO rows (padding rows as zeros) and their scalars
    for (int x = tid; x < RB * D; x += 256) {
      const int rr = x / D, dd = x % D, r = r0 + rr;
      float qx = 0.f, dx = 0.f;
      if (r < nrow) {
        const int e = r / p.G, hh = r % p.G, hq = g * p.G + hh;
        const int i = e < nwq ? iw_lo + e : p.q0 + lst[e - nwq] / p.K;
        const size_t off = (((size_t)b * p.Hq + hq) * L + slot_of_c(i)) * D + dd;
        qx = q[off];
        dx = dO[off];
      }
      sq[rr][dd] = qx;
      sdo[rr][dd] = dx;
    }
    if (tid < RB) {
      const int r = r0 + tid;
      float bias = -INFINITY, sub = 0.f;
      int qi = INT_MIN / 2;
      if (r < nrow) {
        const int e = r / p.G, hh = r % p.G, hq = g * p.G + hh;
        if (e < nwq) {
          qi = iw_lo + e;
          const size_t rq = ((size_t)b * p.Hq + hq) * p.nq + (qi - p.q0);
          bias = -p.lse[rq];
          sub = p.dsum[rq];
        } else {
          const int ent = lst[e - nwq];
          const size_t rq = ((size_t)b * p.Hq + hq) * p.nq + ent / p.K;
          bias = p.cbias[rq * p.K + ent % p.K];
          sub = p.cu[rq * p.K + ent % p.K];
        }
      }
      sbias[tid] = bias;
      ssub[tid] = sub;
      squery[tid] = qi;
    }
    __syncthreads();
    const int nr = min(RB, nrow - r0);
    for (int rr = 0; rr < nr; ++rr) {
      float a = 0.f, dd = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        a += sq[rr][d0 + e] * kf[e];
        dd += sdo[rr][d0 + e] * vf[e];
      }
      // the key's four lanes hold quarters of the dimensions
      a += __shfl_xor(a, 1);
      a += __shfl_xor(a, 2);
      dd += __shfl_xor(dd, 1);
      dd += __shfl_xor(dd, 2);
      const int qi = squery[rr];
      bool ok = key < kContent;
      if (qi != INT_MIN / 2) ok = ok && abs(u_key - qi) <= p.R;
      const float pr = ok ? expf(p.scale * a + sbias[rr]) : 0.f;
      const float ds = pr * (dd - ssub[rr]);
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        dka[e] += ds * sq[rr][d0 + e];
        dva[e] += pr * sdo[rr][d0 + e];
      }
    }
  }
  float* dkb = p.dk + krow;
  float* dvb = p.dv + krow;
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    dkb[d0 + e] = p.scale * dka[e];
    dvb[d0 + e] = dva[e];
  }
}

// ---------------------------------------------------------------- 4. summary pooling backward
// "Prefilling-dLLM v2", Figure 3 caption: alpha = softmax_j(scale q_m . k_j) over the
// chunk's 63 content keys, s = sum_j alpha_j k_j; "The 172x Speedup...": entropy
// H = -sum_j alpha_j ln alpha_j. For upstream gradients ds, dH:
//   g_j = ds . k_j - (ln alpha_j + 1) dH,  dlam_j = alpha_j (g_j - sum_i alpha_i g_i)
//   dq_m = scale sum_j dlam_j k_j,  dk_j += alpha_j ds + scale dlam_j q_m.
// One wave per (batch, KV group, chunk) walks the group's heads; K (float32, padded
// rows) and the key gradient live in LDS; lanes own keys for the logits and
// columns for the d-vectors.
template <typename T, int D>
__global__ __launch_bounds__(64) void summary_bwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         float scale, const float* __restrict__ ds,
                                                         const float* __restrict__ dH, float* __restrict__ dq,
                                                         float* __restrict__ dk, int Hq, int Hkv, int N) {
  constexpr int LK = D + 1;
  extern __shared__ float sbw[];            // kt [63][D+1], gk [63][D], vq [D], vds [D], wal [64], wdl [64]
  float* kt = sbw;
  float* gk = kt + kContent * LK;
  float* vq = gk + kContent * D;
  float* vds = vq + D;
  float* wal = vds + D;
  float* wdl = wal + 64;
  const int lane = threadIdx.x;
  const int c = blockIdx.x % N, bg = blockIdx.x / N, b = bg / Hkv, g = bg % Hkv, G = Hq / Hkv;
  const size_t L = (size_t)N * kSlots;
  const T* kc = k + ((size_t)bg * L + (size_t)c * kSlots) * D;
  for (int x = lane; x < kContent * D; x += 64) {
    kt[(x / D) * LK + x % D] = Elem<T>::to_f(kc[x]);
    gk[x] = 0.f;
  }
  __syncthreads();
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const size_t hn = ((size_t)b * Hq + h) * N + c;
    const T* qm = q + (((size_t)b * Hq + h) * L + (size_t)c * kSlots + kSlots - 1) * D;
    for (int e = lane; e < D; e += 64) {
      vq[e] = Elem<T>::to_f(qm[e]);
      vds[e] = ds[hn * D + e];
    }
    __syncthreads();
    // lane j < 63: logit and ds . k_j
    float lam = -INFINITY, gdk = 0.f;
    if (lane < kContent) {
      float a = 0.f;
      for (int e = 0; e < D; ++e) {
        const float kv = kt[lane * LK + e];
        a += vq[e] * kv;
        gdk += vds[e] * kv;
      }
      lam = scale * a;
    }
    const float m = wave_max(lam);
    const float ex = lane < kContent ? __expf(lam - m) : 0.f;
    const float z = wave_sum(ex);
    const float al = ex / z;
    const float lnal = lam - m - __logf(z);
    const float gj = lane < kContent ? gdk - (lnal + 1.f) * dH[hn] : 0.f;
    const float ag = wave_sum(al * gj);
    const float dl = lane < kContent ? al * (gj - ag) : 0.f;
    wal[lane] = al;
    wdl[lane] = dl;
    __syncthreads();
    // columns e: dq_m[e] and this head's share of dk[j][e]
    float* dqm = dq + (((size_t)b * Hq + h) * L + (size_t)c * kSlots + kSlots - 1) * D;
    for (int e = lane; e < D; e += 64) {
      float acc = 0.f;
      const float dse = vds[e], qe = scale * vq[e];
      for (int j = 0; j < kContent; ++j) {
        acc += wdl[j] * kt[j * LK + e];
        gk[j * D + e] += wal[j] * dse + wdl[j] * qe;
      }
      dqm[e] = scale * acc;
    }
    __syncthreads();
  }
  float* dkc = dk + ((size_t)bg * L + (size_t)c * kSlots) * D;
  for (int x = lane; x < kContent * D; x += 64) dkc[x] += gk[x];
}

template <typename T>
static hipError_t launch_summary_bwd_t(const RouteDims& dm, const void* q, const void* k, float scale,
                                       const float* ds, const float* dH, float* dq, float* dk, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)dm.B * dm.Hkv * dm.N));
  const size_t lds = ((size_t)kContent * (dm.d + 1) + (size_t)kContent * dm.d + 2 * dm.d + 128) * 4;
  const void* fn = dm.d == 128 ? (const void*)summary_bwd_kernel<T, 128> : (const void*)summary_bwd_kernel<T, 64>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (dm.d == 128)
    hipLaunchKernelGGL((summary_bwd_kernel<T, 128>), grid, dim3(64), lds, st, (const T*)q, (const T*)k, scale, ds,
                       dH, dq, dk, dm.Hq, dm.Hkv, dm.N);
  else
    hipLaunchKernelGGL((summary_bwd_kernel<T, 64>), grid, dim3(64), lds, st, (const T*)q, (const T*)k, scale, ds,
                       dH, dq, dk, dm.Hq, dm.Hkv, dm.N);
  return hipGetLastError();
}

hipError_t launch_chunk_summary_backward(const RouteDims& dm, const void* q, const void* k, float scale,
                                         const float* ds, const float* dH, float* dq, float* dk, hipStream_t st) {
  return dm.dtype == 1 ? launch_summary_bwd_t<bf16_t>(dm, q, k, scale, ds, dH, dq, dk, st)
                       : launch_summary_bwd_t<float>(dm, q, k, scale, ds, dH, dq, dk, st);
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


// ---------------------------------------------------------------- 5. scoring backward
// "Prefilling-dLLM v2", Figure 3 caption: the residual-augmented query
// q~ = q + (x A) B_h scores the summaries; "The 172x Speedup...": similarity minus
// beta times the pooling entropy. zsel[b,h,t,k] = scale q~ . s[b,h,c] - beta H[b,h,c]
// with c = idx[b,g,t,k] fixed, so for an upstream dzsel:
//   dq~[b,h,t] = scale sum_k dzsel s[c_k]            (added to dq at slot(i))
//   ds[b,h,c]  = scale sum over entries (t,k) of c of dzsel q~[b,h,t]
//   dH[b,h,c]  = -beta sum over the same entries of dzsel
//   dU = dq~ B^T (per row, over all heads), dB = U^T dq~, dA = x^T dU, dx = dU A^T
// All in float32 (ds as split-bf16 MFMA products, near float32). The sums over rows
// for ds, dA and dB are split into fixed row ranges whose partials are added in order
// (no atomics).

// dq~ as a dense product: dq~[b,h,t,:] = scale sum_c Z[t][c] s[b,h,c,:], Z the rows' dzsel
// scattered over chunks. One block per (64 rows, batch and head); the rows' entries are
// staged in LDS once; chunks go 32 at a time (a [64 x 32] Z tile and the 32 summaries
// as bf16 hi and lo planes); split-bf16 MFMA (three products, near float32). Writes dq~
// and adds it to dq at the rows' slots.
constexpr int kDqR = 64, kDqC = 32;

template <int D>
__global__ __launch_bounds__(256) void sbwd_dqt_dense_kernel(const int32_t* __restrict__ idx,
                                                             const float* __restrict__ dzsel,
                                                             const float* __restrict__ s, float* __restrict__ dqt,
                                                             float* __restrict__ dq, float scale, int Hq, int Hkv,
                                                             int N, int K, int q0, int nq) {
  constexpr int ZS = kDqC + 8, SS = D + 16;
  __shared__ short ei[kDqR * kMaxTopK];   // chunk indices (N <= 32768 on this path), -1 for none
  __shared__ float ew[kDqR * kMaxTopK];
  __shared__ float zf[kDqR * (kDqC + 1)];
  __shared__ __align__(16) bf16_t zp[2][kDqR * ZS];
  __shared__ __align__(16) bf16_t sp[2][kDqC * SS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, L16 = lane & 15, g16 = lane >> 4;
  const int bh = blockIdx.y, b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const int t0 = blockIdx.x * kDqR;
  for (int x = tid; x < kDqR * K; x += 256) {
    const int tl = x / K, k = x % K, t = t0 + tl;
    ei[x] = (short)(t < nq ? idx[(((size_t)b * Hkv + g) * nq + t) * K + k] : -1);
    ew[x] = t < nq ? dzsel[((size_t)bh * nq + t) * K + k] : 0.f;
  }
  f32x4 acc[D / 16];
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) acc[nt] = zero4();
  for (int c0 = 0; c0 < N; c0 += kDqC) {
    __syncthreads();
    for (int x = tid; x < kDqR * (kDqC + 1); x += 256) zf[x] = 0.f;
    for (int x = tid; x < kDqC * D / 4; x += 256) {
      const int cl = x / (D / 4), e = 4 * (x % (D / 4)), c = c0 + cl;
      f32x4 v = zero4();
      if (c < N) v = *reinterpret_cast<const f32x4*>(s + ((size_t)bh * N + c) * D + e);
      uint2 hi, lo;
      split4_bf16(v, hi, lo);
      *reinterpret_cast<uint2*>(&sp[0][cl * SS + e]) = hi;   // 8-byte aligned: SS and e are multiples of 4
      *reinterpret_cast<uint2*>(&sp[1][cl * SS + e]) = lo;
    }
    __syncthreads();
    for (int x = tid; x < kDqR * K; x += 256) {
      const int c = ei[x] - c0;
      if (c >= 0 && c < kDqC) zf[(x / K) * (kDqC + 1) + c] = ew[x];
    }
    __syncthreads();
    for (int x = tid; x < kDqR * kDqC; x += 256) {
      const int tl = x / kDqC, cl = x % kDqC;
      bf16_t hi, lo;
      split_bf16(zf[tl * (kDqC + 1) + cl], hi, lo);
      zp[0][tl * ZS + cl] = hi;
      zp[1][tl * ZS + cl] = lo;
    }
    __syncthreads();
    // wave w: rows 16 w .. 16 w + 15 (M) x all of d (N), k = the 32 chunks
    const s16x8 ah = load8(zp[0] + (16 * w + L16) * ZS + 8 * g16);
    const s16x8 al = load8(zp[1] + (16 * w + L16) * ZS + 8 * g16);
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const s16x8 bhi = lds_col_frag(sp[0], SS, 8 * g16, 8 * g16 + 4, 16 * nt, lane);
      const s16x8 blo = lds_col_frag(sp[1], SS, 8 * g16, 8 * g16 + 4, 16 * nt, lane);
      acc[nt] = mfma16(ah, blo, acc[nt]);
      acc[nt] = mfma16(al, bhi, acc[nt]);
      acc[nt] = mfma16(ah, bhi, acc[nt]);
    }
  }
  const size_t L = (size_t)N * kSlots;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * w + 4 * g16 + i;
    if (t >= nq) continue;
    float* dtr = dqt + ((size_t)bh * nq + t) * D;
    float* dqr = dq + ((size_t)bh * L + slot_of_c(q0 + t)) * D;
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const float v = scale * acc[nt][i];
      dtr[16 * nt + L16] = v;
      dqr[16 * nt + L16] += v;
    }
  }
}

// ds and dH as a dense product: ds[b,h,c,:] = sum_t Z[t][c] q~[b,h,t,:] with Z the chosen
// chunk logits' gradients scattered on a [32 rows x 64 chunks] LDS tile per step (zero where
// row t did not choose c). One block per (64 chunks, batch and head, row range); q~ is read
// once per block. Products in split bf16 (hi and lo planes, three MFMAs: near float32);
// dH takes the tile's column sums in row order. Each row range writes a partial; the
// partials are added in range order.
constexpr int kDsC = 64, kDsT = 32, kDsSplit = 8;

template <int D>
__global__ __launch_bounds__(256) void sbwd_ds_dense_kernel(const int32_t* __restrict__ idx,
                                                            const float* __restrict__ dzsel,
                                                            const float* __restrict__ qt, float* __restrict__ dspart,
                                                            float* __restrict__ dhpart, int BHq, int Hq, int Hkv,
                                                            int N, int K, int nq, int rows_per) {
  constexpr int ZS = kDsT + 8, QS = D + 16, FS = kDsT + 1;
  __shared__ __align__(16) bf16_t zt[2][kDsC * ZS];
  __shared__ __align__(16) bf16_t qp[2][kDsT * QS];
  __shared__ float zf[kDsC * FS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, L16 = lane & 15, g16 = lane >> 4;
  const int c0 = blockIdx.x * kDsC, bh = blockIdx.y, sp = blockIdx.z;
  const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const int tbeg = sp * rows_per, tend = min(nq, tbeg + rows_per);
  f32x4 acc[D / 16];
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) acc[nt] = zero4();
  float hs = 0.f;
  for (int t0 = tbeg; t0 < tend; t0 += kDsT) {
    __syncthreads();
    for (int x = tid; x < kDsC * FS; x += 256) zf[x] = 0.f;
    __syncthreads();
    for (int x = tid; x < kDsT * K; x += 256) {
      const int tl = x / K, k = x % K, row = t0 + tl;
      if (row < tend) {
        const int c = idx[(((size_t)b * Hkv + g) * nq + row) * K + k] - c0;
        if (c >= 0 && c < kDsC) zf[c * FS + tl] = dzsel[((size_t)bh * nq + row) * K + k];
      }
    }
    for (int x = tid; x < kDsT * D / 4; x += 256) {
      const int tl = x / (D / 4), e = 4 * (x % (D / 4)), row = t0 + tl;
      f32x4 v = zero4();
      if (row < tend) v = *reinterpret_cast<const f32x4*>(qt + ((size_t)bh * nq + row) * D + e);
      uint2 hi, lo;
      split4_bf16(v, hi, lo);
      *reinterpret_cast<uint2*>(&qp[0][tl * QS + e]) = hi;   // 8-byte aligned: QS and e are multiples of 4
      *reinterpret_cast<uint2*>(&qp[1][tl * QS + e]) = lo;
    }
    __syncthreads();
    for (int x = tid; x < kDsC * kDsT; x += 256) {
      const int c = x / kDsT, tl = x % kDsT;
      bf16_t hi, lo;
      split_bf16(zf[c * FS + tl], hi, lo);
      zt[0][c * ZS + tl] = hi;
      zt[1][c * ZS + tl] = lo;
    }
    if (tid < kDsC) {
      float cs = 0.f;
      for (int tl = 0; tl < kDsT; ++tl) cs += zf[tid * FS + tl];
      hs += cs;
    }
    __syncthreads();
    // wave w: chunks 16 w .. 16 w + 15 (M) x all of d (N), k = the 32 rows
    const s16x8 ah = load8(zt[0] + (16 * w + L16) * ZS + 8 * g16);
    const s16x8 al = load8(zt[1] + (16 * w + L16) * ZS + 8 * g16);
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const s16x8 bhi = lds_col_frag(qp[0], QS, 8 * g16, 8 * g16 + 4, 16 * nt, lane);
      const s16x8 blo = lds_col_frag(qp[1], QS, 8 * g16, 8 * g16 + 4, 16 * nt, lane);
      acc[nt] = mfma16(ah, blo, acc[nt]);
      acc[nt] = mfma16(al, bhi, acc[nt]);
      acc[nt] = mfma16(ah, bhi, acc[nt]);
    }
  }
  float* dst = dspart + ((size_t)sp * BHq + bh) * N * D;
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + 16 * w + 4 * g16 + i;
      if (c < N) dst[(size_t)c * D + 16 * nt + L16] = acc[nt][i];
    }
  if (tid < kDsC && c0 + tid < N) dhpart[((size_t)sp * BHq + bh) * N + c0 + tid] = hs;
}

__global__ __launch_bounds__(256) void sbwd_ds_reduce_kernel(const float* __restrict__ dspart,
                                                             const float* __restrict__ dhpart, float* __restrict__ ds,
                                                             float* __restrict__ dH, size_t nds, size_t ndh, float scale,
                                                             float beta) {
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < nds + ndh; x += (size_t)gridDim.x * 256) {
    float a = 0.f;
    if (x < nds) {
      for (int sp = 0; sp < kDsSplit; ++sp) a += dspart[(size_t)sp * nds + x];
      ds[x] = scale * a;
    } else {
      const size_t y = x - nds;
      for (int sp = 0; sp < kDsSplit; ++sp) a += dhpart[(size_t)sp * ndh + y];
      dH[y] = -beta * a;
    }
  }
}

// U[b,t,j] = sum of the u_kernel partials over the hidden-dimension splits
__global__ __launch_bounds__(256) void sbwd_usum_kernel(const float* __restrict__ upart, int nsplit, size_t n,
                                                        float* __restrict__ U) {
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) {
    float a = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) a += upart[(size_t)sp * n + x];
    U[x] = a;
  }
}

// Eight consecutive values of a row as split-bf16 MFMA operands (hi + lo); `n` of them valid.
template <typename T>
__device__ __forceinline__ void load8_split(const T* p, int n, s16x8& hi, s16x8& lo) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = j < n ? Elem<T>::to_f(p[j]) : 0.f;
  pack8_split_hw(v, hi, lo);
}

// dU[b,t,j] = sum_h sum_e dq~[b,h,t,e] Bm[j][h*D + e] on MFMA: one wave per 16 rows x RP
// columns, k over (head, e) in steps of 32. A = dq~ rows split into bf16 hi + lo; B = Bm
// rows (bf16 inputs: exact, two products; float32 inputs: split, three products).
template <typename T, int D, int RP>
__global__ __launch_bounds__(256) void sbwd_du_kernel(const float* __restrict__ dqt, const T* __restrict__ Bm, int r,
                                                      float* __restrict__ dU, int Hq, int nq, int ntiles) {
  const int lane = threadIdx.x & 63, L16 = lane & 15, g16 = lane >> 4;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= ntiles) return;
  const int ntb = (nq + 15) / 16, b = tile / ntb, t0 = (tile % ntb) * 16;
  const int t = min(t0 + L16, nq - 1);
  const bool tv = t0 + L16 < nq;
  f32x4 acc[RP / 16];
#pragma unroll
  for (int nt = 0; nt < RP / 16; ++nt) acc[nt] = zero4();
  for (int h = 0; h < Hq; ++h) {
    const float* arow = dqt + (((size_t)b * Hq + h) * nq + t) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      s16x8 ah, al;
      load8_split<float>(arow + 32 * ks + 8 * g16, tv ? 8 : 0, ah, al);
#pragma unroll
      for (int nt = 0; nt < RP / 16; ++nt) {
        const int j = 16 * nt + L16;
        const T* brow = Bm + (size_t)min(j, r - 1) * Hq * D + (size_t)h * D + 32 * ks + 8 * g16;
        if constexpr (sizeof(T) == 2) {
          const s16x8 bv = j < r ? load8(brow) : zero8();
          acc[nt] = mfma16(ah, bv, acc[nt]);
          acc[nt] = mfma16(al, bv, acc[nt]);
        } else {
          s16x8 bh, bl;
          load8_split<T>(brow, j < r ? 8 : 0, bh, bl);
          acc[nt] = mfma16(ah, bl, acc[nt]);
          acc[nt] = mfma16(al, bh, acc[nt]);
          acc[nt] = mfma16(ah, bh, acc[nt]);
        }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < RP / 16; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t0 + 4 * g16 + i;
      if (row < nq) dU[((size_t)b * nq + row) * RP + 16 * nt + L16] = acc[nt][i];
    }
}

// dx[b, slot(q0+t), m] = sum_j dU[b,t,j] A[m][j]: 64 rows x 256 hidden columns per block
template <typename T, int RP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RP <= 64 ? 4 : 2))) void sbwd_dx_kernel(
    const float* __restrict__ dU, const T* __restrict__ A, int Dh, int r, float* __restrict__ dx, int N, int q0,
    int nq) {
  // a block: 64 rows x 256 columns; a thread: one column, 4 rows at a time, so that
  // one 16-byte LDS read of dU feeds 4 FMAs; every output element still sums its r
  // products in rank order
  constexpr int TR = 64, CPT = 1;
  __shared__ __align__(16) float us[TR * RP];
  const int tid = threadIdx.x, b = blockIdx.z;
  const int t0 = blockIdx.x * TR, mb = blockIdx.y * 256 * CPT + tid;
  for (int x = tid; x < TR * RP; x += 256) {
    const int tt = t0 + x / RP;
    us[x] = tt < nq ? dU[((size_t)b * nq + tt) * RP + x % RP] : 0.f;
  }
  __syncthreads();
  if (mb >= Dh) return;
  float a[CPT][RP];
  // the thread's row of A: 16-byte loads when whole, aligned rows fill the padding
  constexpr int EV = 16 / sizeof(T);
  const bool vec = r == RP && ((uintptr_t)A & 15) == 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int m = mb + 256 * c;
    if (vec && m < Dh) {
      const T* ar = A + (size_t)m * RP;
#pragma unroll
      for (int j = 0; j < RP; j += EV) {
        T e[EV];
        *reinterpret_cast<uint4*>(e) = *reinterpret_cast<const uint4*>(ar + j);
#pragma unroll
        for (int i = 0; i < EV; ++i) a[c][j + i] = Elem<T>::to_f(e[i]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < RP; ++j) a[c][j] = (m < Dh && j < r) ? Elem<T>::to_f(A[(size_t)m * r + j]) : 0.f;
    }
  }
  const size_t L = (size_t)N * kSlots;
  const int tn = min(TR, nq - t0);
  for (int tl = 0; tl < tn; tl += 4) {   // rows tl .. tl + 3 < TR: past nq they are zero in LDS
    float acc[4][CPT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc[i][c] = 0.f;
#pragma unroll
    for (int j = 0; j < RP; j += 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(us + (tl + i) * RP + j);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          acc[i][c] += u[0] * a[c][j];
          acc[i][c] += u[1] * a[c][j + 1];
          acc[i][c] += u[2] * a[c][j + 2];
          acc[i][c] += u[3] * a[c][j + 3];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (tl + i >= tn) break;
      float* row = dx + ((size_t)b * L + slot_of_c(q0 + t0 + tl + i)) * Dh;
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        if (mb + 256 * c < Dh) row[mb + 256 * c] = acc[i][c];
    }
  }
}

// Partial dB over one range of rows: part[sp][j][col] = sum_rows U[row][j] dq~[b,h,t,e], col = h*D + e
template <int D, int RP>
__global__ __launch_bounds__(256) void sbwd_db_kernel(const float* __restrict__ U, const float* __restrict__ dqt,
                                                      float* __restrict__ part, int Hq, int nq, int rows_total,
                                                      int rows_per) {
  __shared__ float us[16 * RP];
  const int tid = threadIdx.x, sp = blockIdx.y;
  const int col = blockIdx.x * 256 + tid;
  const int HD = Hq * D;
  const int r0 = sp * rows_per, r1 = min(rows_total, r0 + rows_per);
  const int h = min(col, HD - 1) / D, e = min(col, HD - 1) % D;
  float acc[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) acc[j] = 0.f;
  for (int rb = r0; rb < r1; rb += 16) {
    __syncthreads();
    for (int x = tid; x < 16 * RP; x += 256) {
      const int row = rb + x / RP;
      us[x] = row < r1 ? U[(size_t)row * RP + x % RP] : 0.f;
    }
    __syncthreads();
    // the tile's 16 dq~ values in flight together; rows past r1 contribute nothing
    const int nr = min(16, r1 - rb);
    float dv[16];
#pragma unroll
    for (int tl = 0; tl < 16; ++tl) {
      const int row = rb + min(tl, nr - 1), b = row / nq, t = row % nq;
      dv[tl] = dqt[(((size_t)b * Hq + h) * nq + t) * D + e];
    }
#pragma unroll
    for (int tl = 0; tl < 16; ++tl) {
      if (tl >= nr) break;
#pragma unroll
      for (int j = 0; j < RP; ++j) acc[j] += us[tl * RP + j] * dv[tl];
    }
  }
  if (col < HD) {
#pragma unroll
    for (int j = 0; j < RP; ++j) part[((size_t)sp * RP + j) * HD + col] = acc[j];
  }
}

// Partial dA over one range of rows: part[sp][m][j] = sum_rows x[b, slot(q0+t), m] dU[row][j]
template <typename T, int RP>
__global__ __launch_bounds__(256) void sbwd_da_kernel(const T* __restrict__ x, const float* __restrict__ dU,
                                                      float* __restrict__ part, int Dh, int N, int q0, int nq,
                                                      int rows_total, int rows_per) {
  __shared__ float us[16 * RP];
  const int tid = threadIdx.x, sp = blockIdx.y;
  const int m = blockIdx.x * 256 + tid;
  const int r0 = sp * rows_per, r1 = min(rows_total, r0 + rows_per);
  const size_t L = (size_t)N * kSlots;
  float acc[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) acc[j] = 0.f;
  for (int rb = r0; rb < r1; rb += 16) {
    __syncthreads();
    for (int y = tid; y < 16 * RP; y += 256) {
      const int row = rb + y / RP;
      us[y] = row < r1 ? dU[(size_t)row * RP + y % RP] : 0.f;
    }
    __syncthreads();
    if (m < Dh) {
      // the tile's 16 x values in flight together; rows past r1 contribute nothing
      const int nr = min(16, r1 - rb);
      float xv[16];
#pragma unroll
      for (int tl = 0; tl < 16; ++tl) {
        const int row = rb + min(tl, nr - 1), b = row / nq, t = row % nq;
        xv[tl] = Elem<T>::to_f(x[((size_t)b * L + slot_of_c(q0 + t)) * Dh + m]);
      }
#pragma unroll
      for (int tl = 0; tl < 16; ++tl) {
        if (tl >= nr) break;
#pragma unroll
        for (int j = 0; j < RP; ++j) acc[j] += us[tl * RP + j] * xv[tl];
      }
    }
  }
  if (m < Dh) {
#pragma unroll
    for (int j = 0; j < RP; ++j) part[((size_t)sp * Dh + m) * RP + j] = acc[j];
  }
}

// dA[m][j] (j < r) and dB[j][col] (j < r) from the partials, added in split order
__global__ __launch_bounds__(256) void sbwd_reduce_kernel(const float* __restrict__ pa, const float* __restrict__ pb,
                                                          float* __restrict__ dA, float* __restrict__ dB, int nsp,
                                                          int Dh, int r, int RP, int HD) {
  const size_t na = (size_t)Dh * r, nb = (size_t)r * HD;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < na + nb; x += (size_t)gridDim.x * 256) {
    float a = 0.f;
    if (x < na) {
      const size_t m = x / r, j = x % r;
      for (int sp = 0; sp < nsp; ++sp) a += pa[((size_t)sp * Dh + m) * RP + j];
      dA[x] = a;
    } else {
      const size_t y = x - na, j = y / HD, col = y % HD;
      for (int sp = 0; sp < nsp; ++sp) a += pb[((size_t)sp * RP + j) * HD + col];
      dB[y] = a;
    }
  }
}

struct ScoreBwdWs {
  float *qt, *upart, *U, *dqt, *dU, *pa, *pb, *dsp, *dhp;
  int nsplit, RP, nsp, rows_per;
};

static int sbwd_nsp(int rows) { return std::max(1, std::min(64, (rows + 127) / 128)); }

static ScoreBwdWs sbwd_carve(void* ws, const RouteDims& dm, int Dh, int r, int K, int nq) {
  ScoreBwdWs o;
  o.nsplit = qtilde_u_splits(dm, Dh, nq);
  o.RP = qtilde_rank_pad(r);
  const int rows = dm.B * nq;
  o.nsp = sbwd_nsp(rows);
  o.rows_per = (rows + o.nsp - 1) / o.nsp;
  const size_t rh = (size_t)dm.B * dm.Hq * nq, bg = (size_t)dm.B * dm.Hkv;
  char* w = (char*)ws;
  auto take = [&](size_t bytes) { char* p = w; w += al256(bytes); return p; };
  o.qt = (float*)take(rh * dm.d * 4);
  o.dqt = (float*)take(rh * dm.d * 4);
  o.upart = (float*)take((size_t)o.nsplit * rows * o.RP * 4);
  o.U = (float*)take((size_t)rows * o.RP * 4);
  o.dU = (float*)take((size_t)rows * o.RP * 4);
  o.pa = (float*)take((size_t)o.nsp * Dh * o.RP * 4);
  o.pb = (float*)take((size_t)o.nsp * o.RP * dm.Hq * dm.d * 4);
  const size_t bhq = (size_t)dm.B * dm.Hq;
  o.dsp = (float*)take((size_t)kDsSplit * bhq * dm.N * dm.d * 4);
  o.dhp = (float*)take((size_t)kDsSplit * bhq * dm.N * 4);
  (void)bg;
  (void)K;
  return o;
}

size_t score_bwd_ws_bytes(const RouteDims& dm, int Dh, int r, int K, int nq) {
  const int nsplit = qtilde_u_splits(dm, Dh, nq), RP = qtilde_rank_pad(r), rows = dm.B * nq, nsp = sbwd_nsp(rows);
  const size_t rh = (size_t)dm.B * dm.Hq * nq, bg = (size_t)dm.B * dm.Hkv;
  const size_t bhq = (size_t)dm.B * dm.Hq;
  (void)bg;
  (void)K;
  return 2 * al256(rh * dm.d * 4) + al256((size_t)nsplit * rows * RP * 4) + 2 * al256((size_t)rows * RP * 4) +
         al256((size_t)nsp * Dh * RP * 4) + al256((size_t)nsp * RP * dm.Hq * dm.d * 4) +
         al256((size_t)kDsSplit * bhq * dm.N * dm.d * 4) + al256((size_t)kDsSplit * bhq * dm.N * 4);
}

template <typename T, int D, int RP>
static hipError_t launch_score_bwd_t(const RouteDims& dm, const void* x, const void* A, const void* Bm, int Dh, int r,
                                     const float* s, float beta, float scale, int K, int q0, int nq,
                                     const int32_t* idx, const float* dzsel, float* dq, float* dx, float* dA,
                                     float* dBm, float* ds, float* dH, const ScoreBwdWs& w, hipStream_t st) {
  const int rows = dm.B * nq;
  if (nq > 0) {
    hipLaunchKernelGGL((sbwd_dqt_dense_kernel<D>), dim3((nq + kDqR - 1) / kDqR, dm.B * dm.Hq), dim3(256), 0, st,
                       idx, dzsel, s, w.dqt, dq, scale, dm.Hq, dm.Hkv, dm.N, K, q0, nq);
  }
  {
    const int bhq = dm.B * dm.Hq;
    const int rows_per = ((nq + kDsSplit - 1) / kDsSplit + kDsT - 1) / kDsT * kDsT;
    hipLaunchKernelGGL((sbwd_ds_dense_kernel<D>), dim3((dm.N + kDsC - 1) / kDsC, bhq, kDsSplit), dim3(256), 0, st,
                       idx, dzsel, (const float*)w.qt, w.dsp, w.dhp, bhq, dm.Hq, dm.Hkv, dm.N, K, nq, rows_per);
    const size_t nds = (size_t)bhq * dm.N * D, ndh = (size_t)bhq * dm.N;
    hipLaunchKernelGGL(sbwd_ds_reduce_kernel, dim3((unsigned)std::min<size_t>((nds + ndh + 255) / 256, 65535)),
                       dim3(256), 0, st, (const float*)w.dsp, (const float*)w.dhp, ds, dH, nds, ndh, scale, beta);
  }
  if (nq > 0) {
    const size_t nu = (size_t)rows * RP;
    hipLaunchKernelGGL(sbwd_usum_kernel, dim3((unsigned)std::min<size_t>((nu + 255) / 256, 65535)), dim3(256), 0,
                       st, (const float*)w.upart, w.nsplit, nu, w.U);
    const int ntu = dm.B * ((nq + 15) / 16);
    hipLaunchKernelGGL((sbwd_du_kernel<T, D, RP>), dim3((ntu + 3) / 4), dim3(256), 0, st, (const float*)w.dqt,
                       (const T*)Bm, r, w.dU, dm.Hq, nq, ntu);
    hipLaunchKernelGGL((sbwd_dx_kernel<T, RP>), dim3((nq + 63) / 64, (Dh + 255) / 256, dm.B), dim3(256), 0, st,
                       (const float*)w.dU, (const T*)A, Dh, r, dx, dm.N, q0, nq);
  }
  const int HD = dm.Hq * D;
  hipLaunchKernelGGL((sbwd_db_kernel<D, RP>), dim3((HD + 255) / 256, w.nsp), dim3(256), 0, st, (const float*)w.U,
                     (const float*)w.dqt, w.pb, dm.Hq, nq, rows, w.rows_per);
  hipLaunchKernelGGL((sbwd_da_kernel<T, RP>), dim3((Dh + 255) / 256, w.nsp), dim3(256), 0, st, (const T*)x,
                     (const float*)w.dU, w.pa, Dh, dm.N, q0, nq, rows, w.rows_per);
  const size_t nred = (size_t)Dh * r + (size_t)r * HD;
  hipLaunchKernelGGL(sbwd_reduce_kernel, dim3((unsigned)std::min<size_t>((nred + 255) / 256, 65535)), dim3(256), 0,
                     st, (const float*)w.pa, (const float*)w.pb, dA, dBm, w.nsp, Dh, r, RP, HD);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_score_bwd_r(const RouteDims& dm, const void* x, const void* A, const void* Bm, int Dh, int r,
                                     const float* s, float beta, float scale, int K, int q0, int nq,
                                     const int32_t* idx, const float* dzsel, float* dq, float* dx, float* dA,
                                     float* dBm, float* ds, float* dH, const ScoreBwdWs& w, hipStream_t st) {
  if (w.RP == 32)
    return launch_score_bwd_t<T, D, 32>(dm, x, A, Bm, Dh, r, s, beta, scale, K, q0, nq, idx, dzsel, dq, dx, dA, dBm,
                                        ds, dH, w, st);
  if (w.RP == 64)
    return launch_score_bwd_t<T, D, 64>(dm, x, A, Bm, Dh, r, s, beta, scale, K, q0, nq, idx, dzsel, dq, dx, dA, dBm,
                                        ds, dH, w, st);
  return launch_score_bwd_t<T, D, 128>(dm, x, A, Bm, Dh, r, s, beta, scale, K, q0, nq, idx, dzsel, dq, dx, dA, dBm,
                                       ds, dH, w, st);
}

hipError_t launch_route_score_backward(const RouteDims& dm, const void* q, const void* x, const void* A,
                                       const void* Bm, int Dh, int r, const float* s, float beta, float scale, int K,
                                       int q0, int nq, const int32_t* idx, const float* dzsel, float* dq, float* dx,
                                       float* dA, float* dBm, float* ds, float* dH, void* ws, hipStream_t st) {
  const ScoreBwdWs w = sbwd_carve(ws, dm, Dh, r, K, nq);
  if (nq > 0) {
    hipError_t e = launch_qtilde_with_u(dm, q, x, A, Bm, Dh, r, w.qt, w.upart, q0, nq, st);
    if (e != hipSuccess) return e;
  }
  if (dm.dtype == 1)
    return dm.d == 128 ? launch_score_bwd_r<bf16_t, 128>(dm, x, A, Bm, Dh, r, s, beta, scale, K, q0, nq, idx, dzsel,
                                                         dq, dx, dA, dBm, ds, dH, w, st)
                       : launch_score_bwd_r<bf16_t, 64>(dm, x, A, Bm, Dh, r, s, beta, scale, K, q0, nq, idx, dzsel,
                                                        dq, dx, dA, dBm, ds, dH, w, st);
  return dm.d == 128 ? launch_score_bwd_r<float, 128>(dm, x, A, Bm, Dh, r, s, beta, scale, K, q0, nq, idx, dzsel, dq,
                                                      dx, dA, dBm, ds, dH, w, st)
                     : launch_score_bwd_r<float, 64>(dm, x, A, Bm, Dh, r, s, beta, scale, K, q0, nq, idx, dzsel, dq,
                                                     dx, dA, dBm, ds, dH, w, st);
}

// the inverse index (per chunk, the (query, slot) entries that selected it)
static hipError_t launch_bwd_index(const BwdParams& prm, hipStream_t st) {
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
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams& prm, hipStream_t st) {
  const size_t bgn = (size_t)prm.B * prm.Hkv * prm.N;
  hipError_t e = launch_bwd_index(prm, st);
  if (e != hipSuccess) return e;
  const int tiles = prm.B * prm.Hkv * ((prm.nq + 1) / 2);
  const size_t lds = routed_bwd_lds_bytes(D);
  e = hipFuncSetAttribute((const void*)bwd_query_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (tiles > 0) {
    if (bwd_query_pool_lds(D, prm.N) <= routed_lds_limit() &&
        (long long)prm.B * prm.Hq * prm.nq * prm.K < (1LL << 31)) {
      // consecutive queries share one chunk stream (the forward's pool)
      e = launch_bwd_query_pool(RouteDims{prm.B, prm.Hq, prm.Hkv, prm.N, D, 1}, prm.q, prm.k, prm.v, prm.o, prm.dO,
                                prm.idx, prm.zsel, prm.lse, prm.K, prm.R, prm.scale, prm.q0, prm.nq, prm.dq,
                                prm.dzsel, prm.dsum, prm.cbias, prm.cu, st);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(bwd_query_kernel<D>, dim3((tiles + 3) / 4), dim3(256), lds, st, prm);
    }
  }
  hipLaunchKernelGGL(bwd_key_kernel<D>, dim3((unsigned)bgn), dim3(256), 0, st, prm);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd32_d(const BwdParams& prm, hipStream_t st) {
  hipError_t e = launch_bwd_index(prm, st);
  if (e != hipSuccess) return e;
  if (prm.nq > 0) hipLaunchKernelGGL(bwd32_query_kernel<D>, dim3(prm.nq, prm.Hq, prm.B), dim3(256), 0, st, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd32_key_kernel<D>, dim3((unsigned)((size_t)prm.B * prm.Hkv * prm.N)), dim3(256), 0, st, prm);
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
  if (dm.dtype == 0) return dm.d == 128 ? launch_bwd32_d<128>(prm, st) : launch_bwd32_d<64>(prm, st);
  return dm.d == 128 ? launch_bwd_d<128>(prm, st) : launch_bwd_d<64>(prm, st);
}

}  // namespace lcr
