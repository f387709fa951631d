// Device helpers shared by the gfx950 kernels: bf16 conversion and splitting,
// 16x16x32 bf16 MFMA fragments, LDS transpose reads, wave reductions.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (lane l of a 64-wide wave):
//   A[m][k]: lane l holds m = l%16, k = 8*(l/16) + j (j = 0..7)
//   B[k][n]: lane l holds n = l%16, k = 8*(l/16) + j
//   D[m][n]: lane l holds n = l%16, m = 4*(l/16) + i (i = 0..3)
// Only the M/N/D placement matters for correctness: A and B share the same
// lane -> k assignment, so any consistent permutation of k is a valid product.
//
// ds_read_b64_tr_b16: within each 16-lane group, lane L supplies an 8-byte
// address; lane L receives element (L%4) of the row addressed by lane
// 4*j + L/4 as its j-th 16-bit value (j = 0..3). Supplying, from lane L, the
// address of M[k0 + L/4][n0 + 4*(L%4)] gives lane L the column
// M[k0 .. k0+3][n0 + L] of a row-major (n-contiguous) tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcr {

typedef uint16_t bf16_t;
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kSlots = 64;
constexpr int kContent = 63;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;

// Workgroups are handed to the 8 XCDs of the chip round-robin by linear block
// id, and each XCD has its own L2. xcd_tile maps a 1-D grid of xcd_grid(total)
// blocks onto `total` tiles so that XCD x runs the contiguous tile range
// [x * per, (x + 1) * per) in order: tiles enumerated batch-head-major then keep
// one head's K and V in the L2 of one or two XCDs instead of all eight.
constexpr int kXcds = 8;
__host__ __device__ __forceinline__ int xcd_per(int total) { return (total + kXcds - 1) / kXcds; }
__host__ __device__ __forceinline__ int xcd_grid(int total) { return xcd_per(total) * kXcds; }
// reversed != 0 walks the tiles in the opposite order (same blocks, same XCD
// ranges mirrored): results do not depend on it, which tests check.
__device__ __forceinline__ int xcd_tile(int total, int reversed = 0) {   // tile of this block, or -1
  const int bid = blockIdx.x;
  const int l = (bid % kXcds) * xcd_per(total) + bid / kXcds;
  return l < total ? (reversed ? total - 1 - l : l) : -1;
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits in total.
__device__ __forceinline__ void split_bf16(float x, bf16_t& hi, bf16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  static __device__ __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4 mfma16(s16x8 a, s16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Pack 8 floats (bf16-rounded) into an operand fragment.
__device__ __forceinline__ s16x8 pack8(const float* v) {
  s16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (short)f2bf(v[j]);
  return r;
}

// Two floats -> packed bf16x2 (v_cvt_pk_bf16_f32, round to nearest even).
typedef __bf16 hbf16x2 __attribute__((ext_vector_type(2)));
typedef float hf32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(hf32x2{a, b}, hbf16x2));
}

// Four floats x -> hi = bf16(x) and lo = bf16(x - hi) as two 8-byte groups (element
// 0 in the low half of the first word), conversions two values per instruction.
__device__ __forceinline__ void split4_bf16(const f32x4& v, uint2& hi, uint2& lo) {
  const uint32_t h01 = pack2_bf16(v[0], v[1]), h23 = pack2_bf16(v[2], v[3]);
  hi = make_uint2(h01, h23);
  lo = make_uint2(pack2_bf16(v[0] - __uint_as_float(h01 << 16), v[1] - __uint_as_float(h01 & 0xFFFF0000u)),
                  pack2_bf16(v[2] - __uint_as_float(h23 << 16), v[3] - __uint_as_float(h23 & 0xFFFF0000u)));
}

// Two groups of four floats -> eight bf16 (a, then b; round to nearest even, two
// values per instruction): an MFMA operand formed from two 16-row output tiles.
__device__ __forceinline__ s16x8 pack8_bf16(const float* a, const float* b) {
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  u32x4 w;
  w[0] = pack2_bf16(a[0], a[1]);
  w[1] = pack2_bf16(a[2], a[3]);
  w[2] = pack2_bf16(b[0], b[1]);
  w[3] = pack2_bf16(b[2], b[3]);
  return __builtin_bit_cast(s16x8, w);
}

// Eight floats x -> hi = bf16(x) and lo = bf16(x - hi), 16 significant bits in total,
// with the round-to-nearest-even conversions done by v_cvt_pk_bf16_f32 (two values per
// instruction).
__device__ __forceinline__ void pack8_split_hw(const float* v, s16x8& hi, s16x8& lo) {
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  u32x4 h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t hp = pack2_bf16(v[2 * j], v[2 * j + 1]);
    h[j] = hp;
    const float h0 = __uint_as_float(hp << 16), h1 = __uint_as_float(hp & 0xFFFF0000u);
    l[j] = pack2_bf16(v[2 * j] - h0, v[2 * j + 1] - h1);
  }
  hi = __builtin_bit_cast(s16x8, h);
  lo = __builtin_bit_cast(s16x8, l);
}

// 16-byte load of 8 bf16 values (any address space the compiler can see).
__device__ __forceinline__ s16x8 load8(const bf16_t* p) { return *reinterpret_cast<const s16x8*>(p); }

// ---------------------------------------------------------------- LDS transpose read

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 ds_read_tr(const bf16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr));
}

// Operand fragment for k-index slots (8*(l/16)+j) from a row-major LDS tile
// M[k][n] (n contiguous, row stride `ld` elements, 8-byte aligned rows):
// lane l receives M[k_lo + j][n0 + l%16] for j = 0..3 and M[k_hi + j][n0 + l%16]
// for j = 4..7, where k_lo/k_hi are chosen by the caller per 16-lane group.
__device__ __forceinline__ s16x8 lds_col_frag(const bf16_t* tile, int ld, int k_lo, int k_hi, int n0,
                                              int lane) {
  const int L = lane & 15;
  const bf16_t* p0 = tile + (k_lo + (L >> 2)) * ld + n0 + 4 * (L & 3);
  const bf16_t* p1 = tile + (k_hi + (L >> 2)) * ld + n0 + 4 * (L & 3);
  s16x4 a = ds_read_tr(p0);
  s16x4 b = ds_read_tr(p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Reduction over the four lanes {l%16 + 16*g}: they share one MFMA output column.
// v_permlane16_swap / v_permlane32_swap exchange 16-lane rows (resp. 32-lane
// halves) between two registers; with both operands equal, element 0 and 1 of
// the result hold, in every lane, the value of the lane itself and of its
// partner l^16 (resp. l^32), in some order. Plain VALU, no LDS round trip.
// Maxima use the NaN-propagating IEEE maximum (v_maximum3_f32 on gfx950): the
// reductions here only see finite values and -inf masks, and unlike fmaxf it
// needs no canonicalisation of MFMA results.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return max2(a, max2(b, c)); }
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float col_max(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float col_sum(float v) { return xor32_sum(xor16_sum(v)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }   // normal x only

// ---------------------------------------------------------------- wait counters

// s_waitcnt lgkmcnt(0): every LDS (and scalar memory) operation of this wave has completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8)); }

// s_waitcnt that waits for vector-memory operations only: at most n outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Order-preserving map float -> uint32 (larger float -> larger key); 0 is
// reserved for "not a candidate" and never produced by a finite float.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k == 0u ? 1u : k;
}

}  // namespace lcr
