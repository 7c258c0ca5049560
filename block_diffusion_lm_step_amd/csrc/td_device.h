// Device helpers for the gfx950 kernels: bf16 conversion, MFMA fragments, wave reductions.
//
// MFMA fragment convention (16x16 output tiles, 64-wide wavefront).  For a product
// D[16][16] += A[16][K] * B[K][16], lane l holds the 8 contraction elements
// {8*(l/16) .. 8*(l/16)+7} of A row (l % 16) and of B column (l % 16), and receives
// D rows 4*(l/16) + r (r = 0..3) of column (l % 16).  Because A and B always use the
// same lane/slot -> k assignment, any bijection between (lane group, slot) and the 32
// contraction indices of one step gives the same sum; the kernels exploit this to pick
// k (or key) orders that make their loads contiguous.
//   bf16: one v_mfma_f32_16x16x32_bf16 per 32-wide step.
//   fp32: eight v_mfma_f32_16x16x4f32, slot j of every lane group forming step j.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "td_kernels.h"

using td::VStat;

typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

#define TD_DEV __device__ __forceinline__

TD_DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bfloat16, round to nearest, ties to even (gfx950 converts in hardware).
TD_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> TD_DEV float to_f32(T v);
template <> TD_DEV float to_f32<float>(float v) { return v; }
template <> TD_DEV float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> TD_DEV T from_f32(float v);
template <> TD_DEV float from_f32<float>(float v) { return v; }
template <> TD_DEV bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

// 16 bytes as a native vector: arrays of these stay in registers where arrays of the
// uint4 struct can end up in scratch.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Eight consecutive contraction elements held by one lane.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  uint4 raw;   // 8 bf16
  TD_DEV void zero() { raw = make_uint4(0, 0, 0, 0); }
  TD_DEV void load(const bf16_t *p) { raw = *reinterpret_cast<const uint4 *>(p); }
  // Streaming load (nontemporal hint): data read once per step, larger than the caches
  // (weights, K/V pages), is not kept where it would evict what is re-read.
  TD_DEV void load_nt(const bf16_t *p) {
    raw = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p)));
  }
  TD_DEV float get(int j) const {
    uint32_t w = (&raw.x)[j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  TD_DEV void set8(const float *v) {
    raw.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    raw.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    raw.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
    raw.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  }
  TD_DEV bf16x8_t vec() const { return __builtin_bit_cast(bf16x8_t, raw); }
};
template <> struct Frag<float> {
  float4 lo, hi;
  TD_DEV void zero() { lo = hi = make_float4(0.f, 0.f, 0.f, 0.f); }
  TD_DEV void load(const float *p) {
    lo = reinterpret_cast<const float4 *>(p)[0];
    hi = reinterpret_cast<const float4 *>(p)[1];
  }
  TD_DEV void load_nt(const float *p) {
    lo = __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p)));
    hi = __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p) + 1));
  }
  TD_DEV float get(int j) const { return j < 4 ? (&lo.x)[j] : (&hi.x)[j - 4]; }
  TD_DEV void set8(const float *v) {
    lo = make_float4(v[0], v[1], v[2], v[3]);
    hi = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// A fragment from / to its 16-byte words (bf16: 1 word, fp32: 2).
template <typename T> constexpr int frag_words() { return sizeof(T) / 2; }
TD_DEV Frag<bf16_t> frag_of(const u32x4_t *w, bf16_t) {
  Frag<bf16_t> f;
  f.raw = __builtin_bit_cast(uint4, w[0]);
  return f;
}
TD_DEV Frag<float> frag_of(const u32x4_t *w, float) {
  Frag<float> f;
  f.lo = __builtin_bit_cast(float4, w[0]);
  f.hi = __builtin_bit_cast(float4, w[1]);
  return f;
}

// acc += A(frag a) * B(frag b) over one 32-wide contraction step.
TD_DEV f32x4_t mma(const Frag<bf16_t> &a, const Frag<bf16_t> &b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.vec(), b.vec(), acc, 0, 0, 0);
}
TD_DEV f32x4_t mma(const Frag<float> &a, const Frag<float> &b, f32x4_t acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
  return acc;
}

// Activation fragment.  Activations are carried at fp32 precision: for the bf16 MFMA
// they are split into a bf16 high part and the bf16 rounding of the remainder
// (hi + lo keeps ~16 significant bits, relative error <= 2^-17), and both parts are
// multiplied into the same fp32 accumulator; the fp32 MFMA takes them as they are.
template <typename T> struct AFrag;
template <> struct AFrag<bf16_t> {
  Frag<bf16_t> hi, lo;
  TD_DEV void zero() { hi.zero(); lo.zero(); }
  TD_DEV void set8(const float *v) {
    hi.set8(v);
    float r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = v[j] - hi.get(j);
    lo.set8(r);
  }
};
template <> struct AFrag<float> {
  Frag<float> f;
  TD_DEV void zero() { f.zero(); }
  TD_DEV void set8(const float *v) { f.set8(v); }
};

// acc += activation(rows) x weight(columns)
TD_DEV f32x4_t mma_a(const AFrag<bf16_t> &a, const Frag<bf16_t> &w, f32x4_t acc) {
  acc = mma(a.hi, w, acc);
  return mma(a.lo, w, acc);
}
TD_DEV f32x4_t mma_a(const AFrag<float> &a, const Frag<float> &w, f32x4_t acc) { return mma(a.f, w, acc); }
// acc += weight-like(rows) x activation(columns)
TD_DEV f32x4_t mma_b(const Frag<bf16_t> &k, const AFrag<bf16_t> &q, f32x4_t acc) {
  acc = mma(k, q.hi, acc);
  return mma(k, q.lo, acc);
}
TD_DEV f32x4_t mma_b(const Frag<float> &k, const AFrag<float> &q, f32x4_t acc) { return mma(k, q.f, acc); }

TD_DEV f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- activation fragments in memory
// Fragment layout ("AFL") of GEMM inputs, as described in td_kernels.h: a GEMM loads each
// lane's MFMA operand with one 32-byte read and no conversion.
// Byte offset of the fragment holding element (row, k) of a matrix with KT k-tiles.
TD_DEV size_t afl_frag(int row, int k, int KT) {
  return ((size_t)((row >> 4) * KT + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (row & 15)) * 32;
}
template <typename T> TD_DEV void afl_put(void *buf, int KT, int row, int k, float v);
template <> TD_DEV void afl_put<bf16_t>(void *buf, int KT, int row, int k, float v) {
  char *f = reinterpret_cast<char *>(buf) + afl_frag(row, k, KT);
  const bf16_t hi = f2bf(v);
  const bf16_t lo = f2bf(v - bf2f(hi));
  reinterpret_cast<bf16_t *>(f)[k & 7] = hi;
  reinterpret_cast<bf16_t *>(f + 16)[k & 7] = lo;
}
template <> TD_DEV void afl_put<float>(void *buf, int KT, int row, int k, float v) {
  reinterpret_cast<float *>(reinterpret_cast<char *>(buf) + afl_frag(row, k, KT))[k & 7] = v;
}
// Elements k .. k+7 (k a multiple of 8) of one row: one whole fragment.
template <typename T> TD_DEV void afl_put8(void *buf, int KT, int row, int k, const float *v);
template <> TD_DEV void afl_put8<bf16_t>(void *buf, int KT, int row, int k, const float *v) {
  AFrag<bf16_t> f;
  f.set8(v);
  uint4 *p = reinterpret_cast<uint4 *>(reinterpret_cast<char *>(buf) + afl_frag(row, k, KT));
  p[0] = f.hi.raw;
  p[1] = f.lo.raw;
}
template <> TD_DEV void afl_put8<float>(void *buf, int KT, int row, int k, const float *v) {
  float4 *p = reinterpret_cast<float4 *>(reinterpret_cast<char *>(buf) + afl_frag(row, k, KT));
  p[0] = make_float4(v[0], v[1], v[2], v[3]);
  p[1] = make_float4(v[4], v[5], v[6], v[7]);
}
// Elements k .. k+3 (k a multiple of 4) of one row: half of a fragment's columns.
template <typename T> TD_DEV void afl_put4(void *buf, int KT, int row, int k, const float *v);
template <> TD_DEV void afl_put4<bf16_t>(void *buf, int KT, int row, int k, const float *v) {
  uint32_t hi[2], lo[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const bf16_t h0 = f2bf(v[2 * e]), h1 = f2bf(v[2 * e + 1]);
    hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lo[e] = (uint32_t)f2bf(v[2 * e] - bf2f(h0)) | ((uint32_t)f2bf(v[2 * e + 1] - bf2f(h1)) << 16);
  }
  char *f = reinterpret_cast<char *>(buf) + afl_frag(row, k, KT) + (k & 7) * 2;
  *reinterpret_cast<uint2 *>(f) = make_uint2(hi[0], hi[1]);
  *reinterpret_cast<uint2 *>(f + 16) = make_uint2(lo[0], lo[1]);
}
template <> TD_DEV void afl_put4<float>(void *buf, int KT, int row, int k, const float *v) {
  *reinterpret_cast<float4 *>(reinterpret_cast<char *>(buf) + afl_frag(row, k, KT) + (k & 7) * 4) =
      make_float4(v[0], v[1], v[2], v[3]);
}
template <typename T> TD_DEV AFrag<T> afl_get(const void *frag);
template <> TD_DEV AFrag<bf16_t> afl_get<bf16_t>(const void *frag) {
  AFrag<bf16_t> f;
  f.hi.raw = reinterpret_cast<const uint4 *>(frag)[0];
  f.lo.raw = reinterpret_cast<const uint4 *>(frag)[1];
  return f;
}
template <> TD_DEV AFrag<float> afl_get<float>(const void *frag) {
  AFrag<float> f;
  f.f.lo = reinterpret_cast<const float4 *>(frag)[0];
  f.f.hi = reinterpret_cast<const float4 *>(frag)[1];
  return f;
}

TD_DEV void load8f(const float *p, float *v) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Cross-lane reductions in registers, no LDS round trip.  Inside a row of 16 lanes the
// partner values come from DPP lane permutations: swap neighbours (quad_perm 1,0,3,2),
// swap pairs (2,3,0,1), reverse each half row (lane i <-> 7 - i), reverse the row
// (i <-> 15 - i); after the first k steps every lane holds the reduction over its aligned
// block of 2^k lanes.  Across rows, the gfx950 lane swaps return, for source = old = v,
// the even and the odd row of each 32-lane half (16-lane swap) or the lower and the
// upper half (32-lane swap) to every lane, combined as (first op second).  Partner lanes
// combine the same two operands in the same order, so every lane of a block ends with a
// bit-identical result.
template <int CTRL>
TD_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
TD_DEV int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_SWAP1 = 0xB1, DPP_SWAP2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

// Sum over aligned blocks of N lanes (N a power of two up to 64).
template <int N>
TD_DEV float sum_lanes(float v) {
  if constexpr (N >= 2) v += dpp_f<DPP_SWAP1>(v);
  if constexpr (N >= 4) v += dpp_f<DPP_SWAP2>(v);
  if constexpr (N >= 8) v += dpp_f<DPP_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp_f<DPP_MIRROR>(v);
  if constexpr (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (N >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}
TD_DEV float sum16(float v) { return sum_lanes<16>(v); }
TD_DEV float max16(float v) {
  v = fmaxf(v, dpp_f<DPP_SWAP1>(v));
  v = fmaxf(v, dpp_f<DPP_SWAP2>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp_f<DPP_MIRROR>(v));
}
TD_DEV int min16(int v) {
  v = min(v, dpp_i<DPP_SWAP1>(v));
  v = min(v, dpp_i<DPP_SWAP2>(v));
  v = min(v, dpp_i<DPP_HALF_MIRROR>(v));
  return min(v, dpp_i<DPP_MIRROR>(v));
}
// Over the four 16-lane rows, per lane position l % 16.
TD_DEV float sum_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
TD_DEV float max_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Merge of two softmax-statistics triples: exact for (max, index), fixed-order for the sum.
TD_DEV VStat vstat_merge(VStat x, VStat y) {
  VStat r;
  r.m = fmaxf(x.m, y.m);
  // exp(m - max) is 1 for the side that holds the max (also when both are -inf, the
  // empty set, so that the empty set stays the identity).
  float ex = (x.m == r.m) ? 1.0f : __expf(x.m - r.m);
  float ey = (y.m == r.m) ? 1.0f : __expf(y.m - r.m);
  r.s = x.s * ex + y.s * ey;
  r.a = (x.m > y.m) ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
  return r;
}

// Vocabulary statistics of one row over the NT column tiles its 16-lane group holds: lane
// l16 holds scaled score sv[j] of column col0 + 16 j.  The lane's own columns first, then
// one reduction each over the 16 lanes: the max, the sum of exp(sv - max), and the lowest
// column holding the max.  Every lane of the group takes part (live is uniform in it); a
// row that is not live gives the empty set (-inf, 0, none).
template <int NT>
TD_DEV VStat vstat_row16(const float (&sv)[NT], int col0, bool live) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NT; ++j) mx = fmaxf(mx, sv[j]);
  mx = max16(mx);
  float se = 0.f;
  int am = 0x7FFFFFFF;
#pragma unroll
  for (int j = NT - 1; j >= 0; --j) {   // descending: the lowest matching column wins
    if (live) {
      se += __expf(sv[j] - mx);
      if (sv[j] == mx) am = col0 + 16 * j;
    }
  }
  return VStat{mx, sum16(se), min16(am)};
}

TD_DEV float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// Exclusive position of each flagged row among the flagged rows, in row order.
// Called by every thread of one workgroup, once per chunk of blockDim.x rows; `row` < 0
// marks a thread past the end.  s_wave holds blockDim.x / 64 ints of LDS.  rowpos may be
// null (no inverse map kept).
TD_DEV int block_compact(bool flag, int base, int *rowlist, int *rowpos, int row, int *s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long mask = __ballot(flag);
  const int before = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(mask);
  __syncthreads();
  int off = base;
  for (int w = 0; w < wave; ++w) off += s_wave[w];
  int total = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) total += s_wave[w];
  if (flag) {
    rowlist[off + before] = row;
    if (rowpos) rowpos[row] = off + before;
  } else if (row >= 0 && rowpos) {
    rowpos[row] = -1;
  }
  __syncthreads();
  return base + total;
}
