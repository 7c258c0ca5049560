// Mixture-of-experts MLP at block-sized row counts (dzen.guru "NVIDIA Nemotron 70B
// генерирует текст…", section "Что нового": the tower's MoE layers activate 6 of 128
// experts plus 2 shared ones per token).
//
//   route    one wave per token row: the top_k experts of largest fp32 router score
//            (lowest id on ties) and gates = softmax over the chosen scores, plus the
//            row's RMSNorm scale; rows of a sequence whose block is already adopted are
//            not routed (their outputs are never read again);
//   bucket   one workgroup: counts per expert, padded segment offsets and the 16-row
//            tile table of the expert-sorted rows, then each (row, slot) placed in its
//            expert's segment; shared experts take every row in row order;
//   W1       per (tile, column group): the expert's up projection over the gathered
//            input rows, GELU, stored in fragment layout for W2;
//   W2       per (tile, column group): the expert's down projection, fp32;
//   combine  per row and column: x += sum_j gate_j * y(slot j) + sum_s y(shared s), in slot order,
//            then the next RMSNorm's partial sums of squares and x * gain in fragment
//            layout, as the dense MLP's down projection leaves them.
//
// At a block of rows most experts hold one or two rows, so the expert GEMMs stream the
// weights of every expert that holds a row once (the bound is HBM) with the layout and
// in-flight window of the dense weight-streaming GEMM: packed 16x32 weight tiles, K split
// over the waves, PASS k-tiles in flight per wave.  Rows of one tile are computed
// independently of each other (an output row reads only its input row), so where a row
// lands inside its expert's segment does not change any result bit; the placement uses
// LDS atomics and the sum over slots is in fixed order.
#include <algorithm>

#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

// (value, id) maximum: the larger value, the lower id among equal values.  A total
// order, so lanes that combine the same pair in either order agree.
TD_DEV void better(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}
template <int CTRL>
TD_DEV void better_dpp(float &v, int &i) {
  better(v, i, dpp_f<CTRL>(v), dpp_i<CTRL>(i));
}
// Over the whole wave; every lane ends with the winner.
TD_DEV void argmax_wave(float &v, int &i) {
  better_dpp<DPP_SWAP1>(v, i);
  better_dpp<DPP_SWAP2>(v, i);
  better_dpp<DPP_HALF_MIRROR>(v, i);
  better_dpp<DPP_MIRROR>(v, i);
  auto rv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  auto ri = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
  v = __uint_as_float(rv[0]);
  i = (int)ri[0];
  better(v, i, __uint_as_float(rv[1]), (int)ri[1]);
  rv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  ri = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
  v = __uint_as_float(rv[0]);
  i = (int)ri[0];
  better(v, i, __uint_as_float(rv[1]), (int)ri[1]);
}

constexpr int SPL = MOE_MAX_EXPERTS / 64;   // router scores per lane

// Routing of token row m by one wave; the chosen experts go to experts[m * top_k + j]
// (global memory, or LDS in the fused kernel).
TD_DEV void route_row(const MoeRoute &a, int m, int lane, int *experts) {
  if (a.seq_done[m / a.B]) {   // no routed expert for this row
    if (lane < a.top_k) experts[(size_t)m * a.top_k + lane] = -1;
    return;
  }
  float s[SPL];
#pragma unroll
  for (int c = 0; c < SPL; ++c) {
    const int e = lane + 64 * c;
    const float v = e < a.E ? a.scores[(size_t)m * a.Epad + e] : -INFINITY;
    s[c] = v == v ? v : -INFINITY;   // a NaN score is never preferred
  }
  float q = 0.f;
  for (int p = lane; p < a.d / 16; p += 64) q += a.ssq[(size_t)p * a.M + m];
  q = sum_lanes<64>(q);

  unsigned taken = 0;
  float sel[MOE_MAX_TOP_K];
  int ids[MOE_MAX_TOP_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
    if (j < a.top_k) {
      float v = -INFINITY;
      int id = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < SPL; ++c) {
        const int e = lane + 64 * c;
        if (e < a.E && !((taken >> c) & 1u)) better(v, id, s[c], e);
      }
      argmax_wave(v, id);   // top_k <= E: an untaken expert always exists
      sel[j] = v;
      ids[j] = id;
      if ((id & 63) == lane) taken |= 1u << (id >> 6);
    }
  }
  if (lane == 0) {
    float z = 0.f, w[MOE_MAX_TOP_K];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
      w[j] = j < a.top_k ? expf(sel[j] - sel[0]) : 0.f;
      z += w[j];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOP_K; ++j) {
      if (j < a.top_k) {
        experts[(size_t)m * a.top_k + j] = ids[j];
        a.gates[(size_t)m * a.top_k + j] = w[j] / z;
      }
    }
    a.rs[m] = 1.0f / sqrtf(q / (float)a.d + a.eps);
  }
}

__global__ __launch_bounds__(256) void moe_route_kernel(MoeRoute a) {
  if (*a.done) return;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m < a.M) route_row(a, m, threadIdx.x & 63, a.experts);
}

constexpr int NE_MAX = MOE_MAX_EXPERTS + MOE_MAX_SHARED;
constexpr int EPL = (NE_MAX + 63) / 64;   // experts per lane in the offset scan

// Counts, offsets, tile table and placement from the chosen experts [M][top_k]; called by
// all 1024 threads of one workgroup.
TD_DEV void bucket(const MoeRoute &a, const int *experts) {
  __shared__ int s_cnt[NE_MAX], s_seg[NE_MAX], s_tile[NE_MAX], s_cur[NE_MAX];
  const int tid = threadIdx.x;
  const int NE = a.E + a.n_shared, KS = a.top_k + a.n_shared;
  const int MK = a.M * a.top_k;
  for (int e = tid; e < NE; e += 1024) {
    s_cnt[e] = e < a.E ? 0 : a.M;
    s_cur[e] = 0;
  }
  __syncthreads();
  for (int i = tid; i < MK; i += 1024) {
    const int e = experts[i];
    if ((unsigned)e < (unsigned)a.E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  if (tid < 64) {   // exclusive scans of the padded rows and tiles over the experts
    int rows[EPL], tl[EPL];
    int rsum = 0, tsum = 0, act = 0;
#pragma unroll
    for (int c = 0; c < EPL; ++c) {
      const int e = tid * EPL + c;
      const int n = e < NE ? s_cnt[e] : 0;
      const int t = (n + 15) >> 4;
      rows[c] = rsum;
      tl[c] = tsum;
      rsum += 16 * t;
      tsum += t;
      act += n > 0;
    }
    int ir = rsum, it = tsum, ia = act;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int pr = __shfl_up(ir, o), pt = __shfl_up(it, o), pa = __shfl_up(ia, o);
      if (tid >= o) {
        ir += pr;
        it += pt;
        ia += pa;
      }
    }
#pragma unroll
    for (int c = 0; c < EPL; ++c) {
      const int e = tid * EPL + c;
      if (e < NE) {
        s_seg[e] = ir - rsum + rows[c];
        s_tile[e] = it - tsum + tl[c];
      }
    }
    if (tid == 63) {
      *a.n_tiles = it;
      if (a.stats) {
        a.stats[0] += 1;
        a.stats[1] += ia;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < NE; e += 1024) {
    const int n = s_cnt[e], t0 = s_tile[e], r0 = s_seg[e];
    for (int t = 0; 16 * t < n; ++t) a.tiles[t0 + t] = make_int4(e, r0 + 16 * t, min(16, n - 16 * t), 0);
    for (int r = n; r < ((n + 15) & ~15); ++r) a.src_row[r0 + r] = 0;
  }
  for (int i = tid; i < MK; i += 1024) {
    const int e = experts[i];
    if ((unsigned)e >= (unsigned)a.E) continue;
    const int m = i / a.top_k, j = i - m * a.top_k;
    const int p = s_seg[e] + atomicAdd(&s_cur[e], 1);
    a.src_row[p] = m;
    a.slot_pos[(size_t)m * KS + j] = p;
  }
  for (int i = tid; i < a.M * a.n_shared; i += 1024) {
    const int sh = i / a.M, m = i - sh * a.M;
    const int p = s_seg[a.E + sh] + m;
    a.src_row[p] = m;
    a.slot_pos[(size_t)m * KS + a.top_k + sh] = p;
  }
}

__global__ __launch_bounds__(1024) void moe_bucket_kernel(MoeRoute a) {
  if (*a.done) return;
  bucket(a, a.experts);
}

// Few rows: routing (16 waves, one row each in turn) and the bucket pass in one
// workgroup, one launch instead of two; the chosen experts stay in LDS.
constexpr int MOE_FUSED_ROWS = 64;
__global__ __launch_bounds__(1024) void moe_route_bucket_kernel(MoeRoute a) {
  __shared__ int s_exp[MOE_FUSED_ROWS * MOE_MAX_TOP_K];
  if (*a.done) return;
  for (int m = threadIdx.x >> 6; m < a.M; m += 16) route_row(a, m, threadIdx.x & 63, s_exp);
  __syncthreads();
  bucket(a, s_exp);
}

// k-tiles in flight per wave: one activation fragment and NT weight fragments per
// k-tile in a budget that keeps two workgroups of NW = 4 waves per CU.
template <typename T, int NT> constexpr int moe_pass() {
  constexpr int per = 8 + NT * (sizeof(T) == 2 ? 4 : 8);
  constexpr int p = 128 / per;
  return p > 16 ? 16 : (p < 1 ? 1 : p);
}

// Work items: (16-row tile of one expert, NT 16-column tiles), tile-major.  A grid of at
// most two workgroups per CU walks the live items (the tile count is known on the device
// only): item blockIdx.x, then every gridDim.x-th.  NW waves split K.  The next item's
// first PASS k-tiles are requested as soon as the current item's last MFMAs have read
// their registers, so the wave reduction and the epilogue overlap those loads.  UP: the
// gathered up projection with the row scale and GELU (W1); else the down projection of
// the sorted rows (W2).
template <typename T, int NT, int NW, bool UP>
__global__ __launch_bounds__(64 * NW) void moe_gemm_kernel(MoeGemm a) {
  constexpr int PASS = moe_pass<T, NT>();
  if (*a.done) return;
  const int ncg = a.N / (16 * NT);
  const int items = *a.n_tiles * ncg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int KT = a.K >> 5;
  const int kwt = (KT + NW - 1) / NW;
  const int kw0 = min(KT, wave * kwt), kw1 = min(KT, kw0 + kwt);
  auto clampk = [&](int kt) { return max(0, min(min(kt, kw1 - 1), KT - 1)); };

  __shared__ f32x4_t s_red[NW][NT][64];

  Frag<T> wb[PASS][NT];
  AFrag<T> xa[PASS];
  const T *Wl;
  const char *Al;
  int row0 = 0, nrows = 0, nt0 = 0;
  float rsv[4] = {1.f, 1.f, 1.f, 1.f};   // row scales of the 4 output rows a lane finishes (W1)
  // Requests the first PASS k-tiles of `item` and sets its addresses.
  auto issue = [&](int item) __attribute__((always_inline)) {
    const int t = item / ncg;
    nt0 = (item - t * ncg) * NT;
    const int4 tile = a.tiles[t];
    row0 = tile.y;
    nrows = tile.z;
    // Gathered row of this lane (W1) or the tile's own rows (W2).
    int srow = row0 + l16;
    if constexpr (UP) srow = a.src_row[row0 + l16];
    Wl = reinterpret_cast<const T *>(a.Wp) + (size_t)tile.x * a.N * a.K + ((size_t)nt0 * KT) * 512 + (size_t)lane * 8;
#pragma unroll
    for (int i = 0; i < PASS; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) wb[i][j].load_nt(Wl + ((size_t)j * KT + clampk(kw0 + i)) * 512);
    // Fragment (row, k-tile kt) of lane (g, l16) in fragment layout: ((row/16 * KT + kt)
    // * 64 + 16 g + row % 16) * 32 bytes.
    Al = reinterpret_cast<const char *>(a.A) + ((size_t)(srow >> 4) * KT * 64 + 16 * g + (srow & 15)) * 32;
#pragma unroll
    for (int i = 0; i < PASS; ++i) xa[i] = afl_get<T>(Al + (size_t)clampk(kw0 + i) * 2048);
    if constexpr (UP) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rsv[r] = a.rs[__shfl(srow, 4 * g + r)];
    }
  };

  int item = blockIdx.x;
  if (item < items) issue(item);
  for (; item < items; item += gridDim.x) {
    f32x4_t acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = zero4();
    int p0 = kw0;
    for (; p0 + PASS < kw1; p0 += PASS) {
#pragma unroll
      for (int i = 0; i < PASS; ++i) {
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = mma_a(xa[i], wb[i][j], acc[j]);
        const int k = clampk(p0 + PASS + i);
        xa[i] = afl_get<T>(Al + (size_t)k * 2048);
#pragma unroll
        for (int j = 0; j < NT; ++j) wb[i][j].load_nt(Wl + ((size_t)j * KT + k) * 512);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < PASS; ++i) {
      if (p0 + i < kw1) {
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = mma_a(xa[i], wb[i][j], acc[j]);
      }
    }
    // This item's epilogue needs its rows, column tiles and row scales; then the next
    // item's loads go out.
    const int row0c = row0, nrowsc = nrows, nt0c = nt0;
    float rsc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rsc[r] = rsv[r];
    __builtin_amdgcn_sched_barrier(0);
    if (item + (int)gridDim.x < items) issue(item + gridDim.x);

#pragma unroll
    for (int j = 0; j < NT; ++j) s_red[wave][j][lane] = acc[j];
    __syncthreads();
    if (wave < NT) {
      const int j = wave;   // wave j finishes column tile j, summing the waves in order
      f32x4_t y4 = s_red[0][j][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) y4 += s_red[w][j][lane];
      const int col = (nt0c + j) * 16 + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ri = 4 * g + r;
        if constexpr (UP) {
          afl_put<T>(a.out_afl, a.N >> 5, row0c + ri, col, gelu_erf(y4[r] * rsc[r]));
        } else {
          if (ri < nrowsc) a.out[(size_t)(row0c + ri) * a.N + col] = y4[r];
        }
      }
    }
    __syncthreads();   // s_red is rewritten by the next item
  }
}

// One workgroup per (row, 256 columns), one column per thread.  The row's slot
// positions and gates are workgroup-uniform (scalar loads, read once).
template <typename T>
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeCombine a) {
  if (*a.done) return;
  const int m = blockIdx.x;
  if (a.seq_done[m / a.B]) return;
  const int KS = a.top_k + a.n_shared;
  int pos[MOE_MAX_TOP_K + MOE_MAX_SHARED];
  float gt[MOE_MAX_TOP_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K + MOE_MAX_SHARED; ++j) pos[j] = j < KS ? a.slot_pos[(size_t)m * KS + j] : 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j) gt[j] = j < a.top_k ? a.gates[(size_t)m * a.top_k + j] : 0.f;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= a.d) return;   // whole 16-column groups (d is a multiple of 64)
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOP_K; ++j)
    if (j < a.top_k) acc += gt[j] * a.y[(size_t)pos[j] * a.d + c];
#pragma unroll
  for (int s = 0; s < MOE_MAX_SHARED; ++s)
    if (s < a.n_shared) acc += a.y[(size_t)pos[a.top_k + s] * a.d + c];
  const float xv = a.x[(size_t)m * a.d + c] + acc;
  a.x[(size_t)m * a.d + c] = xv;
  afl_put<T>(a.out_afl, a.d >> 5, m, c, xv * to_f32<T>(reinterpret_cast<const T *>(a.gain_next)[c]));
  const float sq = sum16(xv * xv);
  if ((threadIdx.x & 15) == 0) a.ssq_out[(size_t)(c >> 4) * a.M + m] = sq;
}

}  // namespace

hipError_t launch_moe_route(const MoeRoute &a, hipStream_t s) {
  if (a.M <= 0 || a.E < 1 || a.E > MOE_MAX_EXPERTS || a.top_k < 1 || a.top_k > MOE_MAX_TOP_K || a.top_k > a.E ||
      a.n_shared < 0 || a.n_shared > MOE_MAX_SHARED || a.Epad < a.E || a.d % 16 || !a.done || !a.seq_done ||
      a.B < 1 || a.M % a.B)
    return hipErrorInvalidValue;
  if (a.M <= MOE_FUSED_ROWS) {
    hipLaunchKernelGGL(moe_route_bucket_kernel, dim3(1), dim3(1024), 0, s, a);
  } else {
    hipLaunchKernelGGL(moe_route_kernel, dim3((a.M + 3) / 4), dim3(256), 0, s, a);
    hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(1024), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_moe_gemm(int dtype, bool up, const MoeGemm &a, hipStream_t s) {
  constexpr int NT = 2, NW = 4;
  if (a.N % (16 * NT) || a.K % 32 || a.max_tiles <= 0 || !a.done || !a.n_tiles || !a.tiles) return hipErrorInvalidValue;
  if (up ? (!a.src_row || !a.rs || !a.out_afl) : !a.out) return hipErrorInvalidValue;
  // Two workgroups per CU (the register budget of the in-flight window), all resident.
  const int64_t max_items = (int64_t)a.max_tiles * (a.N / (16 * NT));
  const dim3 grid((unsigned)std::min<int64_t>(max_items, 512));
  if (dtype == DT_BF16) {
    if (up) hipLaunchKernelGGL((moe_gemm_kernel<bf16_t, NT, NW, true>), grid, dim3(64 * NW), 0, s, a);
    else hipLaunchKernelGGL((moe_gemm_kernel<bf16_t, NT, NW, false>), grid, dim3(64 * NW), 0, s, a);
  } else {
    if (up) hipLaunchKernelGGL((moe_gemm_kernel<float, NT, NW, true>), grid, dim3(64 * NW), 0, s, a);
    else hipLaunchKernelGGL((moe_gemm_kernel<float, NT, NW, false>), grid, dim3(64 * NW), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_moe_combine(int dtype, const MoeCombine &a, hipStream_t s) {
  if (a.M <= 0 || a.d % 64 || !a.done || !a.seq_done || a.B < 1 || a.M % a.B) return hipErrorInvalidValue;
  const dim3 grid(a.M, (a.d + 255) / 256);
  if (dtype == DT_BF16) hipLaunchKernelGGL(moe_combine_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(moe_combine_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace td
