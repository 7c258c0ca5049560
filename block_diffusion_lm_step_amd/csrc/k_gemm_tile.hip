// Tiled MFMA GEMM for many rows (batches of sequences): Y[M][N] = A[M][K] * W[N][K]^T.
//
// At M >= 128 every weight element is used by many rows and the projections are bound
// by the matrix cores, not by the weight stream.  A workgroup of 4 waves computes a
// BM x 128 output tile; wave (wm, wn) owns a (BM/2) x 64 quarter ((BM/32) x 4 MFMA tiles
// of 16 x 16).  BM = 128, or 64 for layer projections whose 128-row tiles would give
// about one workgroup per CU: that leaves each SIMD a single wave, whose LDS and barrier
// latencies nothing overlaps (measured: the MFMA pipes were busy 22% of such a launch).  K advances one 32-wide k-tile per stage through double-buffered LDS (48 KiB,
// so two workgroups share a CU and one's LDS traffic overlaps the other's MFMAs), one
// barrier per stage: the next stage is loaded from memory into registers while the
// current one is multiplied, then written to the other buffer.
// Both operands are already in MFMA fragment order in memory (weights packed at
// creation, activations written in fragment layout by their producers), so staging is
// a straight 16-byte copy; the activation fragments' bf16 high and low halves go to two
// separate LDS planes so that a wave's 16-byte LDS reads are contiguous (no bank
// conflicts).  Per k-tile and wave: 8 activation + 4 weight fragment reads from LDS,
// 32 MFMAs (high and low parts of the activations against the bf16 weights).
//
// Epilogues as in the weight-streaming kernels (the RMSNorm row scale multiplies the
// accumulator): STORE (q/k/v), GELU and RESID (fragment-layout outputs, partial sums of
// squares per 16 columns), and VSTAT for the LM head (rows gathered through the row
// list; per row one (max, sum of exp, argmax) triple per 128-column group).
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

constexpr int BN = 128;             // workgroup tile columns
constexpr int KS = 1;               // k-tiles per stage
constexpr int NTW = 4;              // MFMA column tiles per wave
constexpr int NFW = (BN / 16) * KS * 64 / 256;   // weight fragments staged per thread

// Small per-thread tables are vector values, not arrays: arrays indexed in loops are
// turned into LDS or scratch copies before the loops are unrolled.
typedef unsigned long long u64x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int BM>
struct alignas(16) StageLds {
  u32x4_t a_hi[BM / 16][KS][64];   // activation fragments, bf16 high parts
  u32x4_t a_lo[BM / 16][KS][64];   // ... bf16 remainders
  u32x4_t w[BN / 16][KS][64];      // weight fragments
};

constexpr int EPI_PART = 100;   // split-K partial: store the raw accumulator tile

template <int EPI, bool NORM, int BM>
__global__ __launch_bounds__(256, 2) void gemm_tile_kernel(GemmArgs a) {
  constexpr int MTW = BM / 32;                     // MFMA row tiles per wave
  constexpr int NFA = (BM / 16) * KS * 64 / 256;   // activation fragments staged per thread
  constexpr int NPAR = 256 / BM;                   // threads per row summing squares
  __shared__ StageLds<BM> s_st[2];
  __shared__ int s_row[BM];
  __shared__ float s_rs[BM];
  __shared__ float s_part[NPAR][BM];
  __shared__ VStat s_stat[2][BM];

  // The loop-exit flag is loaded before any operand: issued behind the operand stream it
  // would queue with it and hold back the first MFMAs; it is tested once the first
  // operand loads are in flight.
  const int stop = __hip_atomic_load(a.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // a vector load
  __builtin_amdgcn_sched_barrier(0);
  const int nrows = a.n_rows ? *a.n_rows : a.M;   // live rows (LM head: masked rows)
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  if (m0 >= nrows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  // K range of this workgroup: split blockIdx.z of a.splits (whole k-tiles).
  const int KTall = a.K >> 5;
  const int kt0 = (int)((int64_t)KTall * blockIdx.z / a.splits), kt1 = (int)((int64_t)KTall * (blockIdx.z + 1) / a.splits);
  const int KT = KTall, nstage = (kt1 - kt0) / KS;

  // Activation rows of this tile (gathered through the row list for the LM head);
  // rows past the live count read a valid row and are never written.
  if (threadIdx.x < BM) {
    const int i = min(m0 + threadIdx.x, nrows - 1);
    s_row[threadIdx.x] = a.rowlist ? a.rowlist[i] : i;
  }
  __syncthreads();

  // Staging: each thread moves NFA activation fragments (32 B) and NFW weight fragments
  // (16 B) per stage; fragment f = threadIdx.x + 256 i covers (tile f / (64 KS), k-tile
  // (f / 64) % KS, lane f % 64).  Source offsets of stage 0; stage s adds s * KS k-tiles.
  const char *Ab = reinterpret_cast<const char *>(a.A);
  const bf16_t *Wb = reinterpret_cast<const bf16_t *>(a.Wp);
  u64x4_t aoff, woff;
#pragma unroll
  for (int i = 0; i < NFA; ++i) {
    const int f = threadIdx.x + 256 * i;
    const int fl = f & 63, kt = (f >> 6) % KS, t = f / (64 * KS);
    const int row = s_row[t * 16 + (fl & 15)];
    aoff[i] = (((size_t)(row >> 4) * KT + kt0 + kt) * 64 + (fl >> 4) * 16 + (row & 15)) * 32;
  }
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    const int f = threadIdx.x + 256 * i;
    const int fl = f & 63, kt = (f >> 6) % KS, t = f / (64 * KS);
    woff[i] = (((size_t)(n0 / 16 + t) * KT + kt0 + kt) * 64 + fl) * 8;
  }
  // (tile, k-tile) of fragment i = 0; fragment i is 4 / KS tiles further.
  const int ft = threadIdx.x / (64 * KS), fkt = (threadIdx.x >> 6) % KS;
  u32x4_t ra_hi[NFA], ra_lo[NFA], rw[NFW];
#define TD_LOAD_STAGE(S)                                                                        \
  _Pragma("unroll") for (int i = 0; i < NFA; ++i) {                                             \
    const u32x4_t *p_ = reinterpret_cast<const u32x4_t *>(Ab + aoff[i] + (size_t)(S) * KS * 2048); \
    ra_hi[i] = p_[0];                                                                           \
    ra_lo[i] = p_[1];                                                                           \
  }                                                                                             \
  _Pragma("unroll") for (int i = 0; i < NFW; ++i)                                               \
    rw[i] = *reinterpret_cast<const u32x4_t *>(Wb + woff[i] + (size_t)(S) * KS * 512);
#define TD_STORE_STAGE(B)                                                                       \
  _Pragma("unroll") for (int i = 0; i < NFA; ++i) {                                             \
    s_st[B].a_hi[ft + (4 / KS) * i][fkt][lane] = ra_hi[i];                                      \
    s_st[B].a_lo[ft + (4 / KS) * i][fkt][lane] = ra_lo[i];                                      \
  }                                                                                             \
  _Pragma("unroll") for (int i = 0; i < NFW; ++i) s_st[B].w[ft + (4 / KS) * i][fkt][lane] = rw[i];

  TD_LOAD_STAGE(0)
  asm volatile("" ::: "memory");   // the loads above are issued before the test below
  if (stop) return;
  if constexpr (NORM && EPI != EPI_PART) {
    // Row scales from the producer's partial sums of squares: thread t sums the parts
    // p = t / BM (mod NPAR) of row t % BM (consecutive threads read consecutive rows).
    const int r = threadIdx.x & (BM - 1), par = threadIdx.x / BM;
    const int row = s_row[r];
    float sacc = 0.f;
    for (int p0 = par; p0 < a.norm_nparts; p0 += NPAR * 16) {
      f32x16_t v;
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = a.ssq[(size_t)min(p0 + NPAR * j, a.norm_nparts - 1) * a.ld_ssq + row];
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc += (p0 + NPAR * j < a.norm_nparts) ? v[j] : 0.f;
    }
    s_part[par][r] = sacc;
  }
  TD_STORE_STAGE(0)
  __syncthreads();
  if constexpr (NORM && EPI != EPI_PART) {
    if (threadIdx.x < BM) {
      float q = 0.f;
#pragma unroll
      for (int p = 0; p < NPAR; ++p) q += s_part[p][threadIdx.x];
      s_rs[threadIdx.x] = 1.0f / sqrtf(q / (float)a.K + a.norm_eps);
    }
  }

  f32x4_t acc[MTW][NTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = zero4();

  for (int s = 0; s < nstage; ++s) {
    const int b = s & 1;
    if (s + 1 < nstage) {
      TD_LOAD_STAGE(s + 1)
    }
#pragma unroll
    for (int kt = 0; kt < KS; ++kt) {
      AFrag<bf16_t> af[MTW];
      Frag<bf16_t> wf[NTW];
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        af[i].hi.raw = __builtin_bit_cast(uint4, s_st[b].a_hi[wm * MTW + i][kt][lane]);
        af[i].lo.raw = __builtin_bit_cast(uint4, s_st[b].a_lo[wm * MTW + i][kt][lane]);
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j) wf[j].raw = __builtin_bit_cast(uint4, s_st[b].w[wn * NTW + j][kt][lane]);
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = mma_a(af[i], wf[j], acc[i][j]);
    }
    if (s + 1 < nstage) {   // the other buffer was last read in stage s - 1
      if (b) {
        TD_STORE_STAGE(0)
      } else {
        TD_STORE_STAGE(1)
      }
    }
    __syncthreads();
  }

#undef TD_LOAD_STAGE
#undef TD_STORE_STAGE

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == EPI_PART) {
    float *part = a.part + (size_t)blockIdx.z * a.M * a.N;
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int col = n0 + (wn * NTW + j) * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + (wm * MTW + i) * 16 + 4 * g + r;
          if (row < a.M) part[(size_t)row * a.N + col] = acc[i][j][r];
        }
      }
  } else if constexpr (EPI == EPI_VSTAT) {
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ri = (wm * MTW + i) * 16 + 4 * g + r;
        const bool live = m0 + ri < nrows;
        const int row = s_row[ri];
        const float rs = s_rs[ri];
        const float tau = (live && a.inv_temp) ? a.inv_temp[row] : 1.0f;
        VStat v{-INFINITY, 0.f, 0x7FFFFFFF};
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int col = n0 + (wn * NTW + j) * 16 + l16;
          const float z = acc[i][j][r] * rs;
          float sv = -INFINITY;
          if (live) {
            if (a.logits) a.logits[(size_t)row * a.N + col] = z;
            sv = tau * z;
          }
          float mx = sv;
          mx = max16(mx);
          const float se = sum16(live ? __expf(sv - mx) : 0.f);
          int am = (live && sv == mx) ? col : 0x7FFFFFFF;
          am = min16(am);
          v = vstat_merge(v, VStat{mx, se, am});
        }
        if (l16 == 0) s_stat[wn][ri] = v;
      }
    __syncthreads();
    if (threadIdx.x < BM && m0 + threadIdx.x < nrows)
      a.vpart[(size_t)(m0 + threadIdx.x) * gridDim.x + blockIdx.x] = vstat_merge(s_stat[0][threadIdx.x], s_stat[1][threadIdx.x]);
  } else {
    const int M = a.M;
    const int KTo = a.N >> 5;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int col = n0 + (wn * NTW + j) * 16 + l16;
      float gnext = 1.0f;
      f32x16_t xold;   // [i * 4 + r]
      if constexpr (EPI == EPI_RESID) {
        gnext = to_f32<bf16_t>(reinterpret_cast<const bf16_t *>(a.gain_next)[col]);
#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            xold[i * 4 + r] = a.out[(size_t)min(m0 + (wm * MTW + i) * 16 + 4 * g + r, M - 1) * a.ldo + col];
      }
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ri = (wm * MTW + i) * 16 + 4 * g + r;
          const int row = m0 + ri;
          const bool ok = row < M;
          float y = acc[i][j][r];
          if constexpr (NORM) y *= s_rs[ri];
          if constexpr (EPI == EPI_STORE) {
            if (ok) a.out[(size_t)row * a.ldo + col] = y;
          } else if constexpr (EPI == EPI_GELU) {
            if (ok) afl_put<bf16_t>(a.out_afl, KTo, row, col, gelu_erf(y));
          } else {
            const float xv = ok ? xold[i * 4 + r] + y : 0.f;
            if (ok) {
              a.out[(size_t)row * a.ldo + col] = xv;
              afl_put<bf16_t>(a.out_afl, KTo, row, col, xv * gnext);
            }
            const float sq16 = sum16(xv * xv);
            if (ok && l16 == 0) a.ssq_out[(size_t)(col >> 4) * M + row] = sq16;
          }
        }
    }
  }
}

// Split-K reduction and epilogue: one workgroup per (row, 1024 columns); thread t holds
// 4 consecutive columns, sums the partials in split order, applies the row scale and
// the epilogue.  Four threads cover a 16-column group (partial sums of squares).
template <int EPI, bool NORM>
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs a) {
  __shared__ float s_red[4];
  const int row = blockIdx.y;
  const int col = blockIdx.x * 1024 + threadIdx.x * 4;
  const bool in = col < a.N;
  f32x4_t y = zero4();
  if (in) {
#pragma unroll 4
    for (int sp = 0; sp < a.splits; ++sp)
      y += *reinterpret_cast<const f32x4_t *>(a.part + ((size_t)sp * a.M + row) * a.N + col);
  }
  if (a.done && *a.done) return;
  if constexpr (NORM) {
    float s = 0.f;
    for (int p = threadIdx.x; p < a.norm_nparts; p += 256) s += a.ssq[(size_t)p * a.ld_ssq + row];
    s = sum_lanes<64>(s);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = s;
    __syncthreads();
    const float rs = 1.0f / sqrtf((s_red[0] + s_red[1] + s_red[2] + s_red[3]) / (float)a.K + a.norm_eps);
    y *= rs;
  }
  if (!in) return;
  const int KTo = a.N >> 5;
  if constexpr (EPI == EPI_STORE) {
    *reinterpret_cast<f32x4_t *>(a.out + (size_t)row * a.ldo + col) = y;
  } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
    for (int e = 0; e < 4; ++e) afl_put<bf16_t>(a.out_afl, KTo, row, col + e, gelu_erf(y[e]));
  } else {
    f32x4_t *xp = reinterpret_cast<f32x4_t *>(a.out + (size_t)row * a.ldo + col);
    const f32x4_t xv = *xp + y;
    *xp = xv;
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      afl_put<bf16_t>(a.out_afl, KTo, row, col + e, xv[e] * to_f32<bf16_t>(reinterpret_cast<const bf16_t *>(a.gain_next)[col + e]));
      sq += xv[e] * xv[e];
    }
    sq = sum_lanes<4>(sq);
    if ((threadIdx.x & 3) == 0) a.ssq_out[(size_t)(col >> 4) * a.M + row] = sq;
  }
}

}  // namespace

// Rows per workgroup tile: 64 for a layer projection with between a half and one
// 128-row tile per CU (the 64-row tiles then fill the chip without a K split), else 128,
// and always 128 for the LM head (its statistics come in 128-column groups of 128-row
// tiles).  Measured: with 1.5-2 tiles of 128 rows per CU the 64-row tiles were slower,
// bound by LDS bandwidth at their lower reuse, and fewer tiles are better split in K.
static int tile_bm(int epi, int M, int N) {
  if (epi == EPI_VSTAT) return 128;
  const int t128 = (N / BN) * ((M + 127) / 128);
  return t128 > 128 && t128 <= 256 ? 64 : 128;
}

bool gemm_tile_supported(int dtype, int M, int N, int K) {
  return dtype == DT_BF16 && M >= 128 && N % BN == 0 && K % (32 * KS) == 0;
}

int gemm_tile_slices(int N) { return N / BN; }

// Split only grids of less than one workgroup per CU (up to ~2 per CU, >= 8 k-tiles per
// split): measured, a grid of 256 tiles runs faster whole than split in two.  (For the
// layer projections, the only ones split.)
int gemm_tile_splits(int M, int N, int K) {
  const int bm = tile_bm(EPI_STORE, M, N);
  const int tiles = (N / BN) * ((M + bm - 1) / bm);
  int s = 1;
  if (tiles >= 256) return s;
  while (tiles * s < 512 && (K / 32) / (2 * s) >= 8) s *= 2;
  return s;
}

hipError_t launch_split_reduce(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.splits < 2 || a.part == nullptr || a.N % 16 || a.M <= 0) return hipErrorInvalidValue;
  const dim3 rgrid((a.N + 1023) / 1024, a.M);
#define TD_R(E, NRM)                                                                \
  if (epi == E && norm == NRM) {                                                \
    hipLaunchKernelGGL((split_reduce_kernel<E, NRM>), rgrid, dim3(256), 0, s, a); \
    return hipGetLastError();                                                   \
  }
  TD_R(EPI_STORE, true)
  TD_R(EPI_GELU, true)
  TD_R(EPI_RESID, false)
#undef TD_R
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_tile(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.N % BN || a.K % (32 * KS) || a.M <= 0 || a.splits < 1) return hipErrorInvalidValue;
  if (a.done == nullptr) return hipErrorInvalidValue;
  if (norm && (a.ssq == nullptr || a.norm_nparts <= 0)) return hipErrorInvalidValue;
  if ((epi == EPI_GELU || epi == EPI_RESID) && a.out_afl == nullptr) return hipErrorInvalidValue;
  const int bm = tile_bm(epi, a.M, a.N);
  if (a.splits > 1) {
    if (epi == EPI_VSTAT || a.part == nullptr || a.n_rows != nullptr) return hipErrorInvalidValue;
    const dim3 pgrid(a.N / BN, (a.M + bm - 1) / bm, a.splits);
    if (bm == 64) hipLaunchKernelGGL((gemm_tile_kernel<EPI_PART, false, 64>), pgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_tile_kernel<EPI_PART, false, 128>), pgrid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_reduce(epi, norm, a, s);
  }
  const dim3 grid(a.N / BN, (a.M + bm - 1) / bm);
#define TD_L(E, NRM)                                                                        \
  if (epi == E && norm == NRM) {                                                        \
    if (bm == 64) hipLaunchKernelGGL((gemm_tile_kernel<E, NRM, 64>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((gemm_tile_kernel<E, NRM, 128>), grid, dim3(256), 0, s, a);         \
    return hipGetLastError();                                                           \
  }
  TD_L(EPI_STORE, true)
  TD_L(EPI_GELU, true)
  TD_L(EPI_RESID, false)
#undef TD_L
  if (epi == EPI_VSTAT && norm) {
    hipLaunchKernelGGL((gemm_tile_kernel<EPI_VSTAT, true, 128>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace td
