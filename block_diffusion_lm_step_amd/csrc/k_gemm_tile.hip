// Tiled MFMA GEMM for many rows (batches of sequences): Y[M][N] = A[M][K] * W[N][K]^T.
//
// At M >= 128 every weight element is used by many rows and the projections are bound
// by the matrix cores, not by the weight stream.  A workgroup of 4 waves computes a
// BM x BNT output tile (BNT = 128, or 256 for the LM head and the widest projections);
// wave (wm, wn) owns a (BM/2) x (BNT/2) quarter ((BM/32) x (BNT/32) MFMA tiles of
// 16 x 16).  The 256-column tiles read a third fewer LDS bytes per product (the
// activations' two planes are loaded once for twice the columns), which is what these
// loops are short of: at 128 columns the matrix cores issue about half of the time.
// BM = 128, or 64 for layer projections whose 128-row tiles would give about one
// workgroup per CU: that leaves each SIMD a single wave, whose LDS and barrier latencies
// nothing overlaps (measured: the MFMA pipes were busy 22% of such a launch).
// K advances one 32-wide k-tile per stage through double-buffered LDS (48 KiB of stages
// at 128 columns; with 141 registers per lane three workgroups share a CU, and one's LDS
// traffic and barrier overlap the others' MFMAs; two at 256 columns), one barrier per
// stage: the next stage is loaded
// from memory into registers while the current one is multiplied, then written to the
// other buffer.  A projection with about one 128-row tile per CU runs two such groups of
// four waves per workgroup, each over one half of the k-tiles (KG = 2).
// Both operands are already in MFMA fragment order in memory (weights packed at
// creation, activations written in fragment layout by their producers), so staging is
// a straight 16-byte copy; the activation fragments' bf16 high and low halves go to two
// separate LDS planes so that a wave's 16-byte LDS reads are contiguous (no bank
// conflicts).  Per k-tile and wave: 8 activation + 4 (BNT = 256: 8) weight fragment
// reads from LDS, 32 (64) MFMAs (high and low parts of the activations against the bf16
// weights).
//
// Epilogues as in the weight-streaming kernels (the RMSNorm row scale multiplies the
// accumulator): STORE (q/k/v), GELU and RESID (fragment-layout outputs, partial sums of
// squares per 16 columns), and VSTAT for the LM head (rows gathered through the row
// list; per row one (max, sum of exp, argmax) triple per BNT-column group).
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

constexpr int BN = 128;             // workgroup tile columns
constexpr int KS = 1;               // k-tiles per stage

// Small per-thread tables are vector values, not arrays: arrays indexed in loops are
// turned into LDS or scratch copies before the loops are unrolled.
typedef unsigned long long u64x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int BM, int BNT>
struct alignas(16) StageLds {
  u32x4_t a_hi[BM / 16][KS][64];   // activation fragments, bf16 high parts
  u32x4_t a_lo[BM / 16][KS][64];   // ... bf16 remainders
  u32x4_t w[BNT / 16][KS][64];     // weight fragments
};

constexpr int EPI_PART = 100;   // split-K partial: store the raw accumulator tile

// K split of a tiled layer GEMM: the static split a.splits, grown (a.dyn) when the live
// row tiles times the column tiles fill less than one workgroup per CU, as happens late in
// a batched block loop once most sequences are adopted (their rows leave the row list):
// then about two workgroups per CU, never more than the grid holds, at least 8 k-tiles
// per split, and no more partials than the workspace holds.  The GEMM and its reduction
// both derive it from the same live row count, so they agree.  Partials are laid out
// [split][live tiles * BM][N] (position in the row list, then column).
constexpr int DYN_MIN_WG = 256, DYN_TARGET_WG = 512;
struct SplitPlan {
  int live, S, pstride;
};
TD_DEV SplitPlan split_plan(const GemmArgs &a, int nrows, int bm, int tiles_x, int grid_y) {
  SplitPlan p;
  p.live = (nrows + bm - 1) / bm;
  p.pstride = p.live * bm;
  p.S = a.splits;
  const int per = p.live * tiles_x;   // workgroups per split
  if (a.dyn && per > 0 && per * a.splits < DYN_MIN_WG) {
    int s = (DYN_TARGET_WG + per - 1) / per;
    s = min(s, grid_y * a.splits / p.live);
    s = min(s, (a.K >> 5) / 8);
    s = (int)min((size_t)s, a.part_cap / ((size_t)p.pstride * a.N));
    p.S = max(s, a.splits);
  }
  return p;
}

// LM-head tile of the workgroup at (blockIdx.x, blockIdx.y), or false if the launch
// index lies past the live row tiles (gy of them; the grid holds row tiles for every
// row).  Workgroups are handed to the eight XCDs round-robin in launch order, each XCD
// with its own L2, and the head matrix (V x d, larger than the last-level cache) must not
// be fetched once per row tile.  So the workgroups an XCD runs together cover a block of
// up to 8 row tiles x 8 column tiles (each k-slice of a column tile is then read once for
// all of the block's row tiles, and of a row tile once for all 8 column tiles): launch
// index i goes to XCD i % 8, and the XCD's j-th workgroup (j = i / 8) takes block
// j / (gm * 8) of its column tiles (c == XCD mod 8), row tile j % gm of the block's rows.
// The live tiles take the first launch indices, so they start first.  Needs
// gridDim.x % 64 == 0 (else the tiles keep the launch order).
TD_DEV bool lmhead_tile(int gy, int &tx, int &ty) {
  const int gx = gridDim.x;
  if (gx % 64) return true;
  const int i = blockIdx.y * gx + blockIdx.x;
  if (i >= gx * gy) return false;
  int gm = gy < 8 ? gy : 8;
  while (gy % gm) --gm;                       // row tiles per block: a divisor of gy
  const int xcd = i & 7, j = i >> 3;
  const int blk = j / (gm * 8), w = j % (gm * 8);
  const int rblocks = gy / gm;
  ty = (blk % rblocks) * gm + w % gm;
  tx = ((blk / rblocks) * 8 + w / gm) * 8 + xcd;
  return true;
}

// KG = 2: eight waves in two groups of four; each group takes one half of the
// workgroup's k-tiles through its own pair of stage buffers, and the second group's
// accumulators are added to the first's through LDS (first half + second half, one
// rounding) before the first group's epilogue.  Twice the waves on a tile without a
// split-K reduction launch.
template <int EPI, bool NORM, int BM, int KG = 1, int BNT = BN>
__global__ __launch_bounds__(256 * KG, KG == 1 ? 2 : 1) void gemm_tile_kernel(GemmArgs a) {
  static_assert(KG == 1 || (KG == 2 && EPI != EPI_VSTAT && EPI != EPI_PART), "two K groups: layer epilogues only");
  static_assert(BNT == BN || (BNT == 256 && KG == 1 && BM == 128 && EPI != EPI_PART), "256-column tiles");
  constexpr int NTW = BNT / 32;                    // 16-column MFMA tiles per wave
  constexpr int NFW = (BNT / 16) * KS * 64 / 256;  // weight fragments staged per thread
  constexpr int MTW = BM / 32;                     // MFMA row tiles per wave
  constexpr int NFA = (BM / 16) * KS * 64 / 256;   // activation fragments staged per thread
  constexpr int NPAR = 256 / BM;                   // threads per row summing squares
  __shared__ StageLds<BM, BNT> s_st[KG][2];
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
  int tx = blockIdx.x, ty = blockIdx.y, sp = blockIdx.z, S = a.splits, pstride = 0;
  if constexpr (EPI == EPI_VSTAT) {
    if (!lmhead_tile((nrows + BM - 1) / BM, tx, ty)) return;
  } else {
    const SplitPlan pl = split_plan(a, nrows, BM, gridDim.x, gridDim.y);
    pstride = pl.pstride;
    if (pl.S != a.splits) {   // grown split: workgroup (y, z) -> live row tile, split
      S = pl.S;
      const int idx = blockIdx.z * gridDim.y + blockIdx.y;
      ty = idx % pl.live;
      sp = idx / pl.live;
      if (sp >= S) return;
    }
  }
  const int m0 = ty * BM, n0 = tx * BNT;
  if (m0 >= nrows) return;
  const int tid = threadIdx.x & 255;                      // thread within its K group
  const int kg = KG == 1 ? 0 : (int)(threadIdx.x >> 8);  // K group (wave-uniform)
  const bool lead = kg == 0;                              // the group that finishes the tile
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  // K range of this workgroup: split sp of S (whole k-tiles).
  const int KTall = a.K >> 5;
  const int kw0 = (int)((int64_t)KTall * sp / S), kw1 = (int)((int64_t)KTall * (sp + 1) / S);
  // This K group's k-tiles [kt0, kt1); the first group takes the larger half.
  const int kmid = KG == 1 ? kw1 : kw0 + (kw1 - kw0 + 1) / 2;
  const int kt0 = lead ? kw0 : kmid, kt1 = lead ? kmid : kw1;
  const int KT = KTall, nstage = (kt1 - kt0) / KS, nmax = (kmid - kw0) / KS;

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
    const int f = tid + 256 * i;
    const int fl = f & 63, kt = (f >> 6) % KS, t = f / (64 * KS);
    const int row = s_row[t * 16 + (fl & 15)];
    aoff[i] = (((size_t)(row >> 4) * KT + kt0 + kt) * 64 + (fl >> 4) * 16 + (row & 15)) * 32;
  }
#pragma unroll
  for (int i = 0; i < NFW; ++i) {
    const int f = tid + 256 * i;
    const int fl = f & 63, kt = (f >> 6) % KS, t = f / (64 * KS);
    woff[i] = (((size_t)(n0 / 16 + t) * KT + kt0 + kt) * 64 + fl) * 8;
  }
  // (tile, k-tile) of fragment i = 0; fragment i is 4 / KS tiles further.
  const int ft = tid / (64 * KS), fkt = (tid >> 6) % KS;
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
    s_st[kg][B].a_hi[ft + (4 / KS) * i][fkt][lane] = ra_hi[i];                                  \
    s_st[kg][B].a_lo[ft + (4 / KS) * i][fkt][lane] = ra_lo[i];                                  \
  }                                                                                             \
  _Pragma("unroll") for (int i = 0; i < NFW; ++i) s_st[kg][B].w[ft + (4 / KS) * i][fkt][lane] = rw[i];

  if (nstage > 0) {   // (a second K group can have no k-tile)
    TD_LOAD_STAGE(0)
  }
  asm volatile("" ::: "memory");   // the loads above are issued before the test below
  if (stop) return;
  if constexpr (NORM && EPI != EPI_PART) {
    // Row scales from the producer's partial sums of squares: thread t sums the parts
    // p = t / BM (mod NPAR) of row t % BM (consecutive threads read consecutive rows).
    const int r = tid & (BM - 1), par = tid / BM;
    if (lead) {
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
  }
  if (nstage > 0) {
    TD_STORE_STAGE(0)
  }
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

  // Both K groups pass the same barriers: nmax stages, the second group idle in the last
  // one when its half is the shorter.
  for (int s = 0; s < nmax; ++s) {
    const int b = s & 1;
    if (s + 1 < nstage) {
      TD_LOAD_STAGE(s + 1)
    }
#pragma unroll
    for (int kt = 0; kt < KS; ++kt) {
      if (KG > 1 && s >= nstage) break;
      AFrag<bf16_t> af[MTW];
      Frag<bf16_t> wf[NTW];
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        af[i].hi.raw = __builtin_bit_cast(uint4, s_st[kg][b].a_hi[wm * MTW + i][kt][lane]);
        af[i].lo.raw = __builtin_bit_cast(uint4, s_st[kg][b].a_lo[wm * MTW + i][kt][lane]);
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j) wf[j].raw = __builtin_bit_cast(uint4, s_st[kg][b].w[wn * NTW + j][kt][lane]);
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

  if constexpr (KG == 2) {   // the second group's sums into the first's, through the idle stages
    static_assert(4 * MTW * NTW * 64 * 16 <= (int)sizeof(s_st), "accumulators fit the stage buffers");
    f32x4_t *xf = reinterpret_cast<f32x4_t *>(&s_st[0][0]) + wave * MTW * NTW * 64 + lane;
    if (!lead) {
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) xf[(i * NTW + j) * 64] = acc[i][j];
    }
    __syncthreads();
    if (lead) {
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] += xf[(i * NTW + j) * 64];
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  // Split partial: the raw accumulator tile at (split, position in the row list).
  auto store_part = [&]() __attribute__((always_inline)) {
    float *part = a.part + (size_t)sp * pstride * a.N;
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int col = n0 + (wn * NTW + j) * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = m0 + (wm * MTW + i) * 16 + 4 * g + r;   // < pstride
          part[(size_t)pos * a.N + col] = acc[i][j][r];
        }
      }
  };
  if constexpr (EPI == EPI_PART) {
    store_part();
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
        // The row's statistics over the wave's 16 NTW columns (a row past the live count
        // gives the empty set).
        const int col0 = n0 + wn * NTW * 16 + l16;
        float sv[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const float z = acc[i][j][r] * rs;
          sv[j] = -INFINITY;
          if (live) {
            if (a.logits) a.logits[(size_t)row * a.N + col0 + 16 * j] = z;
            sv[j] = tau * z;
          }
        }
        const VStat v = vstat_row16<NTW>(sv, col0, live);
        if (l16 == 0) s_stat[wn][ri] = v;
      }
    __syncthreads();
    if (threadIdx.x < BM && m0 + threadIdx.x < nrows)
      a.vpart[(size_t)(m0 + threadIdx.x) * gridDim.x + tx] = vstat_merge(s_stat[0][threadIdx.x], s_stat[1][threadIdx.x]);
  } else {
    if (S > 1) {   // a grown split (workgroup-uniform): split_reduce applies the epilogue
      if (lead) store_part();
      return;
    }
    // STORE / GELU / RESID, a half of the wave's columns at a time: the wave parks its
    // accumulators (row scale applied) in the now idle stage buffers, one padded row per
    // tile row, and reads them back as 8 consecutive columns of one row per lane, so that
    // every output is a whole 32-byte fragment-layout chunk (hi and lo parts of 8 columns)
    // or a 32-byte run of a row-major fp32 row, instead of per-element stores.
    // Output row of tile row ri: through the row list when one is given (the rows of the
    // sequences still active), else m0 + ri; positions past the live count are not written.
    constexpr int RW = MTW * 16;        // rows of the wave's tile
    constexpr int EP = 32 + 4;          // padded row of 32 columns (floats)
    static_assert(4 * RW * EP * 4 <= (int)sizeof(s_st), "epilogue staging fits the stage buffers");
    float *ep = reinterpret_cast<float *>(&s_st[0][0]) + wave * RW * EP;
    const int M = a.M;
    const int KTo = a.N >> 5;
#pragma unroll
    for (int h = 0; h < NTW / 2; ++h) {
      // (With two K groups the first one does the epilogue; the second passes the
      // barriers.)
      if (lead) {
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rl = i * 16 + 4 * g + r;
            float y = acc[i][2 * h + jj][r];
            if constexpr (NORM) y *= s_rs[wm * RW + rl];
            ep[rl * EP + jj * 16 + l16] = y;
          }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < RW * 4 / 64; ++q) {
        if (!lead) break;
        const int o = lane + 64 * q;               // octet: row o / 4, columns 8 (o % 4) ..
        const int rl = o >> 2, c8 = (o & 3) * 8;
        const int ri = wm * RW + rl;
        const bool ok = m0 + ri < nrows;
        const int row = a.rowlist ? s_row[ri] : m0 + ri;
        const int col = n0 + (wn * NTW + 2 * h) * 16 + c8;
        float v[8];
        load8f(ep + rl * EP + c8, v);
        if constexpr (EPI == EPI_STORE) {
          if (ok) {
            float4 *o4 = reinterpret_cast<float4 *>(a.out + (size_t)row * a.ldo + col);
            o4[0] = make_float4(v[0], v[1], v[2], v[3]);
            o4[1] = make_float4(v[4], v[5], v[6], v[7]);
          }
        } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e]);
          if (ok) afl_put8<bf16_t>(a.out_afl, KTo, row, col, v);
        } else {
          float xo[8], gn[8], sq = 0.f;
          load8f(a.out + (size_t)(ok ? row : 0) * a.ldo + col, xo);
          Frag<bf16_t> gf;
          gf.load(reinterpret_cast<const bf16_t *>(a.gain_next) + col);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] += xo[e];
            sq += v[e] * v[e];
            gn[e] = v[e] * gf.get(e);
          }
          sq += dpp_f<DPP_SWAP1>(sq);   // the neighbouring lane holds the other 8 columns of the 16
          if (ok) {
            float4 *x4 = reinterpret_cast<float4 *>(a.out + (size_t)row * a.ldo + col);
            x4[0] = make_float4(v[0], v[1], v[2], v[3]);
            x4[1] = make_float4(v[4], v[5], v[6], v[7]);
            afl_put8<bf16_t>(a.out_afl, KTo, row, col, gn);
            if ((o & 1) == 0) a.ssq_out[(size_t)(col >> 4) * M + row] = sq;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Split-K reduction and epilogue: a workgroup per (row position, 1024 columns), rows
// taken with a stride of gridDim.y; thread t holds 4 consecutive columns, sums the
// partials in split order, applies the row scale and the epilogue.  Four threads cover a
// 16-column group (partial sums of squares).  After a tiled GEMM the split is the one it
// used (split_plan: possibly grown, or none, in which case there is nothing to do).
template <int EPI, bool NORM>
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs a) {
  __shared__ float s_red[4];
  const int nrows = a.n_rows ? *a.n_rows : a.M;   // loaded with the loop-exit flag
  int S = a.splits, pstride = a.M;
  if (a.tile_rows > 0) {
    const SplitPlan pl = split_plan(a, nrows, a.tile_rows, a.N / BN, (a.M + a.tile_rows - 1) / a.tile_rows);
    S = pl.S;
    pstride = pl.pstride;
  }
  if (a.done && *a.done) return;
  if (S < 2) return;
  const int col = blockIdx.x * 1024 + threadIdx.x * 4;
  const bool in = col < a.N;
  // Partials are indexed by position; the output row is the row list's entry there when
  // a row list is given (positions past the live count have nothing to do).
  for (int pos = blockIdx.y; pos < nrows; pos += gridDim.y) {   // workgroup-uniform
    const int row = a.rowlist ? a.rowlist[min(pos, a.M - 1)] : pos;
    f32x4_t y = zero4();
    if (in) {
#pragma unroll 4
      for (int sp = 0; sp < S; ++sp)
        y += *reinterpret_cast<const f32x4_t *>(a.part + ((size_t)sp * pstride + pos) * a.N + col);
    }
    if constexpr (NORM) {
      float s = 0.f;
      for (int p = threadIdx.x; p < a.norm_nparts; p += 256) s += a.ssq[(size_t)p * a.ld_ssq + row];
      s = sum_lanes<64>(s);
      if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = s;
      __syncthreads();
      const float rs = 1.0f / sqrtf((s_red[0] + s_red[1] + s_red[2] + s_red[3]) / (float)a.K + a.norm_eps);
      y *= rs;
      __syncthreads();   // s_red is rewritten for the next position
    }
    if (!in) continue;
    const int KTo = a.N >> 5;
    if constexpr (EPI == EPI_STORE) {
      *reinterpret_cast<f32x4_t *>(a.out + (size_t)row * a.ldo + col) = y;
    } else if constexpr (EPI == EPI_GELU) {
      float u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = gelu_erf(y[e]);
      afl_put4<bf16_t>(a.out_afl, KTo, row, col, u);
    } else {
      f32x4_t *xp = reinterpret_cast<f32x4_t *>(a.out + (size_t)row * a.ldo + col);
      const f32x4_t xv = *xp + y;
      *xp = xv;
      float sq = 0.f, gx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gx[e] = xv[e] * to_f32<bf16_t>(reinterpret_cast<const bf16_t *>(a.gain_next)[col + e]);
        sq += xv[e] * xv[e];
      }
      afl_put4<bf16_t>(a.out_afl, KTo, row, col, gx);
      sq = sum_lanes<4>(sq);
      if ((threadIdx.x & 3) == 0) a.ssq_out[(size_t)(col >> 4) * a.M + row] = sq;
    }
  }
}

}  // namespace

// Rows per workgroup tile: 64 for a layer projection with between a half and three
// quarters of a 128-row tile per CU (the 64-row tiles then fill the chip without a K
// split), except a deep contraction (K >= 4 N, the MLP down projection), which keeps
// 128-row tiles and splits K in two instead (measured at 2048 x 2048 x 8192: 151 us
// against 194 us in 64-row tiles); else 128, and always 128 for the LM head (its
// statistics come per column group of 128-row tiles).  Measured: with 1.5-2 tiles of
// 128 rows per CU the 64-row tiles were slower, bound by LDS bandwidth at their lower
// reuse, and fewer tiles are better split in K.
static int tile_bm(int epi, int M, int N, int K) {
  if (epi == EPI_VSTAT) return 128;
  const int t128 = (N / BN) * ((M + 127) / 128);
  return t128 > 128 && t128 <= 192 && K < 4 * N ? 64 : 128;
}

// K groups per workgroup: two (eight waves, 128-row tiles) for a layer projection with
// between three quarters of and one 128-row tile per CU, which 64-row tiles used to
// cover (bound by LDS bandwidth at their lower reuse).  Measured: the output projection
// of 2048 rows 55.7 -> 49.1 us, the MLP up projection of 512 rows 54.5 -> 51.5 us.  The
// MLP down projection keeps its two-way K split: as two K groups with its split grown on
// the device only at few rows it took 137.8 us against 132.5 (the two halves of a
// 256-k-tile range in one workgroup).
static int tile_kg(int epi, int M, int N, int K) {
  if (epi == EPI_VSTAT) return 1;
  const int t128 = (N / BN) * ((M + 127) / 128);
  return t128 > 192 && t128 <= 256 && K < 4 * N ? 2 : 1;
}

bool gemm_tile_supported(int dtype, int M, int N, int K) {
  return dtype == DT_BF16 && M >= 128 && N % BN == 0 && K % (32 * KS) == 0;
}

// The LM head runs 256-column tiles whenever the vocabulary allows: one statistics
// triple per row and 256 columns.  Measured at 2048 rows x 131072 x 2048: 1.80-1.85 ms
// against 2.22 in 128-column tiles (logits bit-identical).
static int lmhead_bn(int N) { return N % 256 == 0 ? 256 : BN; }
int gemm_tile_slices(int N) { return N / lmhead_bn(N); }

// 256-column tiles for an unsplit layer projection whose 128 x 256 tiles still number at
// least two per CU (two workgroups of 233 registers and 66 KiB of LDS share a CU).
// Measured at 2048 rows: the MLP up projection 141-144 us against 147-148 in 128-column
// tiles; the QKV projection (384 such tiles) keeps 128 columns.
static bool tile_wide(int M, int N, int bm, int kg, const GemmArgs &a) {
  return bm == 128 && kg == 1 && a.splits == 1 && !a.dyn && N % 256 == 0 && (N / 256) * ((M + 127) / 128) >= 512;
}

// Split only grids of less than one workgroup per CU (up to ~2 per CU, >= 8 k-tiles per
// split): measured, a grid of 256 tiles runs faster whole than split in two.  (For the
// layer projections, the only ones split.)
int gemm_tile_splits(int M, int N, int K) {
  const int bm = tile_bm(EPI_STORE, M, N, K);
  const int tiles = (N / BN) * ((M + bm - 1) / bm);
  int s = 1;
  if (tiles >= 512 || (tiles >= 256 && K < 4 * N)) return s;
  while (tiles * s < 512 && (K / 32) / (2 * s) >= 8) s *= 2;
  return s;
}

hipError_t launch_split_reduce(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.part == nullptr || a.N % 16 || a.M <= 0) return hipErrorInvalidValue;
  if (a.splits < 2 && !(a.dyn && a.tile_rows > 0)) return hipErrorInvalidValue;
  // A static split covers every row, one workgroup per row; after a GEMM whose split only
  // grows at few live rows, 128 row positions per column chunk (nothing to do, and cheap,
  // at full batch).
  const dim3 rgrid((a.N + 1023) / 1024, a.splits > 1 ? a.M : std::min(a.M, 128));
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

hipError_t launch_gemm_tile(int epi, bool norm, const GemmArgs &a_in, hipStream_t s) {
  GemmArgs a = a_in;
  if (a.N % BN || a.K % (32 * KS) || a.M <= 0 || a.splits < 1) return hipErrorInvalidValue;
  if (a.done == nullptr) return hipErrorInvalidValue;
  if (norm && (a.ssq == nullptr || a.norm_nparts <= 0)) return hipErrorInvalidValue;
  if ((epi == EPI_GELU || epi == EPI_RESID) && a.out_afl == nullptr) return hipErrorInvalidValue;
  const int bm = tile_bm(epi, a.M, a.N, a.K);
  if ((a.n_rows == nullptr) != (a.rowlist == nullptr)) return hipErrorInvalidValue;
  if (a.dyn && (epi == EPI_VSTAT || a.part == nullptr || a.n_rows == nullptr)) return hipErrorInvalidValue;
  a.tile_rows = bm;
  if (a.splits > 1) {
    if (epi == EPI_VSTAT || a.part == nullptr) return hipErrorInvalidValue;
    const dim3 pgrid(a.N / BN, (a.M + bm - 1) / bm, a.splits);
    if (bm == 64) hipLaunchKernelGGL((gemm_tile_kernel<EPI_PART, false, 64>), pgrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_tile_kernel<EPI_PART, false, 128>), pgrid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_reduce(epi, norm, a, s);
  }
  const dim3 grid(a.N / BN, (a.M + bm - 1) / bm);
  const int kg = tile_kg(epi, a.M, a.N, a.K);
  const bool wide = tile_wide(a.M, a.N, bm, kg, a);
  const dim3 wgrid(a.N / 256, (a.M + bm - 1) / bm);
#define TD_L(E, NRM)                                                                        \
  if (epi == E && norm == NRM) {                                                        \
    if (bm == 64) hipLaunchKernelGGL((gemm_tile_kernel<E, NRM, 64>), grid, dim3(256), 0, s, a); \
    else if (kg == 2) hipLaunchKernelGGL((gemm_tile_kernel<E, NRM, 128, 2>), grid, dim3(512), 0, s, a); \
    else if (wide) hipLaunchKernelGGL((gemm_tile_kernel<E, NRM, 128, 1, 256>), wgrid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((gemm_tile_kernel<E, NRM, 128>), grid, dim3(256), 0, s, a);         \
    hipError_t e = hipGetLastError();                                                   \
    if (e != hipSuccess || !a.dyn) return e;                                            \
    return launch_split_reduce(epi, norm, a, s);                                        \
  }
  TD_L(EPI_STORE, true)
  TD_L(EPI_GELU, true)
  TD_L(EPI_RESID, false)
#undef TD_L
  if (epi == EPI_VSTAT && norm) {
    if (lmhead_bn(a.N) == 256)
      hipLaunchKernelGGL((gemm_tile_kernel<EPI_VSTAT, true, 128, 1, 256>), dim3(a.N / 256, (a.M + bm - 1) / bm),
                         dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_tile_kernel<EPI_VSTAT, true, 128>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace td
