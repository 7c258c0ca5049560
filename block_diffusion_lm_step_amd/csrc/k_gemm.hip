// LM head with the vocabulary statistics fused into its epilogue:
//   z[r][v] = rmsnorm(x_r) . W_head[v],  and per row and column group the tau-scaled
//   max, sum of exp(tau z - max) and lowest argmax.
//
// The head matrix (V x d) is the largest weight of the step and is read once per step;
// at block sizes (16 masked rows per sequence or fewer) the kernel is bound by that
// stream.  Each of the NW waves of a workgroup owns NT consecutive 16-column tiles and
// the whole K range, and keeps PASS k-tiles of its weights (pre-packed 16x32 MFMA tiles, one contiguous KiB per
// load) and of the activation fragments in flight, refilling a slot right after its
// MFMA; all loads are unconditional (clamped addresses) so the compiler's waits before
// each MFMA are exact.  No LDS staging and no barrier inside the stream: the waves of a
// workgroup only meet to merge their statistics.
//
// Rows are gathered through the row list (only positions still masked need logits).
// Activations are the final RMSNorm's input in fragment layout, stored by the last
// residual update as x * gain; the row scale 1/sqrt(mean(x^2) + eps) comes from that
// update's partial sums of squares and multiplies the accumulator.
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

template <typename T, int MT, int NT, int NW> constexpr int lm_pass() {
  constexpr int per = MT * 8 + NT * (sizeof(T) == 2 ? 4 : 8);   // VGPRs per k-tile in flight
  constexpr int p = (NW == 8 ? 72 : 160) / per;   // two workgroups per CU
  return p > 8 ? 8 : (p < 1 ? 1 : p);
}

template <typename T, int MT, int NT, int NW>
__global__ __launch_bounds__(64 * NW) void lmhead_kernel(GemmArgs a) {
  constexpr int PASS = lm_pass<T, MT, NT, NW>();
  constexpr int ROWS = 16 * MT;
  constexpr int TPR = (64 * NW / ROWS) < 64 ? 64 * NW / ROWS : 64;   // threads per row (row scales)
  constexpr int SQB = 16;
  // The loop-exit flag decides before any operand is requested (a launch in a step after
  // the block is adopted then reads nothing else).
  if (__hip_atomic_load(a.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
  const int nrows = a.n_rows ? *a.n_rows : a.M;
  const int m0 = blockIdx.z * ROWS;
  if (m0 >= nrows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int KT = a.K >> 5;
  const int ntw = (blockIdx.x * NW + wave) * NT;   // this wave's first column tile

  __shared__ int s_row[ROWS];
  __shared__ float s_rs[ROWS];
  __shared__ VStat s_stat[NW][ROWS];
  if (threadIdx.x < ROWS) {
    const int i = m0 + threadIdx.x;
    s_row[threadIdx.x] = i < nrows ? (a.rowlist ? a.rowlist[i] : i) : -1;
  }
  __syncthreads();

  // Partial sums of squares of the rows first (TPR threads per row).
  const int rr = threadIdx.x / TPR, sub = threadIdx.x % TPR;
  const int srow = s_row[rr] >= 0 ? s_row[rr] : s_row[0];
  float sq[SQB];
#pragma unroll
  for (int j = 0; j < SQB; ++j) sq[j] = a.ssq[(size_t)min(sub + TPR * j, a.norm_nparts - 1) * a.ld_ssq + srow];

  // Activation fragment bases: lane's row of each row tile, group g of every k-tile.
  const char *Al[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r0 = s_row[mt * 16 + l16];
    const int row = r0 >= 0 ? r0 : s_row[0];
    Al[mt] = reinterpret_cast<const char *>(a.A) + ((size_t)(row >> 4) * KT * 64 + g * 16 + (row & 15)) * 32;
  }
  const T *Wl = reinterpret_cast<const T *>(a.Wp) + ((size_t)ntw * KT) * 512 + (size_t)lane * 8;
  AFrag<T> xa[PASS][MT];
  Frag<T> wb[PASS][NT];
  auto fill = [&](int i, int kt) __attribute__((always_inline)) {
    const int k = min(kt, KT - 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xa[i][mt] = afl_get<T>(Al[mt] + (size_t)k * 2048);
#pragma unroll
    for (int j = 0; j < NT; ++j) wb[i][j].load_nt(Wl + ((size_t)j * KT + k) * 512);
  };
#pragma unroll
  for (int i = 0; i < PASS; ++i) fill(i, i);
  {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < SQB; ++j) s += (sub + TPR * j < a.norm_nparts) ? sq[j] : 0.f;
    for (int p = sub + TPR * SQB; p < a.norm_nparts; p += TPR) s += a.ssq[(size_t)p * a.ld_ssq + srow];
    s = sum_lanes<TPR>(s);
    if (sub == 0) s_rs[rr] = 1.0f / sqrtf(s / (float)a.K + a.norm_eps);
  }

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[mt][j] = zero4();
  int p0 = 0;
  for (; p0 + PASS < KT; p0 += PASS) {
#pragma unroll
    for (int i = 0; i < PASS; ++i) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[mt][j] = mma_a(xa[i][mt], wb[i][j], acc[mt][j]);
      fill(i, p0 + PASS + i);
      __builtin_amdgcn_sched_barrier(0);   // keep the refill right behind its MFMAs
    }
  }
#pragma unroll
  for (int i = 0; i < PASS; ++i) {
    if (p0 + i < KT) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[mt][j] = mma_a(xa[i][mt], wb[i][j], acc[mt][j]);
    }
  }
  __syncthreads();   // row scales visible

  // Statistics of this wave's 16 NT columns per row, then of the workgroup's columns.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ri = mt * 16 + 4 * g + r;
      const int row = s_row[ri];
      const float rs = s_rs[ri];
      const float tau = (row >= 0 && a.inv_temp) ? a.inv_temp[row] : 1.0f;
      const int col0 = ntw * 16 + l16;
      float sv[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float z = acc[mt][j][r] * rs;
        sv[j] = -INFINITY;
        if (row >= 0) {
          if (a.logits) a.logits[(size_t)row * a.N + col0 + 16 * j] = z;
          sv[j] = tau * z;
        }
      }
      const VStat v = vstat_row16<NT>(sv, col0, row >= 0);
      if (l16 == 0) s_stat[wave][ri] = v;
    }
  __syncthreads();
  if (threadIdx.x < ROWS && s_row[threadIdx.x] >= 0) {
    VStat v = s_stat[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < NW; ++w) v = vstat_merge(v, s_stat[w][threadIdx.x]);
    a.vpart[(size_t)(m0 + threadIdx.x) * gridDim.x + blockIdx.x] = v;
  }
}

// ---------------------------------------------------------------- few rows, activations in LDS
// At most 16 rows and a contraction of at most 2048 (bf16 towers): the activation block
// (rows 0..15 in fragment layout: K / 32 slots of 2 KiB, one contiguous run) fits in
// LDS.  Each workgroup copies it there once, with loads issued before its first weights,
// and its 16 waves then stream only weights -- PASS k-tiles of two column tiles each in
// flight -- taking the activation fragments from LDS instead of re-reading them from L2
// per wave.  Every row is multiplied (the MFMA is 16 rows wide either way); statistics
// are written only for rows still masked, at their position in the row list.  The
// arithmetic of each row and column is that of lmhead_kernel.
constexpr int LDS_NW = 16, LDS_NT = 2, LDS_KMAX = 2048;

__global__ __launch_bounds__(64 * LDS_NW) void lmhead_lds_kernel(GemmArgs a) {
  constexpr int NW = LDS_NW, NT = LDS_NT, KTMAX = LDS_KMAX / 32;
  constexpr int PASS = 10;                        // weight k-tiles in flight per wave (measured: 8 and 6 slower)
  constexpr int APT = KTMAX * 128 / (64 * NW);    // 16-byte words of the block per thread
  __shared__ u32x4_t s_a[KTMAX * 128];            // [k-tile][lane][hi, lo]
  __shared__ float s_rs[16], s_tau[16];
  __shared__ int s_pos[16];
  __shared__ VStat s_stat[NW][16];

  // The loop-exit flag first (see lmhead_kernel), then the small per-row values, the
  // activation block and the first weights.
  if (__hip_atomic_load(a.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
  const int M = a.M, KT = a.K >> 5;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int ntw = (blockIdx.x * NW + wave) * NT;   // this wave's first column tile

  static_assert(16 % NW == 0 || NW % 16 == 0, "rows per wave");
  constexpr int RPW = NW >= 16 ? 1 : 16 / NW;    // rows whose scale each wave forms
  const int r16 = min((int)(threadIdx.x & 15), M - 1);
  const int pos = a.rowpos[r16];
  const float tau = a.inv_temp ? a.inv_temp[r16] : 1.0f;
  float sq0[RPW], sq1[RPW];   // wave w sums the partial squares of rows w, w + NW, ...
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int srow = min(wave + NW * i, M - 1);
    sq0[i] = a.ssq[(size_t)min(lane, a.norm_nparts - 1) * a.ld_ssq + srow];
    sq1[i] = a.ssq[(size_t)min(lane + 64, a.norm_nparts - 1) * a.ld_ssq + srow];
  }

  const u32x4_t *ga = reinterpret_cast<const u32x4_t *>(a.A);
  const int nwords = KT * 128;
  u32x4_t ra[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) ra[i] = ga[min((int)threadIdx.x + 64 * NW * i, nwords - 1)];

  const bf16_t *Wl = reinterpret_cast<const bf16_t *>(a.Wp) + ((size_t)ntw * KT) * 512 + (size_t)lane * 8;
  Frag<bf16_t> wb[PASS][NT];
  auto fill = [&](int i, int kt) __attribute__((always_inline)) {
    const int k = min(kt, KT - 1);
#pragma unroll
    for (int j = 0; j < NT; ++j) wb[i][j].load_nt(Wl + ((size_t)j * KT + k) * 512);
  };
#pragma unroll
  for (int i = 0; i < PASS; ++i) fill(i, i);

  // Waiting for the block waits for nothing issued after it: the weights stay in flight.
#pragma unroll
  for (int i = 0; i < APT; ++i) s_a[threadIdx.x + 64 * NW * i] = ra[i];
  if (threadIdx.x < 16) {
    s_pos[threadIdx.x] = threadIdx.x < (unsigned)M ? pos : -1;
    s_tau[threadIdx.x] = tau;
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    float sq = (lane < a.norm_nparts ? sq0[i] : 0.f) + (lane + 64 < a.norm_nparts ? sq1[i] : 0.f);
    sq = sum_lanes<64>(sq);
    if (lane == 0 && wave + NW * i < 16) s_rs[wave + NW * i] = 1.0f / sqrtf(sq / (float)a.K + a.norm_eps);
  }
  __syncthreads();

  auto afrag = [&](int kt) __attribute__((always_inline)) {
    const u32x4_t *p = s_a + ((size_t)min(kt, KT - 1) * 64 + lane) * 2;
    AFrag<bf16_t> f;
    f.hi.raw = __builtin_bit_cast(uint4, p[0]);
    f.lo.raw = __builtin_bit_cast(uint4, p[1]);
    return f;
  };
  f32x4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = zero4();
  AFrag<bf16_t> xa = afrag(0);   // one k-tile ahead of its MFMAs
  int p0 = 0;
  for (; p0 + PASS < KT; p0 += PASS) {
#pragma unroll
    for (int i = 0; i < PASS; ++i) {
      const AFrag<bf16_t> cur = xa;
      xa = afrag(p0 + i + 1);
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mma_a(cur, wb[i][j], acc[j]);
      fill(i, p0 + PASS + i);
      __builtin_amdgcn_sched_barrier(0);   // keep the refill right behind its MFMAs
    }
  }
#pragma unroll
  for (int i = 0; i < PASS; ++i) {
    if (p0 + i < KT) {
      const AFrag<bf16_t> cur = xa;
      xa = afrag(p0 + i + 1);
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = mma_a(cur, wb[i][j], acc[j]);
    }
  }

  // Statistics of this wave's 16 NT columns per row, then of the workgroup's columns.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * g + r;
    const bool live = s_pos[row] >= 0;
    const float rs = s_rs[row], tr = s_tau[row];
    const int col0 = ntw * 16 + l16;
    float sv[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const float z = acc[j][r] * rs;
      sv[j] = -INFINITY;
      if (live) {
        if (a.logits) a.logits[(size_t)row * a.N + col0 + 16 * j] = z;
        sv[j] = tr * z;
      }
    }
    const VStat v = vstat_row16<NT>(sv, col0, live);
    if (l16 == 0) s_stat[wave][row] = v;
  }
  __syncthreads();
  if (threadIdx.x < 16 && s_pos[threadIdx.x] >= 0) {
    VStat v = s_stat[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < NW; ++w) v = vstat_merge(v, s_stat[w][threadIdx.x]);
    a.vpart[(size_t)s_pos[threadIdx.x] * gridDim.x + blockIdx.x] = v;
  }
}

template <typename T, int MT, int NW>
hipError_t launch_nw(const GemmArgs &a, dim3 grid, hipStream_t s) {
  if (a.nt == 1) hipLaunchKernelGGL((lmhead_kernel<T, MT, 1, NW>), grid, dim3(64 * NW), 0, s, a);
  else if (a.nt == 2) hipLaunchKernelGGL((lmhead_kernel<T, MT, 2, NW>), grid, dim3(64 * NW), 0, s, a);
  else if (a.nt == 4) hipLaunchKernelGGL((lmhead_kernel<T, MT, 4, NW>), grid, dim3(64 * NW), 0, s, a);
  else if (MT == 1 && a.nt == 8) hipLaunchKernelGGL((lmhead_kernel<T, 1, 8, NW>), grid, dim3(64 * NW), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int MT>
hipError_t launch_t(const GemmArgs &a, dim3 grid, hipStream_t s) {
  if (a.nw == 4) return launch_nw<T, MT, 4>(a, grid, s);
  if (a.nw == 8) return launch_nw<T, MT, 8>(a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Column groups (one vocabulary-statistics triple per row each) of the LM head.
int lmhead_slices(int N, int nt, int nw) { return N / (16 * nt * nw); }

hipError_t launch_gemm(int dtype, int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (epi != EPI_VSTAT || !norm || a.ssq == nullptr || a.norm_nparts <= 0) return hipErrorInvalidValue;
  if (a.done == nullptr) return hipErrorInvalidValue;
  if (a.nt < 1 || a.nw < 1 || a.N % (16 * a.nt * a.nw) || a.K % 32 || a.M <= 0) return hipErrorInvalidValue;
  if (a.nt == LDS_NT && a.nw == LDS_NW) {   // few rows, activations staged in LDS
    if (dtype != DT_BF16 || a.M > 16 || a.K > LDS_KMAX || a.rowpos == nullptr || a.norm_nparts > 128)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(lmhead_lds_kernel, dim3(lmhead_slices(a.N, a.nt, a.nw)), dim3(64 * LDS_NW), 0, s, a);
    return hipGetLastError();
  }
  const int mt = a.M <= 16 ? 1 : 4;
  const dim3 grid(lmhead_slices(a.N, a.nt, a.nw), 1, (a.M + 16 * mt - 1) / (16 * mt));
  if (dtype == DT_BF16) return mt == 1 ? launch_t<bf16_t, 1>(a, grid, s) : launch_t<bf16_t, 4>(a, grid, s);
  return mt == 1 ? launch_t<float, 1>(a, grid, s) : launch_t<float, 4>(a, grid, s);
}

}  // namespace td
