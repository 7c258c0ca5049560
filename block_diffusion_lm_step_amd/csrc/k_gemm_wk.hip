// Layer projections at block-sized M: Y[M][N] = A[M][K] * W[N][K]^T with the weight
// stream kept in flight.
//
// With B = 16 rows per sequence the fused QKV, output and MLP projections read every
// weight once per step and do only ~2*M FLOP per weight element: the time is the
// latency and bandwidth of the weight stream.  Each workgroup owns NT 16-column tiles
// and the whole K range; its NW waves split K.  Every wave keeps PASS k-tiles of weights
// (pre-packed 16x32 MFMA tiles: one contiguous KiB per load) and of activation fragments
// in flight: a slot
// is refilled right after its MFMAs, so the loads stream without bubbles, and all loads
// are unconditional (clamped addresses) so that the waits the compiler places before
// each MFMA are exact.  One activation fragment feeds NT MFMAs: the activation traffic
// from L2 is 2 KiB per k-tile per wave against NT KiB of weights.
//
// The activations arrive in fragment layout, written by their producer: fp32 values
// split into a bf16 high part and a bf16 remainder against bf16 weights (fp32 as is
// against fp32 weights); a lane's operand is one 32-byte load, no conversion.  A normed
// input is stored by its producer as x * gain (this GEMM's RMSNorm gain); the per-row
// scale 1/sqrt(mean(x^2) + eps) factors out of the sum over K and multiplies the
// accumulator.  It is formed from the producer's partial sums of squares, which are
// loaded before the weights so that waiting for them never waits for the weights.
//
// With a.splits > 1 the K range is also split over workgroups (blockIdx.y: a contiguous
// run of whole k-tiles each) so that few column tiles still fill the chip and each CU
// re-reads less of the activations: the workgroups store fp32 partials
// part[split][M][N] and launch_split_reduce sums them in split order (deterministic)
// and applies the row scale and the epilogue.  (An in-kernel reduction by the last
// workgroup to arrive needs device-scope release/acquire fences, which measured ~10 us.)
//
// The waves' accumulators meet in LDS; wave w sums tile w (and w + NW, ...) over the
// waves in wave order (deterministic, no device-scope fence) and applies the epilogue:
//   STORE  q/k/v (fp32, row-major),
//   GELU   u = gelu_erf(y), written in fragment layout for the MLP down projection,
//   RESID  x += y (fp32 residual stream), partial sums of squares of the new rows per
//          16 columns, and x * (next RMSNorm gain) in fragment layout.
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

// k-tiles in flight per wave: the VGPRs per k-tile (activation fragments of MT row
// tiles + NT weight fragments) into a budget that keeps two 256/512-thread workgroups
// per CU (1024-thread workgroups: one workgroup, 128 VGPRs).  (Every k-tile of a
// 2048-deep wave range in flight at once, one workgroup per CU, measured slower.)
template <typename T, int MT, int NT, int NW> constexpr int wk_pass() {
  constexpr int per = MT * 8 + NT * (sizeof(T) == 2 ? 4 : 8);
  constexpr int budget = NW == 16 ? 72 : 176;
  constexpr int p = budget / per;
  return p > 16 ? 16 : (p < 1 ? 1 : p);
}

template <typename T, int MT, int NT, int NW, int EPI, bool NORM>
__global__ __launch_bounds__(64 * NW) void gemm_wk_kernel(GemmArgs a) {
  constexpr int PASS = wk_pass<T, MT, NT, NW>();
  constexpr int ROWS = 16 * MT;
  constexpr int TPR = (64 * NW / ROWS) < 64 ? 64 * NW / ROWS : 64;   // threads per row (row scales)
  constexpr int SQB = 16;                                             // partial sums loaded per batch
  // The loop-exit flag decides before any operand is requested.  Steps after the block is
  // adopted still launch every kernel; requesting a PASS window of weights before the
  // test made each such launch as long as a working one (measured at the batch-1 tower:
  // 0.3 ms per such step; testing first costs a working launch about 0.2 us).
  if (__hip_atomic_load(a.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
  const int M = a.M;
  const int m0 = blockIdx.z * ROWS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nt0 = blockIdx.x * NT;
  const int KT = a.K >> 5;
  const int ks0 = (int)((int64_t)KT * blockIdx.y / a.splits), ks1 = (int)((int64_t)KT * (blockIdx.y + 1) / a.splits);
  const int kwt = (ks1 - ks0 + NW - 1) / NW;     // k-tiles per wave
  const int kw0 = min(ks1, ks0 + wave * kwt), kw1 = min(ks1, kw0 + kwt);

  __shared__ float s_rs[ROWS];
  __shared__ f32x4_t s_red[NW][MT * NT][64];

  const T *Wl = reinterpret_cast<const T *>(a.Wp) + ((size_t)nt0 * KT) * 512 + (size_t)lane * 8;
  const char *Al = reinterpret_cast<const char *>(a.A) + ((size_t)(m0 >> 4) * KT) * 2048 + (size_t)lane * 32;
  // Loads past the wave's range re-read its last k-tile (unconditional loads keep the
  // compiler's waits exact; they are never multiplied).
  auto clampk = [&](int kt) { return max(0, min(min(kt, kw1 - 1), KT - 1)); };
  AFrag<T> xa[PASS][MT];
  Frag<T> wb[PASS][NT];
  auto fill = [&](int i, int kt) __attribute__((always_inline)) {
    const int k = clampk(kt);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xa[i][mt] = afl_get<T>(Al + ((size_t)mt * KT + k) * 2048);
#pragma unroll
    for (int j = 0; j < NT; ++j) wb[i][j].load_nt(Wl + ((size_t)j * KT + k) * 512);
  };

  // Partial sums of squares of this thread's row first (TPR threads per row).
  const int rr = threadIdx.x / TPR, sub = threadIdx.x % TPR;
  const int srow = min(m0 + rr, M - 1);
  float sq[SQB];
  if constexpr (NORM) {
#pragma unroll
    for (int j = 0; j < SQB; ++j)
      sq[j] = a.ssq[(size_t)min(sub + TPR * j, a.norm_nparts - 1) * a.ld_ssq + srow];
  }
  // First PASS k-tiles of activations and weights.
#pragma unroll
  for (int i = 0; i < PASS; ++i) fill(i, kw0 + i);
  if constexpr (NORM) {
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
  int p0 = kw0;
  for (; p0 + PASS < kw1; p0 += PASS) {
#pragma unroll
    for (int i = 0; i < PASS; ++i) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[mt][j] = mma_a(xa[i][mt], wb[i][j], acc[mt][j]);
      fill(i, p0 + PASS + i);
      // Keep each refill right behind its MFMAs: left alone, the scheduler sinks all
      // refills below the pass's MFMAs and the stream stalls once per pass.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < PASS; ++i) {
    if (p0 + i < kw1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[mt][j] = mma_a(xa[i][mt], wb[i][j], acc[mt][j]);
    }
  }

  // Waves' partial sums meet in LDS; wave w finishes tiles w, w + NW, ... in wave order.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) s_red[wave][mt * NT + j][lane] = acc[mt][j];
  __syncthreads();
  constexpr int QW = (MT * NT + NW - 1) / NW;   // tiles finished per wave
  f32x4_t yq[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int q = wave + NW * i;
    if (q < MT * NT) {
      yq[i] = s_red[0][q][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) yq[i] += s_red[w][q][lane];
    }
  }
  if (a.splits > 1) {   // this split's partial; launch_split_reduce finishes
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int q = wave + NW * i;
      if (q < MT * NT) {
        const int col = (nt0 + q % NT) * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + (q / NT) * 16 + 4 * g + r;
          if (row < M) a.part[((size_t)blockIdx.y * M + row) * a.N + col] = yq[i][r];
        }
      }
    }
    return;
  }

  const int KTo = a.N >> 5;   // k-tiles of a fragment-layout output (its K is this GEMM's N)
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int q = wave + NW * i;
    if (q >= MT * NT) break;
    const int mt = q / NT, j = q % NT;
    const f32x4_t y4 = yq[i];
    const int col = (nt0 + j) * 16 + l16;
    // Residual rows and the next gain, loaded before any store (the compiler cannot
    // tell that the outputs alias nothing and would otherwise serialise the loads).
    float xold[4], gnext = 1.0f;
    if constexpr (EPI == EPI_RESID) {
      gnext = to_f32<T>(reinterpret_cast<const T *>(a.gain_next)[col]);
#pragma unroll
      for (int r = 0; r < 4; ++r) xold[r] = a.out[(size_t)min(m0 + mt * 16 + 4 * g + r, M - 1) * a.ldo + col];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ri = mt * 16 + 4 * g + r;
      const int row = m0 + ri;
      const bool ok = row < M;
      float y = y4[r];
      if constexpr (NORM) y *= s_rs[ri];
      if constexpr (EPI == EPI_STORE) {
        if (ok) a.out[(size_t)row * a.ldo + col] = y;
      } else if constexpr (EPI == EPI_GELU) {
        if (ok) afl_put<T>(a.out_afl, KTo, row, col, gelu_erf(y));
      } else {
        const float xv = ok ? xold[r] + y : 0.f;
        if (ok) {
          a.out[(size_t)row * a.ldo + col] = xv;
          afl_put<T>(a.out_afl, KTo, row, col, xv * gnext);
        }
        const float sq16 = sum16(xv * xv);
        if (ok && l16 == 0) a.ssq_out[(size_t)(nt0 + j) * M + row] = sq16;
      }
    }
  }
}

template <typename T, int MT, int NT, int NW>
hipError_t launch_nw(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  const dim3 grid(a.N / (16 * NT), a.splits, (a.M + 16 * MT - 1) / (16 * MT));
#define TD_L(E, NRM)                                                                               \
  if (epi == E && norm == NRM) {                                                               \
    hipLaunchKernelGGL((gemm_wk_kernel<T, MT, NT, NW, E, NRM>), grid, dim3(64 * NW), 0, s, a); \
    return hipGetLastError();                                                                  \
  }
  TD_L(EPI_STORE, true)
  TD_L(EPI_GELU, true)
  TD_L(EPI_RESID, false)
#undef TD_L
  return hipErrorInvalidValue;
}

template <typename T, int MT, int NT>
hipError_t launch_nt(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.nw == 4) return launch_nw<T, MT, NT, 4>(epi, norm, a, s);
  if (a.nw == 8) return launch_nw<T, MT, NT, 8>(epi, norm, a, s);
  // Four row tiles with 16 waves would spill (128 VGPRs per lane): 8 waves instead.
  if (a.nw == 16) {
    if constexpr (MT == 4) return launch_nw<T, MT, NT, 8>(epi, norm, a, s);
    else return launch_nw<T, MT, NT, 16>(epi, norm, a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int MT>
hipError_t launch_mt(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.nt == 1) return launch_nt<T, MT, 1>(epi, norm, a, s);
  if constexpr (sizeof(T) == 2) {   // several column tiles per workgroup: bf16 towers
    if (a.nt == 2) return launch_nt<T, MT, 2>(epi, norm, a, s);
    if (a.nt == 4) return launch_nt<T, MT, 4>(epi, norm, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_wk(int dtype, int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.N % 32 || a.K % 32 || a.M <= 0 || a.nt < 1 || a.N % (16 * a.nt)) return hipErrorInvalidValue;
  if (a.done == nullptr) return hipErrorInvalidValue;
  if (norm && (a.ssq == nullptr || a.norm_nparts <= 0)) return hipErrorInvalidValue;
  if ((epi == EPI_GELU || epi == EPI_RESID) && a.out_afl == nullptr) return hipErrorInvalidValue;
  // Split K only for bf16 towers (the reduction writes bf16 fragment layout).
  if (a.splits < 1 || a.splits > a.K / 32 || (a.splits > 1 && (a.part == nullptr || dtype != DT_BF16)))
    return hipErrorInvalidValue;
  const bool small = a.M <= 16;
  hipError_t e;
  if (dtype == DT_BF16) e = small ? launch_mt<bf16_t, 1>(epi, norm, a, s) : launch_mt<bf16_t, 4>(epi, norm, a, s);
  else e = small ? launch_mt<float, 1>(epi, norm, a, s) : launch_mt<float, 4>(epi, norm, a, s);
  if (e != hipSuccess || a.splits == 1) return e;
  return launch_split_reduce(epi, norm, a, s);
}

}  // namespace td
