// Layer projections at block-sized M: Y[M][N] = A[M][K] * W[N][K]^T, weights in flight
// all at once.
//
// With B = 16 rows per sequence the fused QKV, output and MLP projections read every
// weight once per step and do only ~2*M FLOP per weight element: the time is the
// latency and bandwidth of the weight stream.  Each workgroup owns one 16-column tile
// and the whole K range; its NW waves split K, and every wave issues the loads of its
// whole weight slice (pre-packed 16x32 MFMA tiles: one contiguous KiB per load) before
// it touches the activations, so that chip-wide most of the matrix is in flight at
// once.  Activation fragments (fp32 rows of the residual stream through the fused
// RMSNorm, or fp32 attention output / MLP activation) are loaded from L2 in groups
// while the weights arrive, split into a bf16 high part and a bf16 remainder against
// bf16 weights (kept fp32 against fp32 weights), and multiplied into one accumulator
// per 16-row tile.  The waves' accumulators are summed through LDS in wave order (no
// cross-workgroup reduction, no device-scope fence, deterministic), and wave 0 applies
// the epilogue: store (q/k/v), exact GELU (MLP up), or residual add + partial sums of
// squares of the new residual rows for the next RMSNorm (output projection, MLP down).
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

template <typename T, int MT, int NW, int EPI, bool NORM>
__global__ __launch_bounds__(64 * NW) void gemm_wk_kernel(GemmArgs a) {
  // k-tiles of weights a wave holds in flight at once, and k-tiles of activations per
  // load group, sized to the register file (1024-thread workgroups get 128 VGPRs).
  constexpr int PASS = NW < 16 ? 16 : (MT == 4 ? 4 : (NORM ? 8 : 16));
  constexpr int AG = MT == 4 ? 1 : (NW == 16 ? 2 : 4);
  if (a.done && *a.done) return;
  const int M = a.M;
  const int m0 = blockIdx.z * 16 * MT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nt = blockIdx.x;
  const int KT = a.K >> 5;
  const int kwt = (KT + NW - 1) / NW;          // k-tiles per wave
  const int kw0 = wave * kwt, kw1 = min(KT, kw0 + kwt);

  __shared__ float s_rs[16 * MT];
  __shared__ f32x4_t s_red[NW - 1][MT][64];

  if constexpr (NORM) {
    // Row scale 1/sqrt(mean(x^2) + eps) from the producer's partial sums of squares:
    // 16 threads per row, fixed order.
    for (int r0 = 0; r0 < 16 * MT; r0 += 4 * NW) {
      const int r = r0 + (threadIdx.x >> 4), sub = threadIdx.x & 15;
      float acc = 0.f;
      if (r < 16 * MT && m0 + r < M)
        for (int p = sub; p < a.norm.nparts; p += 16) acc += a.norm.ssq[(size_t)p * a.ld_ssq + m0 + r];
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      acc += __shfl_xor(acc, 8);
      if (r < 16 * MT && sub == 0) s_rs[r] = 1.0f / sqrtf(acc / (float)a.K + a.norm.eps);
    }
    __syncthreads();
  }

  const T *Wp = reinterpret_cast<const T *>(a.Wp) + ((size_t)nt * KT) * 512 + (size_t)lane * 8;
  const float *Abase = NORM ? a.norm.x : a.A;
  const int lda = NORM ? a.K : a.lda;

  // Raw activation fragments (8 fp32) of rows m0 + 16 mt + lane%16 for k-tile kt.
  auto load_a = [&](float (&v)[8], int mt, int kt) __attribute__((always_inline)) {
    const int row = m0 + mt * 16 + l16;
    if (row < M && kt < kw1) {
      load8f(Abase + (size_t)row * lda + kt * 32 + g * 8, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
  };
  auto to_frag = [&](const float (&v)[8], int mt, int kt) __attribute__((always_inline)) {
    AFrag<T> f;
    if constexpr (NORM) {
      float u[8];
      Frag<T> gg;
      gg.load(reinterpret_cast<const T *>(a.norm.gain) + kt * 32 + g * 8);
      const float r = s_rs[mt * 16 + l16];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = v[j] * r * gg.get(j);
      f.set8(u);
    } else {
      f.set8(v);
    }
    return f;
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = zero4();

  for (int p0 = kw0; p0 < kw1; p0 += PASS) {
    // Whole pass of weights in flight first.
    Frag<T> wb[PASS];
#pragma unroll
    for (int i = 0; i < PASS; ++i)
      if (p0 + i < kw1) wb[i].load(Wp + (size_t)(p0 + i) * 512);
    // Activations in groups of AG k-tiles, one group ahead.
    float xa[2][AG][MT][8];
#pragma unroll
    for (int i = 0; i < AG; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) load_a(xa[0][i][mt], mt, p0 + i);
#pragma unroll
    for (int gi = 0; gi < PASS / AG; ++gi) {
      const int cur = gi & 1;
      if (p0 + (gi + 1) * AG < kw1 && gi + 1 < PASS / AG) {
#pragma unroll
        for (int i = 0; i < AG; ++i)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) load_a(xa[cur ^ 1][i][mt], mt, p0 + (gi + 1) * AG + i);
      }
#pragma unroll
      for (int i = 0; i < AG; ++i) {
        const int kt = p0 + gi * AG + i;
        if (kt < kw1) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = mma_a(to_frag(xa[cur][i][mt], mt, kt), wb[gi * AG + i], acc[mt]);
        }
      }
    }
  }

  // Waves' partial sums, in wave order.
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s_red[wave - 1][mt][lane] = acc[mt];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < NW - 1; ++w)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] += s_red[w][mt][lane];

  const int col = nt * 16 + l16;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + mt * 16 + 4 * g + r;
      const bool ok = row < M;
      const float y = acc[mt][r];
      float *op = a.out + (size_t)row * a.ldo + col;
      if constexpr (EPI == EPI_STORE) {
        if (ok) *op = y;
      } else if constexpr (EPI == EPI_GELU) {
        if (ok) *op = gelu_erf(y);
      } else {
        float xv = 0.f;
        if (ok) {
          xv = *op + y;
          *op = xv;
        }
        const float sq = sum16(xv * xv);
        if (ok && l16 == 0) a.ssq_out[(size_t)nt * M + row] = sq;
      }
    }
  }
}

template <typename T, int MT, int NW>
hipError_t launch_nw(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  const dim3 grid(a.N / 16, 1, (a.M + 16 * MT - 1) / (16 * MT));
#define TD_L(E, NRM)                                                                           \
  if (epi == E && norm == NRM) {                                                           \
    hipLaunchKernelGGL((gemm_wk_kernel<T, MT, NW, E, NRM>), grid, dim3(64 * NW), 0, s, a); \
    return hipGetLastError();                                                              \
  }
  TD_L(EPI_STORE, true)
  TD_L(EPI_GELU, true)
  TD_L(EPI_RESID, false)
#undef TD_L
  return hipErrorInvalidValue;
}

template <typename T, int MT>
hipError_t launch_mt(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.nw == 4) return launch_nw<T, MT, 4>(epi, norm, a, s);
  if (a.nw == 8) return launch_nw<T, MT, 8>(epi, norm, a, s);
  if (a.nw == 16) return launch_nw<T, MT, 16>(epi, norm, a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_wk(int dtype, int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.N % 16 || a.K % 32 || a.M <= 0) return hipErrorInvalidValue;
  const bool small = a.M <= 16;
  if (dtype == DT_BF16) return small ? launch_mt<bf16_t, 1>(epi, norm, a, s) : launch_mt<bf16_t, 4>(epi, norm, a, s);
  return small ? launch_mt<float, 1>(epi, norm, a, s) : launch_mt<float, 4>(epi, norm, a, s);
}

}  // namespace td
