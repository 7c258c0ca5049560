// Weight-streaming MFMA GEMM: Y[M][N] = A[M][K] * W[N][K]^T with fused prologue/epilogue.
//
// The denoiser's projections (fused QKV, output, MLP up/down) are the only dense
// contractions of the step besides the LM head.  At the block sizes of the method
// (B = 16 rows per sequence) they read every weight once per step and do ~2*M FLOP per
// weight element, so for M up to a few hundred rows the weight stream from HBM is the
// bound and the kernel is shaped for it:
//   * weights are pre-packed in 16x32 MFMA tiles, so each lane's fragment is one
//     contiguous 16-byte load and a wave reads 1 KiB contiguous per tile;
//   * one workgroup owns one 16-column tile and a range of 32-wide k-tiles; its four
//     waves interleave over that range and are summed through LDS in a fixed order;
//   * when N/16 tiles cannot fill the chip, K is also split across workgroups; the last
//     workgroup of a tile (integer counter) adds the split partials in split order, so
//     results are deterministic and no float atomics are used;
//   * activations are fp32; for bf16 weights each activation fragment enters the MFMA
//     as a bf16 high part plus a bf16 remainder (two MFMAs per weight fragment, free
//     while the weight stream is the bound), so no activation is ever rounded to bf16;
//   * prologue: RMSNorm of the fp32 residual stream (row scale from the partial sums of
//     squares left by the producer) fused into the A-fragment load;
//   * epilogue (fp32 out): store (q/k/v), GELU (MLP up), or residual add + partial sums
//     of squares for the next RMSNorm (output projection, MLP down).
#include "td_device.h"
#include "td_kernels.h"

#include <type_traits>

namespace td {

namespace {

constexpr int KTW_MAX = 16;   // k-tiles per wave

// A fragment of rows m0 + 16 mt + (lane % 16), k-tile kt: fp32 activations (or the RMSNorm
// of the residual stream), split for the bf16 MFMA.
template <typename T, bool NORM>
struct AOperand {
  const GemmArgs &a;
  const float *rs;   // LDS row scales (NORM)
  int m0, lane;
  TD_DEV AFrag<T> load(int mt, int kt) const {
    AFrag<T> f;
    const int row = m0 + mt * 16 + (lane & 15);
    const int k = kt * 32 + (lane >> 4) * 8;
    if (row >= a.M) { f.zero(); return f; }
    float v[8];
    if constexpr (NORM) {
      load8f(a.norm.x + (size_t)row * a.K + k, v);
      Frag<T> g;
      g.load(reinterpret_cast<const T *>(a.norm.gain) + k);
      const float r = rs[mt * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * r * g.get(j);
    } else {
      load8f(a.A + (size_t)row * a.lda + k, v);
    }
    f.set8(v);
    return f;
  }
};

template <typename T, int MT, int EPI, bool NORM>
__global__ __launch_bounds__(256) void gemm_ws_kernel(GemmArgs a) {
  constexpr int CH = MT == 1 ? 4 : 2;   // k-tiles per pipeline chunk
  if (a.done && *a.done) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = blockIdx.x, ks = blockIdx.y;
  const int m0 = blockIdx.z * 16 * MT;
  const int KT = a.K >> 5;
  const int kbeg = ks * 4 * a.ktw;
  const int kend = min(KT, kbeg + 4 * a.ktw);

  __shared__ float s_rs[16 * MT];
  __shared__ f32x4_t s_red[3][MT][64];

  if constexpr (NORM) {
    // Row scale 1/sqrt(mean(x^2) + eps): four threads per row, fixed summation order.
    const int r = threadIdx.x >> 2, sub = threadIdx.x & 3;
    float acc = 0.f;
    if (r < 16 * MT && m0 + r < a.M)
      for (int p = sub; p < a.norm.nparts; p += 4) acc += a.norm.ssq[(size_t)p * a.M + m0 + r];
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (r < 16 * MT && sub == 0) s_rs[r] = 1.0f / sqrtf(acc / (float)a.K + a.norm.eps);
    __syncthreads();
  }

  AOperand<T, NORM> A{a, s_rs, m0, lane};
  const T *Wp = reinterpret_cast<const T *>(a.Wp) + ((size_t)nt * KT) * 512 + (size_t)lane * 8;

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = zero4();

  // Wave `wave` owns k-tiles kbeg + wave + 4*i; chunks of CH tiles, next chunk in flight.
  const int nk = (kend - kbeg - wave + 3) / 4;   // tiles of this wave (may be <= 0)
  Frag<T> wb[2][CH];
  AFrag<T> ab[2][CH][MT];
  // Buffer indices are literals after inlining, so both buffers stay in registers.
  auto issue = [&](auto buf, int c) __attribute__((always_inline)) {
    constexpr int b = decltype(buf)::value;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = c * CH + j;
      if (i < nk) {
        const int kt = kbeg + wave + 4 * i;
        wb[b][j].load(Wp + (size_t)kt * 512);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ab[b][j][mt] = A.load(mt, kt);
      }
    }
  };
  auto compute = [&](auto buf, int c) __attribute__((always_inline)) {
    constexpr int b = decltype(buf)::value;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (c * CH + j < nk) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mma_a(ab[b][j][mt], wb[b][j], acc[mt]);
      }
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const int nchunks = (nk + CH - 1) / CH;
  if (nchunks > 0) issue(B0{}, 0);
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) issue(B1{}, c + 1);
    compute(B0{}, c);
    if (c + 1 < nchunks) {
      if (c + 2 < nchunks) issue(B0{}, c + 2);
      compute(B1{}, c + 1);
    }
  }

  // Sum the four waves in a fixed order.
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s_red[wave - 1][mt][lane] = acc[mt];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] += s_red[w][mt][lane];

  const int col = nt * 16 + (lane & 15);
  const int g = lane >> 4;

  if (a.ksplit > 1) {
    float *part = a.part;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + mt * 16 + 4 * g + r;
        if (row < a.M) part[((size_t)ks * a.M + row) * a.N + col] = acc[mt][r];
      }
    __threadfence();
    unsigned old = 0;
    unsigned *ctr = a.counters + (size_t)blockIdx.z * gridDim.x + nt;
    if (lane == 0) old = atomicAdd(ctr, 1u);
    old = __shfl(old, 0);
    if (old != (unsigned)(a.ksplit - 1)) return;
    __threadfence();
    if (lane == 0) atomicExch(ctr, 0u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + mt * 16 + 4 * g + r;
        float y = 0.f;
        if (row < a.M)
          for (int k2 = 0; k2 < a.ksplit; ++k2) y += part[((size_t)k2 * a.M + row) * a.N + col];
        acc[mt][r] = y;
      }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + mt * 16 + 4 * g + r;
      const bool ok = row < a.M;
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
        if (ok && (lane & 15) == 0) a.ssq_out[(size_t)nt * a.M + row] = sq;
      }
    }
  }
}

template <typename T, int MT>
hipError_t launch_typed(int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  dim3 grid(a.N / 16, a.ksplit, (a.M + 16 * MT - 1) / (16 * MT));
  if (epi == EPI_STORE && norm) hipLaunchKernelGGL((gemm_ws_kernel<T, MT, EPI_STORE, true>), grid, dim3(256), 0, s, a);
  else if (epi == EPI_GELU && norm) hipLaunchKernelGGL((gemm_ws_kernel<T, MT, EPI_GELU, true>), grid, dim3(256), 0, s, a);
  else if (epi == EPI_RESID && !norm) hipLaunchKernelGGL((gemm_ws_kernel<T, MT, EPI_RESID, false>), grid, dim3(256), 0, s, a);
  else if (epi == EPI_STORE && !norm) hipLaunchKernelGGL((gemm_ws_kernel<T, MT, EPI_STORE, false>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int dtype, int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  if (a.N % 16 || a.K % 32 || a.ktw < 1 || a.ktw > KTW_MAX || a.M <= 0) return hipErrorInvalidValue;
  if ((long)a.ksplit * 4 * a.ktw < a.K / 32) return hipErrorInvalidValue;
  const bool small = a.M <= 16;
  if (dtype == DT_BF16) return small ? launch_typed<bf16_t, 1>(epi, norm, a, s) : launch_typed<bf16_t, 4>(epi, norm, a, s);
  return small ? launch_typed<float, 1>(epi, norm, a, s) : launch_typed<float, 4>(epi, norm, a, s);
}

}  // namespace td
