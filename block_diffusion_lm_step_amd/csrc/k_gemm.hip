// Weight-streaming MFMA GEMM: Y[M][N] = A[M][K] * W[N][K]^T with fused prologue/epilogues,
// used for the four layer projections and for the LM head.
//
// The denoiser's projections (fused QKV, output, MLP up/down) and the LM head are the
// dense contractions of the step.  At the block sizes of the method (B = 16 rows per
// sequence) they read every weight once per step and do ~2*M FLOP per weight element,
// so for M up to a few hundred rows the weight stream from HBM is the bound:
//   * weights are pre-packed in 16x32 MFMA tiles, so a wave's fragment load is one
//     contiguous KiB and a column tile's whole K range is one contiguous block;
//   * per chunk of k-tiles a workgroup stages the activation rows ONCE in LDS, already
//     normalised and split (bf16 high part + bf16 remainder against bf16 weights, fp32
//     as is against fp32 weights), while the next chunk's weights and activations are
//     in flight;
//   * wide outputs (the LM head): the 4 waves own different column tiles (NT each) and
//     share every staged chunk;  narrower outputs (the layer projections): the 4 waves
//     own the same NT column tiles and take different k-tiles of each chunk, and their
//     accumulators are summed through LDS in wave order.  Nothing is split across
//     workgroups: a cross-workgroup reduction needs a device-scope release fence per
//     workgroup, which costs more here than the whole weight stream;
//   * prologue: RMSNorm of the fp32 residual stream, with the row scale taken from the
//     partial sums of squares the producer of x left behind;
//   * epilogues (fp32): store (q/k/v), exact GELU (MLP up), residual add + partial sums
//     of squares (output projection, MLP down), or the LM head's tau-scaled vocabulary
//     statistics (max, sum of exp, lowest argmax) per row and column group.
#include "td_device.h"
#include "td_kernels.h"

#include <type_traits>

namespace td {

namespace {

// k-tiles per wave per chunk: 8 KiB of weights per wave per chunk at 16 rows when the
// waves share the chunk, 4 KiB when they split it (the chunk is then 4x as deep), and
// a quarter of that at 64 rows, so that the two LDS activation buffers stay small.
template <int MT, int NT, bool WK> constexpr int chunk_ktiles() {
  constexpr int base = (WK ? 4 : 8) / (MT == 1 ? 1 : 4);
  return base / NT > 0 ? base / NT : 1;
}

// One 8-element activation fragment in LDS: hi|lo bf16 parts, or 8 fp32 values.
struct alignas(16) LdsFrag {
  uint4 p0, p1;
};

template <typename T> TD_DEV void afrag_store(LdsFrag &d, const AFrag<T> &f);
template <> TD_DEV void afrag_store<bf16_t>(LdsFrag &d, const AFrag<bf16_t> &f) {
  d.p0 = f.hi.raw;
  d.p1 = f.lo.raw;
}
template <> TD_DEV void afrag_store<float>(LdsFrag &d, const AFrag<float> &f) {
  d.p0 = __builtin_bit_cast(uint4, f.f.lo);
  d.p1 = __builtin_bit_cast(uint4, f.f.hi);
}
template <typename T> TD_DEV AFrag<T> afrag_load(const LdsFrag &s);
template <> TD_DEV AFrag<bf16_t> afrag_load<bf16_t>(const LdsFrag &s) {
  AFrag<bf16_t> f;
  f.hi.raw = s.p0;
  f.lo.raw = s.p1;
  return f;
}
template <> TD_DEV AFrag<float> afrag_load<float>(const LdsFrag &s) {
  AFrag<float> f;
  f.f.lo = __builtin_bit_cast(float4, s.p0);
  f.f.hi = __builtin_bit_cast(float4, s.p1);
  return f;
}

// WK: the 4 waves split each chunk's k-tiles (same NT column tiles); otherwise they
// split the column tiles (4 x NT per workgroup) and share each chunk.
template <typename T, int MT, int NT, int EPI, bool NORM, bool WK>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  constexpr int ROWS = 16 * MT;
  constexpr int KC = chunk_ktiles<MT, NT, WK>();   // k-tiles per wave per chunk
  constexpr int CK = WK ? 4 * KC : KC;             // k-tiles per chunk
  constexpr int NFRAG = MT * CK * 64;              // activation fragments per chunk
  constexpr int FPT = (NFRAG + 255) / 256;         // ... staged per thread
  if (a.done && *a.done) return;
  const int M = a.n_rows ? *a.n_rows : a.M;
  const int m0 = blockIdx.z * ROWS;
  if (m0 >= M) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int KT = a.K >> 5;
  const int kbeg = 0, kend = KT;
  const int nchunks = (KT + CK - 1) / CK;
  const int kw = WK ? wave * KC : 0;                                 // wave's first k-tile in a chunk
  const int nt0 = WK ? blockIdx.x * NT : blockIdx.x * 4 * NT + wave;   // wave's tiles: nt0 + NTS j
  constexpr int NTS = WK ? 1 : 4;

  __shared__ int s_row[ROWS];
  __shared__ float s_rs[ROWS];
  __shared__ LdsFrag s_a[2][NFRAG];

  // Rows of this workgroup (gathered through the row list for the LM head) and, with
  // the RMSNorm prologue, their scales 1/sqrt(mean(x^2) + eps) in a fixed order.
  {
    constexpr int TPR = 256 / ROWS;   // threads per row
    const int r = threadIdx.x / TPR, sub = threadIdx.x % TPR;
    int row = -1;
    if (m0 + r < M) row = a.rowlist ? a.rowlist[m0 + r] : m0 + r;
    if constexpr (NORM) {
      float acc = 0.f;
      if (row >= 0)
        for (int p = sub; p < a.norm.nparts; p += TPR) acc += a.norm.ssq[(size_t)p * a.ld_ssq + row];
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o);
      if (sub == 0) s_rs[r] = 1.0f / sqrtf(acc / (float)a.K + a.norm.eps);
    }
    if (sub == 0) s_row[r] = row;
    __syncthreads();
  }

  // Activation staging: fragment f (mt, kt, lane) of a chunk <- rows m0 + 16 mt + lane%16.
  float xr[FPT][8];
  Frag<T> gr[FPT];
  auto load_x = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      const int f = threadIdx.x + 256 * i;
      const int fl = f & 63, kt = (f >> 6) % CK, mt = min(f / (64 * CK), MT - 1);
      const int row = s_row[mt * 16 + (fl & 15)];
      const int k = (kbeg + c * CK + kt) * 32 + (fl >> 4) * 8;
      if (f < NFRAG && row >= 0 && kbeg + c * CK + kt < kend) {
        load8f((NORM ? a.norm.x : a.A) + (size_t)row * (NORM ? a.K : a.lda) + k, xr[i]);
        if constexpr (NORM) gr[i].load(reinterpret_cast<const T *>(a.norm.gain) + k);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xr[i][j] = 0.f;
        if constexpr (NORM) gr[i].zero();
      }
    }
  };
  auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      const int f = threadIdx.x + 256 * i;
      if (f >= NFRAG) break;
      const int fl = f & 63, mt = f / (64 * CK);
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = xr[i][j];
      if constexpr (NORM) {
        const float r = s_rs[mt * 16 + (fl & 15)];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] * r * gr[i].get(j);
      }
      AFrag<T> af;
      af.set8(v);
      afrag_store<T>(s_a[buf][f], af);
    }
  };

  // Weight fragments of this wave's NT column tiles.
  const T *Wp = reinterpret_cast<const T *>(a.Wp) + (size_t)lane * 8;
  Frag<T> wb[2][KC][NT];
  auto issue_w = [&](auto bufc, int c) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
#pragma unroll
    for (int kt = 0; kt < KC; ++kt) {
      const int k = kbeg + c * CK + kw + kt;
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (k < kend) wb[b][kt][j].load(Wp + ((size_t)(nt0 + NTS * j) * KT + k) * 512);
    }
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[mt][j] = zero4();

  auto compute = [&](auto bufc, int c) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    const LdsFrag *sa = s_a[c & 1];
#pragma unroll
    for (int kt = 0; kt < KC; ++kt) {
      if (kbeg + c * CK + kw + kt < kend) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const AFrag<T> af = afrag_load<T>(sa[(mt * CK + kw + kt) * 64 + lane]);
#pragma unroll
          for (int j = 0; j < NT; ++j) acc[mt][j] = mma_a(af, wb[b][kt][j], acc[mt][j]);
        }
      }
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  // Chunk c's activations live in LDS buffer c & 1, its weights in register buffer c & 1.
  // A buffer is rewritten only after the barrier that follows every wave's last read of it.
  if (nchunks > 0) {
    load_x(0);
    issue_w(B0{}, 0);
    store_x(0);
  }
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) {
      load_x(c + 1);
      issue_w(B1{}, c + 1);
    }
    __syncthreads();
    compute(B0{}, c);
    if (c + 1 < nchunks) {
      store_x(1);
      if (c + 2 < nchunks) {
        load_x(c + 2);
        issue_w(B0{}, c + 2);
      }
      __syncthreads();
      compute(B1{}, c + 1);
      if (c + 2 < nchunks) store_x(0);
    }
  }

  // ---------------------------------------------------------------- wave reduction (WK)
  if constexpr (WK) {
    static_assert(sizeof(s_a) >= 3 * MT * NT * 64 * sizeof(f32x4_t), "the wave reduction reuses LDS");
    f32x4_t *s_red = reinterpret_cast<f32x4_t *>(&s_a[0][0]);
    __syncthreads();   // every wave is done reading the staged activations
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) s_red[(((wave - 1) * MT + mt) * NT + j) * 64 + lane] = acc[mt][j];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[mt][j] += s_red[((w * MT + mt) * NT + j) * 64 + lane];
  }

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == EPI_VSTAT) {
    static_assert(!WK, "vocabulary statistics need the column-split layout");
    __shared__ VStat s_stat[4][ROWS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = mt * 16 + 4 * g + r;
        const int row = s_row[rr];
        const float tau = (row >= 0 && a.inv_temp) ? a.inv_temp[row] : 1.0f;
        VStat v{-INFINITY, 0.f, 0x7FFFFFFF};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int col = (nt0 + NTS * j) * 16 + l16;
          const float z = acc[mt][j][r];
          float sv = -INFINITY;
          if (row >= 0) {
            if (a.logits) a.logits[(size_t)row * a.N + col] = z;
            sv = tau * z;
          }
          float mx = sv;
          mx = fmaxf(mx, __shfl_xor(mx, 1)); mx = fmaxf(mx, __shfl_xor(mx, 2));
          mx = fmaxf(mx, __shfl_xor(mx, 4)); mx = fmaxf(mx, __shfl_xor(mx, 8));
          const float se = sum16(row >= 0 ? __expf(sv - mx) : 0.f);
          int am = (row >= 0 && sv == mx) ? col : 0x7FFFFFFF;
          am = min(am, __shfl_xor(am, 1)); am = min(am, __shfl_xor(am, 2));
          am = min(am, __shfl_xor(am, 4)); am = min(am, __shfl_xor(am, 8));
          v = vstat_merge(v, VStat{mx, se, am});
        }
        if (l16 == 0) s_stat[wave][rr] = v;
      }
    __syncthreads();
    if (threadIdx.x < ROWS && s_row[threadIdx.x] >= 0) {
      VStat v = s_stat[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < 4; ++w) v = vstat_merge(v, s_stat[w][threadIdx.x]);
      a.vpart[(size_t)(m0 + threadIdx.x) * gridDim.x + blockIdx.x] = v;
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int nt = nt0 + NTS * j;
        const int col = nt * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + mt * 16 + 4 * g + r;
          const bool ok = row < M;
          const float y = acc[mt][j][r];
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
            if (ok && l16 == 0) a.ssq_out[(size_t)nt * a.M + row] = sq;
          }
        }
      }
  }
}

template <typename T, int MT, int NT>
hipError_t launch_typed(int epi, bool norm, const GemmArgs &a, dim3 grid, hipStream_t s) {
#define TD_L(E, NRM, WKV)                                                                     \
  if (epi == E && norm == NRM) {                                                         \
    hipLaunchKernelGGL((gemm_kernel<T, MT, NT, E, NRM, WKV>), grid, dim3(256), 0, s, a); \
    return hipGetLastError();                                                            \
  }
  TD_L(EPI_VSTAT, true, false)
#undef TD_L
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_t(int epi, bool norm, const GemmArgs &a, dim3 grid, int mt, hipStream_t s) {
  if (a.nt == 1) return mt == 1 ? launch_typed<T, 1, 1>(epi, norm, a, grid, s) : launch_typed<T, 4, 1>(epi, norm, a, grid, s);
  if (a.nt == 2) return mt == 1 ? launch_typed<T, 1, 2>(epi, norm, a, grid, s) : launch_typed<T, 4, 2>(epi, norm, a, grid, s);
  if (a.nt == 4) return mt == 1 ? launch_typed<T, 1, 4>(epi, norm, a, grid, s) : launch_typed<T, 4, 4>(epi, norm, a, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int dtype, int epi, bool norm, const GemmArgs &a, hipStream_t s) {
  const int cols_per_wg = (epi == EPI_VSTAT ? 64 : 16) * a.nt;
  if (a.N % cols_per_wg || a.K % 32 || a.M <= 0) return hipErrorInvalidValue;
  const int mt = a.M <= 16 ? 1 : 4;
  dim3 grid(a.N / cols_per_wg, 1, (a.M + 16 * mt - 1) / (16 * mt));
  return dtype == DT_BF16 ? launch_t<bf16_t>(epi, norm, a, grid, mt, s) : launch_t<float>(epi, norm, a, grid, mt, s);
}

}  // namespace td
