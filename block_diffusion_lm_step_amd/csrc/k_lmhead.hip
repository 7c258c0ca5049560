// LM head fused with the vocabulary softmax statistics, and the on-device commit.
//
// Confidence of a masked position = largest softmax probability of its logits scaled by
// the position's inverse temperature; prediction = lowest vocabulary id of the largest
// scaled logit.  The final-normed hidden state is fp32 (hi + lo bf16 parts against the
// bf16 head).  Each 16-column logit tile stays in the MFMA accumulators: the epilogue
// scales it by tau and reduces it to (max, sum exp(s - max), argmax) per row, merges the
// four waves' tiles, and writes one 12-byte triple per (row, 64-column slice).  The
// [rows x V] logit matrix never reaches HBM (except in the optional debug capture).
//
// The merge kernel combines the slices of a row in a fixed tree order; the last
// workgroup to finish (integer counter) applies the adoption rule of PredNext
// "人工知能は拡散言語モデルの夢を見るか？", section 拡散言語モデルで推論するには
// (adopt masked positions whose confidence clears the threshold, the others stay
// [MASK]) with the fixed fallback of adopting the single most confident masked
// position when none clears it, then rebuilds the list of still-masked rows for the
// next step, so the block loop needs no host round-trip.
#include "td_device.h"
#include "td_kernels.h"

#include <type_traits>

namespace td {

namespace {

constexpr int CH = 4;

// Grid: x = 64-column vocabulary slices (one 16-column tile per wave), y = groups of 16
// still-masked rows (a group past the live row count exits at once).
template <typename T>
__global__ __launch_bounds__(256) void lmhead_kernel(LmArgs a) {
  if (*a.st.done) return;
  const int n_rows = *a.st.n_rows;
  const int m0 = blockIdx.y * 16;
  if (m0 >= n_rows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nt = blockIdx.x * 4 + wave;
  const int KT = a.d >> 5;
  const T *Wp = reinterpret_cast<const T *>(a.Wp) + ((size_t)nt * KT) * 512 + (size_t)lane * 8;
  const int col = nt * 16 + l16;

  __shared__ float s_rs[16];
  __shared__ int s_row[16];
  __shared__ VStat s_stat[4][16];

  {  // rows of this group and their RMSNorm scales
    const int r = threadIdx.x >> 2, sub = threadIdx.x & 3;
    float acc = 0.f;
    int row = -1;
    if (r < 16 && m0 + r < n_rows) {
      row = a.st.rowlist[m0 + r];
      for (int p = sub; p < a.norm.nparts; p += 4) acc += a.norm.ssq[(size_t)p * (a.n * a.B) + row];
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (r < 16 && sub == 0) {
      s_rs[r] = 1.0f / sqrtf(acc / (float)a.d + a.norm.eps);
      s_row[r] = row;
    }
    __syncthreads();
  }
  const int arow = s_row[l16];
  const float ars = s_rs[l16];

  auto load_a = [&](int kt) __attribute__((always_inline)) {
    AFrag<T> f;
    if (arow < 0) { f.zero(); return f; }
    const int k = kt * 32 + g * 8;
    float v[8];
    load8f(a.norm.x + (size_t)arow * a.d + k, v);
    Frag<T> gg;
    gg.load(reinterpret_cast<const T *>(a.norm.gain) + k);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * ars * gg.get(j);
    f.set8(v);
    return f;
  };

  f32x4_t acc = zero4();
  Frag<T> wb[2][CH];
  AFrag<T> ab[2][CH];
  auto issue = [&](auto buf, int c) __attribute__((always_inline)) {
    constexpr int b = decltype(buf)::value;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int kt = c * CH + j;
      if (kt < KT) {
        wb[b][j].load(Wp + (size_t)kt * 512);
        ab[b][j] = load_a(kt);
      }
    }
  };
  auto compute = [&](auto buf, int c) __attribute__((always_inline)) {
    constexpr int b = decltype(buf)::value;
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (c * CH + j < KT) acc = mma_a(ab[b][j], wb[b][j], acc);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const int nchunks = (KT + CH - 1) / CH;
  issue(B0{}, 0);
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) issue(B1{}, c + 1);
    compute(B0{}, c);
    if (c + 1 < nchunks) {
      if (c + 2 < nchunks) issue(B0{}, c + 2);
      compute(B1{}, c + 1);
    }
  }

  // Epilogue: tau-scaled statistics of each row over this wave's 16 columns.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = 4 * g + r;      // row slot within the group
    const int row = s_row[rr];
    const float z = acc[r];
    float sv = -INFINITY;
    if (row >= 0) {
      if (a.logits) a.logits[(size_t)row * a.V + col] = z;
      sv = (a.inv_temp ? a.inv_temp[row] : 1.0f) * z;
    }
    float mx = sv;
    mx = fmaxf(mx, __shfl_xor(mx, 1)); mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4)); mx = fmaxf(mx, __shfl_xor(mx, 8));
    const float e = (row >= 0) ? __expf(sv - mx) : 0.f;
    const float se = sum16(e);
    int am = (row >= 0 && sv == mx) ? col : 0x7FFFFFFF;
    am = min(am, __shfl_xor(am, 1)); am = min(am, __shfl_xor(am, 2));
    am = min(am, __shfl_xor(am, 4)); am = min(am, __shfl_xor(am, 8));
    if (l16 == 0) s_stat[wave][rr] = VStat{mx, se, am};
  }
  __syncthreads();
  if (threadIdx.x < 16 && s_row[threadIdx.x] >= 0) {
    VStat v = s_stat[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < 4; ++w) v = vstat_merge(v, s_stat[w][threadIdx.x]);
    reinterpret_cast<VStat *>(a.vpart)[(size_t)(m0 + threadIdx.x) * gridDim.x + blockIdx.x] = v;
  }
}

__global__ __launch_bounds__(256) void merge_commit_kernel(CommitArgs a) {
  if (*a.st.done) return;
  __shared__ VStat s_v[256];
  __shared__ int s_wave[4];
  __shared__ int s_last;
  const int n_rows = *a.st.n_rows;
  const int b = blockIdx.x;
  if (b < n_rows) {
    const VStat *vp = reinterpret_cast<const VStat *>(a.vpart) + (size_t)b * a.nslices;
    VStat v{-INFINITY, 0.f, 0x7FFFFFFF};
    for (int i = threadIdx.x; i < a.nslices; i += 256) v = vstat_merge(v, vp[i]);
    s_v[threadIdx.x] = v;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) s_v[threadIdx.x] = vstat_merge(s_v[threadIdx.x], s_v[threadIdx.x + w]);
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      a.conf_row[b] = 1.0f / s_v[0].s;
      a.arg_row[b] = s_v[0].a;
    }
  }
  // Last workgroup to arrive applies the commit rule for the whole batch.
  __threadfence();
  if (threadIdx.x == 0) s_last = (atomicAdd(a.st.counter, 1u) == gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (threadIdx.x == 0) atomicExch(a.st.counter, 0u);
  const int t = *a.st.t;
  for (int i = threadIdx.x; i < a.n; i += blockDim.x) {
    bool any_masked = false, any_clear = false;
    float best = -INFINITY;
    int best_p = -1;
    for (int p = 0; p < a.B; ++p) {
      const int r = i * a.B + p;
      const int pos = a.st.rowpos[r];
      if (a.committed[r] || pos < 0) continue;   // pos < 0: row rejected by the state check
      const float c = a.conf_row[pos];
      if (a.conf_out) a.conf_out[r] = c;
      if (a.argmax_out) a.argmax_out[r] = a.arg_row[pos];
      any_masked = true;
      if (c >= a.gamma) any_clear = true;
      if (c > best) { best = c; best_p = p; }
    }
    for (int p = 0; p < a.B; ++p) {
      const int r = i * a.B + p;
      bool adopt = false;
      const int pos = a.st.rowpos[r];
      if (!a.committed[r] && pos >= 0) {
        adopt = any_clear ? (a.conf_row[pos] >= a.gamma) : (p == best_p);
        if (adopt) {
          a.tokens[r] = a.arg_row[pos];
          a.committed[r] = 1;
          if (a.commit_step) a.commit_step[r] = (int8_t)t;
        }
      }
      if (a.newly) a.newly[r] = adopt ? 1 : 0;
    }
    if (a.steps && any_masked) a.steps[i] += 1;
  }
  __syncthreads();
  // Rows still masked, in row order, for the next step.
  const int M = a.n * a.B;
  int base = 0;
  for (int r0 = 0; r0 < M; r0 += blockDim.x) {
    const int r = r0 + threadIdx.x;
    const bool masked = r < M && !a.committed[r];
    base = block_compact(masked, base, a.st.rowlist, a.st.rowpos, r < M ? r : -1, s_wave);
  }
  if (threadIdx.x == 0) {
    *a.st.n_rows = base;
    *a.st.done = base == 0 ? 1 : 0;
    *a.st.t = t + 1;
  }
}

}  // namespace

hipError_t launch_lmhead(int dtype, const LmArgs &a, hipStream_t s) {
  if (a.V % 64 || a.d % 32) return hipErrorInvalidValue;
  dim3 grid(a.V / 64, (a.n * a.B + 15) / 16);
  if (dtype == DT_BF16) hipLaunchKernelGGL(lmhead_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(lmhead_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge_commit(const CommitArgs &a, int max_rows, hipStream_t s) {
  hipLaunchKernelGGL(merge_commit_kernel, dim3(max_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace td
