// Vocabulary merge and the on-device commit.
//
// Confidence of a masked position = largest softmax probability of its logits scaled by
// the position's inverse temperature; prediction = lowest vocabulary id of the largest
// scaled logit.  The LM-head GEMM (vocabulary-statistics epilogue) leaves one
// (max, sum exp(s - max), argmax) triple per row and column group, so the [rows x V]
// logit matrix never reaches HBM.
//
// The merge kernel combines the groups of a row in a fixed tree order; the last
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

__global__ __launch_bounds__(256) void merge_commit_kernel(CommitArgs a) {
  if (*a.st.done) return;
  __shared__ VStat s_v[256];
  __shared__ int s_wave[4];
  __shared__ int s_last;
  const int n_rows = *a.st.n_rows;
  const int b = blockIdx.x;
  if (b < n_rows) {
    const VStat *vp = a.vpart + (size_t)b * a.nslices;
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

hipError_t launch_merge_commit(const CommitArgs &a, int max_rows, hipStream_t s) {
  hipLaunchKernelGGL(merge_commit_kernel, dim3(max_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace td
