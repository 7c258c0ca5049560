// Vocabulary merge and the on-device commit.
//
// Confidence of a masked position = largest softmax probability of its logits scaled by
// the position's inverse temperature; prediction = lowest vocabulary id of the largest
// scaled logit.  The LM-head GEMM (vocabulary-statistics epilogue) leaves one
// (max, sum exp(s - max), argmax) triple per row and column group, so the [rows x V]
// logit matrix never reaches HBM.
//
// The groups of a row are combined in a fixed tree order; then the adoption rule of
// PredNext "人工知能は拡散言語モデルの夢を見るか？", section 拡散言語モデルで推論するには
// (adopt masked positions whose confidence clears the threshold, the others stay
// [MASK]) with the fixed fallback of adopting the single most confident masked position
// when none clears it -- or one of the variants chosen by td_set_commit_rule: the
// min_adopt most confident forced (the same step names forcing the top few), or the
// lowest masked position only (the mock-AR mode) -- and the list of still-masked rows
// is rebuilt for the next step, so the block loop needs no host round-trip.  Two shapes:
//   * few rows (the block sizes of one or a few sequences): ONE workgroup merges every
//     row (a wave per row, eight groups per lane in flight) and commits: no
//     cross-workgroup synchronisation at all;
//   * many rows: a wave per row merges (four rows per workgroup, no cross-workgroup
//     synchronisation), then a second launch of one workgroup commits for the whole
//     batch.  (A single launch whose last workgroup to finish commits needs a
//     device-scope fence in every workgroup, a write-back of the XCD's L2 each: at
//     2048 rows that launch took 142 us.)
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

// Adoption rule for every sequence, then the compacted list of still-masked rows.
// Called by all threads of one workgroup after conf_row / arg_row are final.  One thread
// per block position; a sequence's B positions are B consecutive lanes of one wave
// (B divides 64 and every pass starts at a multiple of 64), so the rule's reductions --
// is any position at or above gamma, which masked position is the most confident
// (lowest position on ties), is any position still masked -- are lane shuffles.
TD_DEV void commit_all(const CommitArgs &a, int *s_wave) {
  const int t = *a.st.t;
  const int M = a.n * a.B;
  for (int r0 = 0; r0 < M; r0 += blockDim.x) {
    const int r = r0 + threadIdx.x;
    const bool in = r < M;
    const int p = r % a.B;
    const int pos = in ? a.st.rowpos[r] : -1;
    const bool masked = in && !a.committed[r] && pos >= 0;   // pos < 0: row rejected by the state check
    const float c = masked ? a.conf_row[pos] : -INFINITY;
    const int arg = masked ? a.arg_row[pos] : 0;
    // Butterfly over the sequence's B lanes: any position masked, the most confident
    // masked position (lowest on ties), the lowest masked position.
    int any = masked ? 1 : 0;
    float best = c;
    int best_p = masked ? p : 0x7FFFFFFF, first_p = best_p;
    for (int o = 1; o < a.B; o <<= 1) {
      any |= __shfl_xor(any, o);
      const float bo = __shfl_xor(best, o);
      const int po = __shfl_xor(best_p, o);
      if (bo > best || (bo == best && po < best_p)) {
        best = bo;
        best_p = po;
      }
      first_p = min(first_p, __shfl_xor(first_p, o));
    }
    if (masked) {
      if (a.conf_out) a.conf_out[r] = c;
      if (a.argmax_out) a.argmax_out[r] = arg;
    }
    bool adopt;
    if (a.rule == RULE_LEFT_TO_RIGHT) {
      adopt = masked && p == first_p;
    } else if (a.min_adopt <= 1) {   // the most confident one is forced; it clears gamma if any does
      adopt = masked && (c >= a.gamma || p == best_p);
    } else {
      // Rank among the sequence's masked positions by (confidence descending, position
      // ascending); unmasked lanes hold -inf and never outrank a masked one.
      const int lane0 = (int)(threadIdx.x & 63) - p;   // lane of the sequence's position 0
      int rank = 0;
      for (int j = 0; j < a.B; ++j) {
        const float cj = __shfl(c, lane0 + j);
        rank += (cj > c || (cj == c && j < p)) ? 1 : 0;
      }
      adopt = masked && (c >= a.gamma || rank < a.min_adopt);
    }
    if (adopt) {
      a.tokens[r] = arg;
      a.committed[r] = 1;
      if (a.commit_step) a.commit_step[r] = (int8_t)t;
    }
    if (in && a.newly) a.newly[r] = adopt ? 1 : 0;
    if (in && p == 0 && a.steps && any) a.steps[r / a.B] += 1;
    // Finished after this step: no position left masked (attention then skips it).
    int rem = (masked && !adopt) ? 1 : 0;
    for (int o = 1; o < a.B; o <<= 1) rem |= __shfl_xor(rem, o);
    if (in && p == 0) a.st.seq_done[r / a.B] = rem ? 0 : 1;
  }
  __syncthreads();
  // Rows still masked, in row order, for the next step, and the rows of the sequences
  // still active (the next step's layer GEMMs compute only those).
  int base = 0, act = 0;
  for (int r0 = 0; r0 < M; r0 += blockDim.x) {
    const int r = r0 + threadIdx.x;
    const bool masked = r < M && !a.committed[r];
    base = block_compact(masked, base, a.st.rowlist, a.st.rowpos, r < M ? r : -1, s_wave);
    act = block_compact(r < M && !a.st.seq_done[r / a.B], act, a.st.act_rows, nullptr, r < M ? r : -1, s_wave);
  }
  if (threadIdx.x == 0) {
    *a.st.n_rows = base;
    *a.st.n_act = act;
    *a.st.done = base == 0 ? 1 : 0;
    *a.st.t = t + 1;
    if (a.host_progress)   // one word, system scope: the host polls it while issuing steps
      __hip_atomic_store(a.host_progress, (a.gen << 8) | ((unsigned)(t + 1) << 1) | (base == 0 ? 1u : 0u),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

TD_DEV VStat shfl_xor(const VStat &v, int o) {
  return VStat{__shfl_xor(v.m, o), __shfl_xor(v.s, o), __shfl_xor(v.a, o)};
}

// One wave merges row `row`: lane l combines groups l, l + 64, ... in order (eight loads
// in flight), then the wave combines its lanes in a fixed tree.
TD_DEV void merge_row(const CommitArgs &a, int row, int lane) {
  constexpr int PER = 8;
  const VStat *vp = a.vpart + (size_t)row * a.nslices;
  VStat v{-INFINITY, 0.f, 0x7FFFFFFF};
  for (int i0 = lane; i0 < a.nslices; i0 += 64 * PER) {
    VStat u[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) u[j] = vp[min(i0 + 64 * j, a.nslices - 1)];
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (i0 + 64 * j < a.nslices) v = vstat_merge(v, u[j]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = vstat_merge(v, shfl_xor(v, o));
  if (lane == 0) {
    a.conf_row[row] = 1.0f / v.s;
    a.arg_row[row] = v.a;
  }
}

// Single workgroup (1024 threads): wave w merges rows w, w + 16, ..., then commits.
__global__ __launch_bounds__(1024) void merge_commit_small_kernel(CommitArgs a) {
  __shared__ int s_wave[16];
  const int n_rows = *a.st.n_rows;   // loaded together with the loop-exit flag
  if (*a.st.done) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int row = wave; row < n_rows; row += 16) merge_row(a, row, lane);
  __syncthreads();
  commit_all(a, s_wave);
}

// Many rows: workgroup b merges rows 4b .. 4b + 3, a wave each.
__global__ __launch_bounds__(256) void merge_rows_kernel(CommitArgs a) {
  const int n_rows = *a.st.n_rows;   // loaded together with the loop-exit flag
  if (*a.st.done) return;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row < n_rows) merge_row(a, row, threadIdx.x & 63);
}

__global__ __launch_bounds__(1024) void commit_kernel(CommitArgs a) {
  __shared__ int s_wave[16];
  if (*a.st.done) return;
  commit_all(a, s_wave);
}

}  // namespace

hipError_t launch_merge_commit(const CommitArgs &a, int max_rows, hipStream_t s) {
  if (max_rows <= COMMIT_SMALL_ROWS)
    hipLaunchKernelGGL(merge_commit_small_kernel, dim3(1), dim3(1024), 0, s, a);
  else {
    hipLaunchKernelGGL(merge_rows_kernel, dim3((max_rows + 3) / 4), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(1024), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace td
