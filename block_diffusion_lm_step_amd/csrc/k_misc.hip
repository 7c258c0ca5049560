// Weight packing, loop-state kernels and the token + block-position embedding.
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

// W [N][K] -> MFMA tile order; one thread per 8-element lane fragment.
template <typename T>
__global__ void pack_weight_kernel(const T *__restrict__ W, T *__restrict__ Wp, int N, int K) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KT = K / 32;
  const int64_t total = (int64_t)N * K / 8;
  if (idx >= total) return;
  const int64_t tile = idx >> 6;
  const int lane = (int)(idx & 63);
  const int nt = (int)(tile / KT), kt = (int)(tile % KT);
  const T *src = W + (int64_t)(nt * 16 + (lane & 15)) * K + kt * 32 + (lane >> 4) * 8;
  T *dst = Wp + idx * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = src[e];
}

__global__ __launch_bounds__(1024) void prep_kernel(const int *tokens, const uint8_t *committed, int M, int B,
                                                    int V, StepState st) {
  __shared__ int s_wave[16];
  int base = 0, act = 0, err = 0;
  for (int r0 = 0; r0 < M; r0 += 1024) {
    const int r = r0 + threadIdx.x;
    bool masked = false;
    if (r < M) {
      const int tok = tokens[r];
      masked = committed[r] == 0;
      const bool bad = tok < 0 || tok > V || masked != (tok == V);
      if (bad) {
        err = 1;
        masked = false;    // an invalid row is left untouched
      }
    }
    // A sequence is finished when none of its B rows (B consecutive lanes) is masked.
    int any = masked ? 1 : 0;
    for (int o = 1; o < B; o <<= 1) any |= __shfl_xor(any, o);
    if (r < M && r % B == 0) st.seq_done[r / B] = any ? 0 : 1;
    base = block_compact(masked, base, st.rowlist, st.rowpos, r < M ? r : -1, s_wave);
    // rows of the sequences still active (the layer GEMMs compute only these)
    act = block_compact(r < M && any, act, st.act_rows, nullptr, r < M ? r : -1, s_wave);
  }
  if (err) atomicOr(st.err, 1);
  if (threadIdx.x == 0) {
    *st.n_rows = base;
    *st.n_act = act;
    *st.done = base == 0 ? 1 : 0;
  }
}

__global__ __launch_bounds__(1024) void init_block_kernel(int *tokens, uint8_t *committed, int8_t *commit_step,
                                                          int *steps, int n, int B, int V, StepState st) {
  const int M = n * B;
  for (int r = threadIdx.x; r < M; r += blockDim.x) {
    tokens[r] = V;
    committed[r] = 0;
    if (commit_step) commit_step[r] = -1;
    st.rowlist[r] = r;
    st.rowpos[r] = r;
    st.act_rows[r] = r;
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    if (steps) steps[i] = 0;
    st.seq_done[i] = 0;
  }
  if (threadIdx.x == 0) {
    *st.n_rows = M;
    *st.n_act = M;
    *st.done = M == 0 ? 1 : 0;
    *st.t = 0;
  }
}

// x[r] = E[tok[r]] + Pos[r % B] (fp32) and the partial sums of squares of every 16-column
// group, [d/16][M], which the next GEMM prologue turns into the RMSNorm row scale.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int *tokens, const T *E, const T *Pos, const T *gain,
                                                    float *x, float *ssq, void *x_afl, int M, int B, int d, int V,
                                                    StepState st) {
  const int r = blockIdx.x;
  int tok = tokens[r];   // loaded together with the loop-exit flag
  if (*st.done) return;
  if (tok < 0 || tok > V) {
    if (threadIdx.x == 0) atomicOr(st.err, 2);
    tok = V;
  }
  const T *e = E + (size_t)tok * d;
  const T *p = Pos ? Pos + (size_t)(r % B) * d : nullptr;   // no table: the context tower
  for (int grp = threadIdx.x; grp < d / 16; grp += blockDim.x) {
    // 16 consecutive columns per thread, moved as 16-byte vectors.
    Frag<T> fe[2], fp[2], fg[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      fe[h].load(e + grp * 16 + 8 * h);
      if (p) fp[h].load(p + grp * 16 + 8 * h);
      else fp[h].zero();
      fg[h].load(gain + grp * 16 + 8 * h);
    }
    float s = 0.f, v[16], vg[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      v[c] = fe[c >> 3].get(c & 7) + fp[c >> 3].get(c & 7);
      vg[c] = v[c] * fg[c >> 3].get(c & 7);
      s += v[c] * v[c];
    }
    float4 *xr = reinterpret_cast<float4 *>(x + (size_t)r * d + grp * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) xr[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    ssq[(size_t)grp * M + r] = s;
    afl_put8<T>(x_afl, d / 32, r, grp * 16, vg);
    afl_put8<T>(x_afl, d / 32, r, grp * 16 + 8, vg + 8);
  }
}

// One thread per (block row, K/V head, element): the k and v of the row go to slot
// t % 32 of page seq_page[seq] + t / 32, t = seq_len[seq] + p.
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(const float *qkv, int Nqkv, int H, int Hkv, int hd, T *kc,
                                                        T *vc, const int *seq_len, const int *seq_page, int B) {
  const int r = blockIdx.x, seq = r / B, p = r % B;
  const int idx = blockIdx.y * blockDim.x + threadIdx.x;
  if (idx >= Hkv * hd) return;
  const int h = idx / hd, e = idx % hd;
  const int t = seq_len[seq] + p;
  const size_t page = (size_t)seq_page[seq] + t / KV_PAGE;
  const int slot = t % KV_PAGE;
  const float kv = qkv[(size_t)r * Nqkv + (size_t)(H + h) * hd + e];
  const float vv = qkv[(size_t)r * Nqkv + (size_t)(H + Hkv + h) * hd + e];
  const int half = (slot / 4) % 2, row = (slot / 8) * 4 + slot % 4;
  kc[(page * Hkv + h) * KV_PAGE * hd + ((e / 32) * 2 + half) * 512 + row * 32 + e % 32] = from_f32<T>(kv);
  vc[((page * Hkv + h) * hd + e) * KV_PAGE + slot] = from_f32<T>(vv);
}

__global__ __launch_bounds__(256) void advance_kernel(AttnItem *items, const int *grow_idx, int n_pairs, int *seq_len,
                                                     int n_seqs, int add) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_pairs) {
    const int k = grow_idx[i];
    if (k >= 0) items[k].k_end += add;
  }
  if (i < n_seqs) seq_len[i] += add;
}

}  // namespace

hipError_t launch_advance(AttnItem *items, const int *grow_idx, int n_pairs, int *seq_len, int n_seqs, int add,
                          hipStream_t s) {
  const int n = n_pairs > n_seqs ? n_pairs : n_seqs;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(advance_kernel, dim3((n + 255) / 256), dim3(256), 0, s, items, grow_idx, n_pairs, seq_len, n_seqs,
                     add);
  return hipGetLastError();
}

hipError_t launch_kv_append(int dtype, const float *qkv, int Nqkv, int H, int Hkv, int hd, void *kc, void *vc,
                            const int *seq_len, const int *seq_page, int n, int B, hipStream_t s) {
  if (n <= 0 || B <= 0 || hd % 32 || !kc || !vc) return hipErrorInvalidValue;
  const dim3 grid(n * B, (Hkv * hd + 255) / 256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(kv_append_kernel<bf16_t>, grid, dim3(256), 0, s, qkv, Nqkv, H, Hkv, hd, (bf16_t *)kc,
                       (bf16_t *)vc, seq_len, seq_page, B);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, s, qkv, Nqkv, H, Hkv, hd, (float *)kc,
                       (float *)vc, seq_len, seq_page, B);
  return hipGetLastError();
}

hipError_t launch_pack_weight(int dtype, const void *W, void *Wp, int N, int K, hipStream_t s) {
  if (N % 16 || K % 32) return hipErrorInvalidValue;
  const int64_t total = (int64_t)N * K / 8;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(pack_weight_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t *)W, (bf16_t *)Wp, N, K);
  else
    hipLaunchKernelGGL(pack_weight_kernel<float>, grid, dim3(256), 0, s, (const float *)W, (float *)Wp, N, K);
  return hipGetLastError();
}

hipError_t launch_prep(const int *tokens, const uint8_t *committed, int M, int B, int V, StepState st, hipStream_t s) {
  if (B < 1 || 64 % B) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(1024), 0, s, tokens, committed, M, B, V, st);
  return hipGetLastError();
}

hipError_t launch_init_block(int *tokens, uint8_t *committed, int8_t *commit_step, int *steps, int n, int B,
                             int V, StepState st, hipStream_t s) {
  hipLaunchKernelGGL(init_block_kernel, dim3(1), dim3(1024), 0, s, tokens, committed, commit_step, steps, n, B, V,
                     st);
  return hipGetLastError();
}

hipError_t launch_embed(int dtype, const int *tokens, const void *E, const void *Pos, const void *gain, float *x,
                        float *ssq, void *x_afl, int M, int B, int d, int V, StepState st, hipStream_t s) {
  if (d % 32) return hipErrorInvalidValue;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(M), dim3(256), 0, s, tokens, (const bf16_t *)E,
                       (const bf16_t *)Pos, (const bf16_t *)gain, x, ssq, x_afl, M, B, d, V, st);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, s, tokens, (const float *)E, (const float *)Pos,
                       (const float *)gain, x, ssq, x_afl, M, B, d, V, st);
  return hipGetLastError();
}

}  // namespace td
