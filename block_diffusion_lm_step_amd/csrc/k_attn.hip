// Split-K block attention over the frozen context tower's prefix K/V plus the block's
// own keys, then a fixed-order log-sum-exp merge.
//
// Each query row of the block (one query head, one block position) takes ONE softmax
// over the concatenation [prefix keys ; block keys] with no mask: the denoiser attends
// bidirectionally inside the block and cross-attends to the cached context
// (poko-everyday.com Nemotron-TwoTower news item, section 技術/ビジネス面 describes the
// two towers; block-wise decoding keeps the prefix K/V read-only while the block is
// refined).  Query head j reads K/V head j / (H / Hkv).
//
// Work decomposition (flash-decoding style): an item is (sequence, K/V head, chunk of
// prefix keys) or (sequence, K/V head, the B block keys).  A workgroup streams its
// item's keys in 32-key sub-tiles from HBM (coalesced 16-byte loads, next sub-tile in
// flight while the current one is consumed) through LDS, where K is stored row-major
// and V transposed, and keeps the online-softmax state (running max m, running sum l,
// unnormalised output O) of every query row the item serves.  All G*B query rows of a
// K/V head share each K/V tile: a 16-row MFMA tile per wave, several tiles and waves
// per workgroup for grouped-query heads.
//   S^T[key][row] = K . Q^T      (MFMA, A = K from LDS, B = Q held in registers)
//   O^T[hd][row] += V^T . P^T    (MFMA, A = V^T from LDS, B = P straight from S^T's
//                                 accumulator layout; the keys are stored in LDS in
//                                 the permuted order that makes this possible)
// Queries are fp32 activations; with bf16 keys each query fragment enters the MFMA as a
// bf16 high part plus a bf16 remainder, and the probabilities are split the same way
// for P.V, so q and P keep ~16 significant bits.  The block's own keys and values are
// fp32 activations as well: the (few) block keys of each pair are handled by a
// separate fp32 VALU kernel that writes the same (m, l, O) partial.
// The merge kernel combines a pair's partial (m, l, O) rows in item order.
#include "td_device.h"
#include "td_kernels.h"

namespace td {

namespace {

constexpr int SUB = 32;   // keys per sub-tile

template <typename T> struct Pad;
template <> struct Pad<bf16_t> { static constexpr int K = 8, V = 8; };
template <> struct Pad<float> { static constexpr int K = 4, V = 4; };

// LDS position of key `key` (0..31) of a sub-tile inside a row of V^T: keys
// 16h + 4g + r go to slot 8g + 4h + r, so lane group g's eight P values (S^T rows
// 4g..4g+3 of both 16-key halves) are eight consecutive slots.
TD_DEV int sigma(int key) { return ((key >> 2) & 3) * 8 + (key >> 4) * 4 + (key & 3); }

template <typename T, int HD, int RT, int NW>
__global__ __launch_bounds__(64 * NW) void attn_split_kernel(AttnArgs a) {
  if (a.done && *a.done) return;
  constexpr int NT = 64 * NW;
  constexpr int KP = HD + Pad<T>::K;       // K row stride in LDS (elements)
  constexpr int VP = SUB + Pad<T>::V;      // V^T row stride in LDS (elements)
  constexpr int CPR = HD / 8;              // 8-element chunks per key row
  constexpr int CHUNKS = SUB * CPR;        // per operand per sub-tile
  constexpr int PER_T = (CHUNKS + NT - 1) / NT;
  constexpr int HC = HD / 32;              // 32-wide contraction steps over hd
  constexpr int OT = HD / 16;              // 16-row output tiles over hd

  __shared__ __attribute__((aligned(16))) T s_k[2][SUB * KP];
  __shared__ __attribute__((aligned(16))) T s_vt[2][HD * VP];

  const AttnItem it = a.items[blockIdx.x];
  if (it.is_block) return;   // block keys: attn_block_kernel
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int nsub = (nkeys + SUB - 1) / SUB;

  // Key/value row pointers of this item.
  const size_t off = (size_t)(a.offsets[it.seq] + it.k_begin) * a.Hkv + it.kvh;
  const T *kbase = reinterpret_cast<const T *>(a.kc) + off * HD;
  const T *vbase = reinterpret_cast<const T *>(a.vc) + off * HD;
  const size_t kstride = (size_t)a.Hkv * HD;

  // Query fragments (B operand of S^T = K Q^T) of this wave's row tiles.
  AFrag<T> qf[RT][HC];
  const int rt0 = (blockIdx.y * NW + wave) * RT;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = (rt0 + rt) * 16 + l16;
#pragma unroll
    for (int c = 0; c < HC; ++c) {
      if (rho < a.R) {
        const int j = rho / a.B, p = rho % a.B;
        float v[8];
        load8f(a.qkv + (size_t)(it.seq * a.B + p) * a.Nqkv + (size_t)(it.kvh * a.G + j) * HD + c * 32 + g * 8, v);
        qf[rt][c].set8(v);
      } else {
        qf[rt][c].zero();
      }
    }
  }

  float m_run[RT], l_run[RT];
  f32x4_t o[RT][OT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[rt][t] = zero4();
  }

  // Register staging of one sub-tile (this thread's chunks of K and V).
  Frag<T> kreg[PER_T], vreg[PER_T];
  auto fetch = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = threadIdx.x + i * NT;
      const int key = c / CPR, part = c % CPR;
      const int kk = s * SUB + key;
      if (c < CHUNKS && kk < nkeys) {
        kreg[i].load(kbase + (size_t)kk * kstride + part * 8);
        vreg[i].load(vbase + (size_t)kk * kstride + part * 8);
      } else {
        kreg[i].zero();
        vreg[i].zero();
      }
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < CHUNKS) {
        const int key = c / CPR, part = c % CPR;
        *reinterpret_cast<Frag<T> *>(&s_k[buf][key * KP + part * 8]) = kreg[i];
        const int col = sigma(key);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          T v;
          if constexpr (sizeof(T) == 2) {
            const uint32_t w = (&vreg[i].raw.x)[e >> 1];
            v = (T)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
          } else {
            v = vreg[i].get(e);
          }
          s_vt[buf][(part * 8 + e) * VP + col] = v;
        }
      }
    }
  };

  if (nsub > 0) fetch(0);
  for (int s = 0; s < nsub; ++s) {
    const int buf = s & 1;
    stash(buf);
    __syncthreads();
    if (s + 1 < nsub) fetch(s + 1);

    const T *ks = s_k[buf];
    const T *vt = s_vt[buf];
    const int kvalid = nkeys - s * SUB;   // valid keys in this sub-tile (>= 1)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4_t st[2] = {zero4(), zero4()};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < HC; ++c) {
          const Frag<T> kf = *reinterpret_cast<const Frag<T> *>(&ks[(16 * h + l16) * KP + c * 32 + g * 8]);
          st[h] = mma_b(kf, qf[rt][c], st[h]);
        }
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * h + 4 * g + r;
          const float v = key < kvalid ? st[h][r] * a.scale : -INFINITY;
          sc[4 * h + r] = v;
          mx = fmaxf(mx, v);
        }
      mx = max_groups(mx);
      const float m_new = fmaxf(m_run[rt], mx);
      const float alpha = (m_run[rt] == -INFINITY) ? 0.f : __expf(m_run[rt] - m_new);
      float pv[8], psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pv[j] = (sc[j] == -INFINITY) ? 0.f : __expf(sc[j] - m_new);
        psum += pv[j];
      }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int t = 0; t < OT; ++t) o[rt][t] *= alpha;
      if constexpr (sizeof(T) == 2) {
        Frag<T> phi, plo;
        phi.set8(pv);
        float rem[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) rem[j] = pv[j] - phi.get(j);
        plo.set8(rem);
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          const Frag<T> vf = *reinterpret_cast<const Frag<T> *>(&vt[(16 * t + l16) * VP + g * 8]);
          o[rt][t] = mma(vf, phi, o[rt][t]);
          o[rt][t] = mma(vf, plo, o[rt][t]);
        }
      } else {
        Frag<T> pf;
        pf.set8(pv);
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          const Frag<T> vf = *reinterpret_cast<const Frag<T> *>(&vt[(16 * t + l16) * VP + g * 8]);
          o[rt][t] = mma(vf, pf, o[rt][t]);
        }
      }
    }
    // The next iteration writes the other buffer; the one after reuses this buffer only
    // after the next barrier, which every wave reaches after finishing this compute.
  }

  // Partials: (m, l) per row and the unnormalised O row.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = (rt0 + rt) * 16 + l16;
    const float l_tot = sum_groups(l_run[rt]);
    if (rho < a.R) {
      const size_t prow = (size_t)blockIdx.x * a.R + rho;
      if (g == 0) {
        a.part_ml[prow * 2 + 0] = m_run[rt];
        a.part_ml[prow * 2 + 1] = l_tot;
      }
#pragma unroll
      for (int t = 0; t < OT; ++t)
        *reinterpret_cast<f32x4_t *>(&a.part_o[prow * HD + 16 * t + 4 * g]) = o[rt][t];
    }
  }
}

// The block's own B keys of one (seq, kv head) pair, in fp32: one workgroup per pair,
// 16 threads per query row (each owning HD/16 head dimensions), partial (m, l, O) into
// the slot of the pair's block item.
template <int HD>
__global__ __launch_bounds__(256) void attn_block_kernel(AttnArgs a) {
  if (a.done && *a.done) return;
  constexpr int EPT = HD / 16;
  constexpr int BMAX = 32;
  __shared__ float s_k[BMAX][HD + 1], s_v[BMAX][HD + 1];
  const int pair = blockIdx.x;
  const int item = a.pair_first[pair] + a.pair_count[pair] - 1;
  const AttnItem it = a.items[item];
  const float *base = a.qkv + (size_t)it.seq * a.B * a.Nqkv;
  for (int i = threadIdx.x; i < a.B * HD; i += blockDim.x) {
    const int key = i / HD, e = i % HD;
    s_k[key][e] = base[(size_t)key * a.Nqkv + (size_t)(a.H + it.kvh) * HD + e];
    s_v[key][e] = base[(size_t)key * a.Nqkv + (size_t)(a.H + a.Hkv + it.kvh) * HD + e];
  }
  __syncthreads();
  const int sub = threadIdx.x & 15, e0 = sub * EPT;
  for (int rho = threadIdx.x >> 4; rho < a.R; rho += blockDim.x >> 4) {
    const int j = rho / a.B, p = rho % a.B;
    const float *q = base + (size_t)p * a.Nqkv + (size_t)(it.kvh * a.G + j) * HD + e0;
    float qv[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) qv[e] = q[e];
    float sc[BMAX];
    float m = -INFINITY;
#pragma unroll
    for (int key = 0; key < BMAX; ++key) {
      if (key < a.B) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) d += qv[e] * s_k[key][e0 + e];
        d = sum16(d) * a.scale;
        sc[key] = d;
        m = fmaxf(m, d);
      }
    }
    float l = 0.f, o[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) o[e] = 0.f;
#pragma unroll
    for (int key = 0; key < BMAX; ++key) {
      if (key < a.B) {
        const float pk = __expf(sc[key] - m);
        l += pk;
#pragma unroll
        for (int e = 0; e < EPT; ++e) o[e] += pk * s_v[key][e0 + e];
      }
    }
    const size_t prow = (size_t)item * a.R + rho;
    if (sub == 0) {
      a.part_ml[prow * 2 + 0] = m;
      a.part_ml[prow * 2 + 1] = l;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) a.part_o[prow * HD + e0 + e] = o[e];
  }
}

// One workgroup per (pair, 16 query rows): 16 threads per row, HD/16 outputs each.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  if (a.done && *a.done) return;
  constexpr int EPT = HD / 16;
  const int pair = blockIdx.x;
  const int rho = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int e0 = (threadIdx.x & 15) * EPT;
  if (rho >= a.R) return;
  const int first = a.pair_first[pair], cnt = a.pair_count[pair];
  float M = -INFINITY;
  for (int i = 0; i < cnt; ++i) M = fmaxf(M, a.part_ml[((size_t)(first + i) * a.R + rho) * 2]);
  float L = 0.f, acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  for (int i = 0; i < cnt; ++i) {
    const size_t prow = (size_t)(first + i) * a.R + rho;
    const float w = __expf(a.part_ml[prow * 2] - M);
    L += a.part_ml[prow * 2 + 1] * w;
    const float *po = a.part_o + prow * HD + e0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] += po[e] * w;
  }
  const float inv = 1.0f / L;
  const AttnItem it = a.items[first];
  const int j = rho / a.B, p = rho % a.B;
  float *out = a.o + (size_t)(it.seq * a.B + p) * a.ldo + (size_t)(it.kvh * a.G + j) * HD + e0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) out[e] = acc[e] * inv;
}

template <typename T, int HD, int RT, int NW>
hipError_t launch_split(const AttnArgs &a, hipStream_t s) {
  const int rows_per_wg = 16 * RT * NW;
  dim3 grid(a.n_items, (a.R + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((attn_split_kernel<T, HD, RT, NW>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t launch_hd(const AttnArgs &a, hipStream_t s) {
  hipError_t e;
  if (a.R <= 16) e = launch_split<T, HD, 1, 1>(a, s);
  else if (a.R <= 32) e = launch_split<T, HD, 2, 1>(a, s);
  else if (a.R <= 64) e = launch_split<T, HD, 1, 4>(a, s);
  else e = launch_split<T, HD, 4, 4>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_block_kernel<HD>), dim3(a.n_pairs), dim3(256), 0, s, a);
  dim3 grid(a.n_pairs, (a.R + 15) / 16);
  hipLaunchKernelGGL((attn_merge_kernel<T, HD>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnArgs &a, hipStream_t s) {
  if (a.n_items <= 0 || a.n_pairs <= 0) return hipErrorInvalidValue;
  if (dtype == DT_BF16) {
    if (a.hd == 128) return launch_hd<bf16_t, 128>(a, s);
    if (a.hd == 64) return launch_hd<bf16_t, 64>(a, s);
  } else {
    if (a.hd == 128) return launch_hd<float, 128>(a, s);
    if (a.hd == 64) return launch_hd<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace td
