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
// Prefix keys (attn_split_kernel, flash-decoding style).  An item is (sequence, K/V
// head, chunk of prefix keys).  Keys are streamed in 32-key sub-tiles with coalesced
// 16-byte loads (the next sub-tile in flight while the current one is consumed) through
// LDS, where K is stored row-major and V transposed, and every query row the item
// serves keeps an online-softmax state (running max m, running sum l, unnormalised O):
//   S^T[key][row] = K . Q^T      (MFMA, A = K from LDS, B = Q held in registers)
//   O^T[hd][row] += V^T . P^T    (MFMA, A = V^T from LDS, B = P straight from S^T's
//                                 accumulator layout; keys are stored in LDS in the
//                                 permuted order that makes this possible)
// Two shapes of work:
//   * few query rows per K/V head (R = G*B <= 32, multi-head attention): the four
//     waves of a workgroup take alternate sub-tiles of the chunk, each through its own
//     LDS slice, and merge their states in LDS at the end (4x the bytes in flight);
//   * many rows (grouped-query heads): the four waves share each sub-tile in LDS and
//     each owns RT 16-row tiles.
// Queries are fp32 activations; against bf16 keys each query fragment enters the MFMA
// as a bf16 high part plus a bf16 remainder, and the probabilities are split the same
// way for P.V, so q and P keep ~16 significant bits.
//
// The block's own keys (attn_finish_kernel) are fp32 activations and few (B per pair):
// they are attended in fp32 on the VALU by the kernel that then merges the prefix
// partials of the pair, in item order, and writes o.
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

// WSPLIT: waves split the sub-tiles (RT row tiles each, all rows of the item);
// otherwise waves split the row tiles and share every sub-tile.
template <typename T, int HD, int RT, bool WSPLIT>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  if (a.done && *a.done) return;
  constexpr int NW = 4;
  constexpr int KP = HD + Pad<T>::K;       // K row stride in LDS (elements)
  constexpr int VP = SUB + Pad<T>::V;      // V^T row stride in LDS (elements)
  constexpr int CPR = HD / 8;              // 8-element chunks per key row
  constexpr int CHUNKS = SUB * CPR;        // per operand per sub-tile
  constexpr int LOADERS = WSPLIT ? 64 : 64 * NW;   // threads that load one sub-tile
  constexpr int PER_T = (CHUNKS + LOADERS - 1) / LOADERS;
  constexpr int HC = HD / 32;              // 32-wide contraction steps over hd
  constexpr int OT = HD / 16;              // 16-row output tiles over hd
  constexpr int NSLICE = WSPLIT ? NW : 1;  // LDS staging slices
  constexpr int SLICE = SUB * KP + HD * VP;
  static_assert(!WSPLIT || (size_t)NSLICE * SLICE * sizeof(T) >= NW * RT * 16 * (HD + 2) * sizeof(float),
                "the wave merge reuses the staging LDS");

  __shared__ __attribute__((aligned(16))) T s_stage[NSLICE][SLICE];

  const AttnItem it = a.items[blockIdx.x];
  if (it.is_block) return;   // block keys: attn_finish_kernel
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int nsub = (nkeys + SUB - 1) / SUB;
  const int ltid = WSPLIT ? lane : threadIdx.x;     // index among this sub-tile's loaders
  T *s_k = s_stage[WSPLIT ? wave : 0];
  T *s_vt = s_k + SUB * KP;

  const size_t off = (size_t)(a.offsets[it.seq] + it.k_begin) * a.Hkv + it.kvh;
  const T *kbase = reinterpret_cast<const T *>(a.kc) + off * HD;
  const T *vbase = reinterpret_cast<const T *>(a.vc) + off * HD;
  const size_t kstride = (size_t)a.Hkv * HD;

  // Query fragments (B operand of S^T = K Q^T) of this wave's row tiles.
  AFrag<T> qf[RT][HC];
  const int rt0 = WSPLIT ? 0 : (blockIdx.y * NW + wave) * RT;
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
      const int c = ltid + i * LOADERS;
      const int key = c / CPR, part = c % CPR;
      const int kk = s * SUB + key;
      if (c < CHUNKS && s < nsub && kk < nkeys) {
        kreg[i].load(kbase + (size_t)kk * kstride + part * 8);
        vreg[i].load(vbase + (size_t)kk * kstride + part * 8);
      } else {
        kreg[i].zero();
        vreg[i].zero();
      }
    }
  };
  auto stash = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = ltid + i * LOADERS;
      if (c < CHUNKS) {
        const int key = c / CPR, part = c % CPR;
        *reinterpret_cast<Frag<T> *>(&s_k[key * KP + part * 8]) = kreg[i];
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
          s_vt[(part * 8 + e) * VP + col] = v;
        }
      }
    }
  };

  // Iteration i2 handles sub-tile i2 (shared) or i2 * NW + wave (split).  Every wave
  // runs the same number of iterations, so the barriers are uniform.
  const int iters = WSPLIT ? (nsub + NW - 1) / NW : nsub;
  auto sub_of = [&](int i2) { return WSPLIT ? i2 * NW + wave : i2; };
  fetch(sub_of(0));
  for (int i2 = 0; i2 < iters; ++i2) {
    const int s = sub_of(i2);
    __syncthreads();   // every wave is done reading the previous sub-tile
    stash();
    __syncthreads();   // this sub-tile is in LDS
    if (i2 + 1 < iters) fetch(sub_of(i2 + 1));
    if (s >= nsub) continue;
    const int kvalid = nkeys - s * SUB;   // valid keys in this sub-tile (>= 1)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4_t st[2] = {zero4(), zero4()};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < HC; ++c) {
          const Frag<T> kf = *reinterpret_cast<const Frag<T> *>(&s_k[(16 * h + l16) * KP + c * 32 + g * 8]);
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
      AFrag<T> pf;
      pf.set8(pv);
#pragma unroll
      for (int t = 0; t < OT; ++t) {
        const Frag<T> vf = *reinterpret_cast<const Frag<T> *>(&s_vt[(16 * t + l16) * VP + g * 8]);
        o[rt][t] = mma_b(vf, pf, o[rt][t]);
      }
    }
  }

  float l_tot[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) l_tot[rt] = sum_groups(l_run[rt]);

  if constexpr (WSPLIT) {
    // Merge the four waves' states (wave order) through the staging LDS.
    __syncthreads();
    float *s_o = reinterpret_cast<float *>(&s_stage[0][0]);   // [NW][RT*16][HD]
    float *s_ml = s_o + NW * RT * 16 * HD;                     // [NW][RT*16][2]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int rr = rt * 16 + l16;
      if (g == 0) {
        s_ml[(wave * RT * 16 + rr) * 2 + 0] = m_run[rt];
        s_ml[(wave * RT * 16 + rr) * 2 + 1] = l_tot[rt];
      }
#pragma unroll
      for (int t = 0; t < OT; ++t)
        *reinterpret_cast<f32x4_t *>(&s_o[(wave * RT * 16 + rr) * HD + 16 * t + 4 * g]) = o[rt][t];
    }
    __syncthreads();
    // Row rr = tid / 16 (+16 per pass), 16 threads per row, HD/16 columns each.
    constexpr int EPT = HD / 16;
    const int e0 = (threadIdx.x & 15) * EPT;
    for (int rr = threadIdx.x >> 4; rr < RT * 16 && rr < a.R; rr += 16) {
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) Mx = fmaxf(Mx, s_ml[(w * RT * 16 + rr) * 2]);
      float L = 0.f, acc[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_ml[(w * RT * 16 + rr) * 2];
        const float f = (mw == -INFINITY) ? 0.f : __expf(mw - Mx);
        L += s_ml[(w * RT * 16 + rr) * 2 + 1] * f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] += s_o[(w * RT * 16 + rr) * HD + e0 + e] * f;
      }
      const size_t prow = (size_t)blockIdx.x * a.R + rr;
      if ((threadIdx.x & 15) == 0) {
        a.part_ml[prow * 2 + 0] = Mx;
        a.part_ml[prow * 2 + 1] = L;
      }
#pragma unroll
      for (int e = 0; e < EPT; ++e) a.part_o[prow * HD + e0 + e] = acc[e];
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int rho = (rt0 + rt) * 16 + l16;
      if (rho < a.R) {
        const size_t prow = (size_t)blockIdx.x * a.R + rho;
        if (g == 0) {
          a.part_ml[prow * 2 + 0] = m_run[rt];
          a.part_ml[prow * 2 + 1] = l_tot[rt];
        }
#pragma unroll
        for (int t = 0; t < OT; ++t)
          *reinterpret_cast<f32x4_t *>(&a.part_o[prow * HD + 16 * t + 4 * g]) = o[rt][t];
      }
    }
  }
}

// One workgroup per (pair, 16 query rows): the B block keys in fp32 (16 threads per row,
// HD/16 head dimensions each), then the merge with the pair's prefix partials in item
// order, and o.  The partial maxima and sums of the pair are first read in parallel
// into LDS; the partial outputs are then read in independent batches.
constexpr int FIN_ITEMS = 256;   // prefix items per pair the finish kernel merges

template <int HD>
__global__ __launch_bounds__(256) void attn_finish_kernel(AttnArgs a) {
  if (a.done && *a.done) return;
  constexpr int EPT = HD / 16;
  constexpr int BMAX = 32;
  constexpr int BATCH = 8;
  __shared__ float s_k[BMAX][HD + 1], s_v[BMAX][HD + 1];
  __shared__ float s_m[FIN_ITEMS][16], s_l[FIN_ITEMS][16];
  const int pair = blockIdx.x;
  const int first = a.pair_first[pair], cnt = a.pair_count[pair];
  const int npre = cnt - 1;                       // prefix items (the block item is last)
  const AttnItem it = a.items[first + npre];
  const int rho0 = blockIdx.y * 16;
  const float *base = a.qkv + (size_t)it.seq * a.B * a.Nqkv;
  for (int i = threadIdx.x; i < a.B * HD; i += blockDim.x) {
    const int key = i / HD, e = i % HD;
    s_k[key][e] = base[(size_t)key * a.Nqkv + (size_t)(a.H + it.kvh) * HD + e];
    s_v[key][e] = base[(size_t)key * a.Nqkv + (size_t)(a.H + a.Hkv + it.kvh) * HD + e];
  }
  for (int i = threadIdx.x; i < npre * 16; i += blockDim.x) {
    const int item = i >> 4, r = i & 15;
    float m = -INFINITY, l = 0.f;
    if (rho0 + r < a.R) {
      const size_t prow = (size_t)(first + item) * a.R + rho0 + r;
      m = a.part_ml[prow * 2];
      l = a.part_ml[prow * 2 + 1];
    }
    s_m[item][r] = m;
    s_l[item][r] = l;
  }
  __syncthreads();
  const int sub = threadIdx.x & 15, e0 = sub * EPT;
  const int r = threadIdx.x >> 4, rho = rho0 + r;
  if (rho >= a.R) return;
  const int j = rho / a.B, p = rho % a.B;
  const float *q = base + (size_t)p * a.Nqkv + (size_t)(it.kvh * a.G + j) * HD + e0;
  float qv[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) qv[e] = q[e];

  // Block keys, fp32.
  float sc[BMAX];
  float mb = -INFINITY;
#pragma unroll
  for (int key = 0; key < BMAX; ++key) {
    if (key < a.B) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) d += qv[e] * s_k[key][e0 + e];
      d = sum16(d) * a.scale;
      sc[key] = d;
      mb = fmaxf(mb, d);
    }
  }
  float lb = 0.f, ob[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) ob[e] = 0.f;
#pragma unroll
  for (int key = 0; key < BMAX; ++key) {
    if (key < a.B) {
      const float pk = __expf(sc[key] - mb);
      lb += pk;
#pragma unroll
      for (int e = 0; e < EPT; ++e) ob[e] += pk * s_v[key][e0 + e];
    }
  }

  // Merge: prefix items in order, then the block keys.
  float M = mb;
  for (int i = 0; i < npre; ++i) M = fmaxf(M, s_m[i][r]);
  float L = 0.f, acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < npre; i0 += BATCH) {
    float po[BATCH][EPT];
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (i0 + b < npre) {
        const float *src = a.part_o + ((size_t)(first + i0 + b) * a.R + rho) * HD + e0;
#pragma unroll
        for (int e = 0; e < EPT; e += 4) *reinterpret_cast<float4 *>(&po[b][e]) = *reinterpret_cast<const float4 *>(src + e);
      }
#pragma unroll
    for (int b = 0; b < BATCH; ++b)
      if (i0 + b < npre) {
        const float mi = s_m[i0 + b][r];
        const float w = (mi == -INFINITY) ? 0.f : __expf(mi - M);
        L += s_l[i0 + b][r] * w;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] += po[b][e] * w;
      }
  }
  const float wb = __expf(mb - M);
  L += lb * wb;
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] += ob[e] * wb;
  const float inv = 1.0f / L;
  float *out = a.o + (size_t)(it.seq * a.B + p) * a.ldo + (size_t)(it.kvh * a.G + j) * HD + e0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) out[e] = acc[e] * inv;
}

template <typename T, int HD, int RT, bool WSPLIT>
hipError_t launch_split(const AttnArgs &a, hipStream_t s) {
  const int rows_per_wg = WSPLIT ? 16 * RT : 16 * RT * 4;
  dim3 grid(a.n_items, (a.R + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((attn_split_kernel<T, HD, RT, WSPLIT>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t launch_hd(const AttnArgs &a, hipStream_t s) {
  hipError_t e;
  if (a.R <= 16) e = launch_split<T, HD, 1, true>(a, s);
  else if (a.R <= 32) e = launch_split<T, HD, 2, true>(a, s);
  else if (a.R <= 64) e = launch_split<T, HD, 1, false>(a, s);
  else e = launch_split<T, HD, 4, false>(a, s);
  if (e != hipSuccess) return e;
  dim3 grid(a.n_pairs, (a.R + 15) / 16);
  hipLaunchKernelGGL((attn_finish_kernel<HD>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnArgs &a, hipStream_t s) {
  if (a.n_items <= 0 || a.n_pairs <= 0 || a.B > 32 || a.max_pair_items > FIN_ITEMS + 1) return hipErrorInvalidValue;
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
