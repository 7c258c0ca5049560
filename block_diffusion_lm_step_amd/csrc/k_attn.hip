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
// Prefix keys, flash-decoding style.  An item is (sequence, K/V head, run of prefix
// pages).  The cache is paged (32 tokens per page; per page and K/V head one contiguous
// 8 KiB block of K as [token][hd] and one of V transposed as [hd][token]), so every
// MFMA operand is a 16-byte load straight from HBM:
//   S^T[key][row] = K . Q^T      (A = K rows, B = Q fragments held in registers; the
//                                 two 16-key halves of a page take key rows in the
//                                 order that leaves lane group g holding the scores
//                                 of keys 8g .. 8g+7)
//   O^T[hd][row] += V^T . P^T    (A = V^T rows of the page, B = P straight from the
//                                 S^T accumulators)
// with an online softmax (running max m, running sum l, unnormalised O) per query row.
// Two shapes of work:
//   * few query rows per K/V head (R = G*B <= 32, multi-head attention): the four
//     waves of a workgroup take alternate pages of the item with no LDS and no barrier
//     in the key loop (the next page in flight while the current one is consumed), and
//     merge their states in LDS at the end;
//   * many rows (grouped-query heads): each page is copied once into LDS and the four
//     waves, each owning RT 16-row tiles, read it from there.
// Queries are fp32 activations; against bf16 keys each query fragment enters the MFMA
// as a bf16 high part plus a bf16 remainder, and the probabilities are split the same
// way for P.V, so q and P keep ~16 significant bits.  Key slots past the end of a
// sequence's last page are masked (scores to -inf, values to 0).
//
// The block's own keys (attn_finish_kernel) are fp32 activations and few (B per pair):
// they are attended in fp32 on the VALU by the kernel that then merges the prefix
// partials of the pair, in item order, and writes o.
#include "td_device.h"
#include "td_kernels.h"

#include <type_traits>

namespace td {

namespace {

constexpr int SUB = KV_PAGE;   // keys per page

// Key row of S^T tile h (0, 1) held by MFMA row i: keys 8g + 4h + r land in lane group g.
TD_DEV int krow(int h, int i) { return 8 * (i >> 2) + 4 * h + (i & 3); }

template <typename T> struct Pad;
template <> struct Pad<bf16_t> { static constexpr int K = 8, V = 8; };
template <> struct Pad<float> { static constexpr int K = 4, V = 4; };

// Zero the value slots of a V^T fragment (keys 8g .. 8g+7 of the page) at or past kvalid.
template <typename T>
TD_DEV void mask_v(Frag<T> &f, int g, int kvalid) {
  if (8 * g + 8 <= kvalid) return;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (8 * g + j < kvalid) ? f.get(j) : 0.f;
  f.set8(v);
}

// Online-softmax update of one 16-row tile with one page: S^T from the key fragments,
// probabilities, P.V into o.
template <typename T, int HD>
struct PageMath {
  static constexpr int HC = HD / 32, OT = HD / 16;
  template <typename KF, typename VF>
  TD_DEV static void run(const KF &kfrag, const VF &vfrag, const AFrag<T> (&qf)[HC], float scale, int kvalid,
                         int g, float &m_run, float &l_run, f32x4_t (&o)[OT]) {
    f32x4_t st[2] = {zero4(), zero4()};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < HC; ++c) st[h] = mma_b(kfrag(h, c), qf[c], st[h]);
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 8 * g + 4 * h + r;
        const float v = key < kvalid ? st[h][r] * scale : -INFINITY;
        sc[4 * h + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = max_groups(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : __expf(m_run - m_new);
    float pv[8], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = (sc[j] == -INFINITY) ? 0.f : __expf(sc[j] - m_new);
      psum += pv[j];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[t] *= alpha;
    AFrag<T> pf;
    pf.set8(pv);
#pragma unroll
    for (int t = 0; t < OT; ++t) o[t] = mma_b(vfrag(t), pf, o[t]);
  }
};

template <typename T, int HD, int RT>
TD_DEV void load_q(const AttnArgs &a, const AttnItem &it, int rt0, int g, int l16, AFrag<T> (&qf)[RT][HD / 32]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = (rt0 + rt) * 16 + l16;
#pragma unroll
    for (int c = 0; c < HD / 32; ++c) {
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
}

// Partial state of rows (rt0 + rt) * 16 + l16 -> the item's slot.
template <int HD, int RT>
TD_DEV void store_partial(const AttnArgs &a, int item, int rt0, int g, int l16, const float (&m_run)[RT],
                          const float (&l_tot)[RT], const f32x4_t (&o)[RT][HD / 16]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = (rt0 + rt) * 16 + l16;
    if (rho < a.R) {
      const size_t prow = (size_t)item * a.R + rho;
      if (g == 0) {
        a.part_ml[prow * 2 + 0] = m_run[rt];
        a.part_ml[prow * 2 + 1] = l_tot[rt];
      }
#pragma unroll
      for (int t = 0; t < HD / 16; ++t)
        *reinterpret_cast<f32x4_t *>(&a.part_o[prow * HD + 16 * t + 4 * g]) = o[rt][t];
    }
  }
}

// Multi-head shape (R <= 32): waves take alternate pages, operands straight from HBM.
template <typename T, int HD, int RT>
__global__ __launch_bounds__(256) void attn_direct_kernel(AttnArgs a) {
  if (a.done && *a.done) return;
  constexpr int NW = 4, HC = HD / 32, OT = HD / 16;
  __shared__ float s_o[NW][RT * 16][HD];
  __shared__ float s_ml[NW][RT * 16][2];

  const AttnItem it = a.items[blockIdx.x];
  if (it.is_block) return;   // block keys: attn_finish_kernel
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int npg = (nkeys + SUB - 1) / SUB;
  const size_t page0 = (size_t)a.page_off[it.seq] + it.k_begin / SUB;
  const size_t pstride = (size_t)a.Hkv * SUB * HD;   // elements between pages
  const T *Kp = reinterpret_cast<const T *>(a.kc) + (page0 * a.Hkv + it.kvh) * SUB * HD;
  const T *Vp = reinterpret_cast<const T *>(a.vc) + (page0 * a.Hkv + it.kvh) * HD * SUB;

  AFrag<T> qf[RT][HC];
  load_q<T, HD, RT>(a, it, 0, g, l16, qf);

  float m_run[RT], l_run[RT];
  f32x4_t o[RT][OT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[rt][t] = zero4();
  }

  Frag<T> kf[2][2][HC], vf[2][OT];   // [buffer] page operands
  auto fetch = [&](auto bufc, int pg) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    if (pg < npg) {
      const T *kp = Kp + (size_t)pg * pstride;
      const T *vp = Vp + (size_t)pg * pstride;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < HC; ++c) kf[b][h][c].load(kp + krow(h, l16) * HD + c * 32 + g * 8);
#pragma unroll
      for (int t = 0; t < OT; ++t) vf[b][t].load(vp + (16 * t + l16) * SUB + g * 8);
    }
  };
  auto consume = [&](auto bufc, int pg) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    const int kvalid = nkeys - pg * SUB;
    if (kvalid < SUB) {
#pragma unroll
      for (int t = 0; t < OT; ++t) mask_v<T>(vf[b][t], g, kvalid);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      PageMath<T, HD>::run([&](int h, int c) -> const Frag<T> & { return kf[b][h][c]; },
                           [&](int t) -> const Frag<T> & { return vf[b][t]; }, qf[rt], a.scale, kvalid, g,
                           m_run[rt], l_run[rt], o[rt]);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int pg = wave;
  fetch(B0{}, pg);
  while (pg < npg) {
    fetch(B1{}, pg + NW);
    consume(B0{}, pg);
    pg += NW;
    if (pg >= npg) break;
    fetch(B0{}, pg + NW);
    consume(B1{}, pg);
    pg += NW;
  }

  // Merge the four waves' states (wave order) through LDS.
  float l_tot[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    l_tot[rt] = sum_groups(l_run[rt]);
    const int rr = rt * 16 + l16;
    if (g == 0) {
      s_ml[wave][rr][0] = m_run[rt];
      s_ml[wave][rr][1] = l_tot[rt];
    }
#pragma unroll
    for (int t = 0; t < OT; ++t) *reinterpret_cast<f32x4_t *>(&s_o[wave][rr][16 * t + 4 * g]) = o[rt][t];
  }
  __syncthreads();
  constexpr int EPT = HD / 16;
  const int e0 = (threadIdx.x & 15) * EPT;
  for (int rr = threadIdx.x >> 4; rr < RT * 16 && rr < a.R; rr += 16) {
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) Mx = fmaxf(Mx, s_ml[w][rr][0]);
    float L = 0.f, acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_ml[w][rr][0];
      const float f = (mw == -INFINITY) ? 0.f : __expf(mw - Mx);
      L += s_ml[w][rr][1] * f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[e] += s_o[w][rr][e0 + e] * f;
    }
    const size_t prow = (size_t)blockIdx.x * a.R + rr;
    if ((threadIdx.x & 15) == 0) {
      a.part_ml[prow * 2 + 0] = Mx;
      a.part_ml[prow * 2 + 1] = L;
    }
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *reinterpret_cast<float4 *>(&a.part_o[prow * HD + e0 + e]) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
}

// Grouped-query shape (R > 32): each page is copied once into LDS (K rows and V^T rows,
// 16-byte copies) and the four waves, RT 16-row tiles each, read it from there.
template <typename T, int HD, int RT>
__global__ __launch_bounds__(256) void attn_shared_kernel(AttnArgs a) {
  if (a.done && *a.done) return;
  constexpr int NW = 4, HC = HD / 32, OT = HD / 16;
  constexpr int KP = HD + Pad<T>::K;       // K row stride in LDS (elements)
  constexpr int VP = SUB + Pad<T>::V;      // V^T row stride in LDS (elements)
  constexpr int KCH = SUB * HD / 8;        // 8-element chunks of a K page (= of a V page)
  constexpr int PER_T = (KCH + 255) / 256;
  __shared__ __attribute__((aligned(16))) T s_k[SUB * KP];
  __shared__ __attribute__((aligned(16))) T s_vt[HD * VP];

  const AttnItem it = a.items[blockIdx.x];
  if (it.is_block) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int npg = (nkeys + SUB - 1) / SUB;
  const size_t page0 = (size_t)a.page_off[it.seq] + it.k_begin / SUB;
  const size_t pstride = (size_t)a.Hkv * SUB * HD;
  const T *Kp = reinterpret_cast<const T *>(a.kc) + (page0 * a.Hkv + it.kvh) * SUB * HD;
  const T *Vp = reinterpret_cast<const T *>(a.vc) + (page0 * a.Hkv + it.kvh) * HD * SUB;
  const int rt0 = (blockIdx.y * NW + wave) * RT;

  AFrag<T> qf[RT][HC];
  load_q<T, HD, RT>(a, it, rt0, g, l16, qf);
  float m_run[RT], l_run[RT];
  f32x4_t o[RT][OT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[rt][t] = zero4();
  }

  Frag<T> kreg[PER_T], vreg[PER_T];
  auto fetch = [&](int pg) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < KCH && pg < npg) {
        kreg[i].load(Kp + (size_t)pg * pstride + (size_t)c * 8);
        vreg[i].load(Vp + (size_t)pg * pstride + (size_t)c * 8);
      }
    }
  };
  auto stash = [&](int kvalid) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c < KCH) {
        const int krow_ = c / (HD / 8), kpart = c % (HD / 8);
        *reinterpret_cast<Frag<T> *>(&s_k[krow_ * KP + kpart * 8]) = kreg[i];
        const int vrow = c / (SUB / 8), vpart = c % (SUB / 8);
        Frag<T> v = vreg[i];
        mask_v<T>(v, vpart, kvalid);
        *reinterpret_cast<Frag<T> *>(&s_vt[vrow * VP + vpart * 8]) = v;
      }
    }
  };

  fetch(0);
  for (int pg = 0; pg < npg; ++pg) {
    const int kvalid = nkeys - pg * SUB;
    __syncthreads();   // every wave is done reading the previous page
    stash(kvalid);
    __syncthreads();   // this page is in LDS
    if (pg + 1 < npg) fetch(pg + 1);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      PageMath<T, HD>::run(
          [&](int h, int c) { return *reinterpret_cast<const Frag<T> *>(&s_k[krow(h, l16) * KP + c * 32 + g * 8]); },
          [&](int t) { return *reinterpret_cast<const Frag<T> *>(&s_vt[(16 * t + l16) * VP + g * 8]); }, qf[rt],
          a.scale, kvalid, g, m_run[rt], l_run[rt], o[rt]);
  }
  float l_tot[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) l_tot[rt] = sum_groups(l_run[rt]);
  store_partial<HD, RT>(a, blockIdx.x, rt0, g, l16, m_run, l_tot, o);
}

// One workgroup per (pair, 16 query rows): the B block keys in fp32 (16 threads per row,
// HD/16 head dimensions each), then the merge with the pair's prefix partials in item
// order, and o.  The partial maxima and sums of the pair are first read in parallel
// into LDS; the partial outputs are then read in independent batches.
constexpr int FIN_ITEMS = 256;   // prefix items per pair the finish kernel merges

template <typename T, int HD>
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
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] *= inv;
  const int orow = it.seq * a.B + p, ocol = (it.kvh * a.G + j) * HD + e0;
  if (a.o) {
    float *out = a.o + (size_t)orow * a.ldo + ocol;
#pragma unroll
    for (int e = 0; e < EPT; ++e) out[e] = acc[e];
  }
  if (a.o_afl) {   // input of the output projection
    const int KTo = a.H * HD / 32;
    if constexpr (EPT % 8 == 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 8) afl_put8<T>(a.o_afl, KTo, orow, ocol + e, acc + e);
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) afl_put<T>(a.o_afl, KTo, orow, ocol + e, acc[e]);
    }
  }
}

template <typename T, int HD>
hipError_t launch_hd(const AttnArgs &a, hipStream_t s) {
  if (a.R <= 16) {
    hipLaunchKernelGGL((attn_direct_kernel<T, HD, 1>), dim3(a.n_items), dim3(256), 0, s, a);
  } else if (a.R <= 32) {
    hipLaunchKernelGGL((attn_direct_kernel<T, HD, 2>), dim3(a.n_items), dim3(256), 0, s, a);
  } else if (a.R <= 64) {
    hipLaunchKernelGGL((attn_shared_kernel<T, HD, 1>), dim3(a.n_items, (a.R + 63) / 64), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_shared_kernel<T, HD, 4>), dim3(a.n_items, (a.R + 255) / 256), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(a.n_pairs, (a.R + 15) / 16);
  hipLaunchKernelGGL((attn_finish_kernel<T, HD>), grid, dim3(256), 0, s, a);
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
