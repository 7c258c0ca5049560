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
// Work items (built on the host per prefix binding): runs of prefix pages of one
// (sequence, K/V head) pair, and one item per pair for the block's own keys.  Every
// item writes a partial state per query row: running max m, sum l of exp(s - m), and
// the unnormalised output o, into its slot; a pair's slots are consecutive in key
// order, and attn_merge_kernel combines them in that order.  Items are launched
// longest first, so that the short ragged ends of the pairs fill the last wave of
// workgroups instead of trailing it.
//
// Prefix items, flash-decoding style.  The cache is paged (32 tokens per page; per page
// and K/V head one contiguous 8 KiB block of K and one of V for bf16), laid out so that
// every MFMA operand is one contiguous KiB per wave instruction straight from HBM:
//   S^T[key][row] = K . Q^T      (A = K rows, B = Q fragments held in registers).  The
//                                 K block is stored as [hd / 32][2 halves][16 rows][32]:
//                                 row i of half h is key krow(h, i), so that lane group g
//                                 holds the scores of keys 8g .. 8g+7 of the page;
//   O^T[hd][row] += V^T . P^T    (A = V^T rows of the page, stored [hd][32 keys]; B = P
//                                 straight from the S^T accumulators)
// with an online softmax per query row.  Two shapes of work:
//   * few query rows per K/V head (R = G*B <= 32, multi-head attention): the four
//     waves of a workgroup take alternate pages of the item with no LDS and no barrier
//     in the key loop (the next page in flight while the current one is consumed), and
//     merge their states in LDS at the end;
//   * many rows (grouped-query heads): each page is staged once into LDS through a
//     three-page register ring and the eight waves, each owning RTW 16-row tiles, read
//     it from there.
// Queries are fp32 activations; against bf16 keys each query fragment enters the MFMA
// as a bf16 high part plus a bf16 remainder, and the probabilities are split the same
// way for P.V, so q and P keep ~16 significant bits.  Key slots past the end of a
// sequence's last page are masked (scores to -inf, values to 0).
//
// Block items: the B block keys/values are fp32 activations from the QKV projection and
// few, so they are attended in fp32 on the VALU (16 threads per query row).  For the
// frozen context tower's pass (causal) block query p sees block keys 0..p only; the
// prefix is always seen whole.
#include "td_device.h"
#include "td_kernels.h"

#include <type_traits>

namespace td {

namespace {

constexpr int SUB = KV_PAGE;   // keys per page
// Pages in flight per wave in the few-row kernel (measured: three were slower at every
// shape, batch 1 to 64 x 4096).
constexpr int DIRECT_DEPTH = 2;
constexpr int BMAX = 32;       // largest block size

// Element offset, within a K page block, of MFMA row i of S^T half h, hd chunk c (32
// elements).  Row i of half h holds key 8 (i / 4) + 4 h + i % 4, so that lane group g
// receives the scores of keys 8g .. 8g+7.
TD_DEV int kpos(int c, int h, int i) { return ((c * 2 + h) * 16 + i) * 32; }

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

// Query values of rows (rt0 + rt) * 16 + l16, dimensions c * 32 + g * 8 .. + 7, as fp32:
// loads only, no branch (rows past R read row 0 and are zeroed by q_frags), so that
// the caller can issue further loads before the first wait.
template <int HD, int RT>
TD_DEV void load_q_raw(const AttnArgs &a, const AttnItem &it, int rt0, int g, int l16, float (&v)[RT][HD / 32][8]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = (rt0 + rt) * 16 + l16;
    const int rr = rho < a.R ? rho : 0;
    const int j = rr / a.B, p = rr % a.B;
#pragma unroll
    for (int c = 0; c < HD / 32; ++c)
      load8f(a.qkv + (size_t)(it.seq * a.B + p) * a.Nqkv + (size_t)(it.kvh * a.G + j) * HD + c * 32 + g * 8, v[rt][c]);
  }
}

template <typename T, int HD, int RT>
TD_DEV void q_frags(const AttnArgs &a, int rt0, int l16, const float (&v)[RT][HD / 32][8], AFrag<T> (&qf)[RT][HD / 32]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const bool valid = (rt0 + rt) * 16 + l16 < a.R;
#pragma unroll
    for (int c = 0; c < HD / 32; ++c) {
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = valid ? v[rt][c][e] : 0.f;
      qf[rt][c].set8(w);
    }
  }
}

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

template <int HD> constexpr int block_item_lds() { return 2 * BMAX * (HD + 1); }   // floats

// The block's own keys of one (sequence, K/V head) pair, fp32 on the VALU: 16 threads
// per query row (HD/16 dimensions each), 16 rows at a time.  sm: block_item_lds floats
// of LDS.  Writes the pair's block partial (m, l, o) to the item's slot.
template <int HD, int NT = 256>
TD_DEV void block_item(const AttnArgs &a, const AttnItem &it, int item, float *sm) {
  constexpr int EPT = HD / 16, KPT = BMAX * HD / NT;
  float *s_k = sm, *s_v = sm + BMAX * (HD + 1);
  const float *base = a.qkv + (size_t)it.seq * a.B * a.Nqkv;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {   // all of the pair's block keys and values in flight at once
    const int idx = threadIdx.x + NT * i;
    const int key = idx / HD, e = idx % HD;
    if (key < a.B) {
      s_k[key * (HD + 1) + e] = base[(size_t)key * a.Nqkv + (size_t)(a.H + it.kvh) * HD + e];
      s_v[key * (HD + 1) + e] = base[(size_t)key * a.Nqkv + (size_t)(a.H + a.Hkv + it.kvh) * HD + e];
    }
  }
  __syncthreads();
  const int sub = threadIdx.x & 15, e0 = sub * EPT;
  for (int rho0 = 0; rho0 < a.R; rho0 += NT / 16) {
    const int rho = rho0 + (threadIdx.x >> 4);
    if (rho >= a.R) break;   // whole 16-lane groups leave together
    const int j = rho / a.B, p = rho % a.B;
    const float *q = base + (size_t)p * a.Nqkv + (size_t)(it.kvh * a.G + j) * HD + e0;
    float qv[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) qv[e] = q[e];
    const int kmax = a.causal ? min(a.B, p + 1) : a.B;   // causal: block keys 0..p
    float sc[BMAX];
    float m = -INFINITY;
#pragma unroll
    for (int key = 0; key < BMAX; ++key) {
      if (key < a.B) {
        float dsum = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) dsum += qv[e] * s_k[key * (HD + 1) + e0 + e];
        sc[key] = key < kmax ? sum16(dsum) * a.scale : -INFINITY;
        m = fmaxf(m, sc[key]);
      }
    }
    float l = 0.f, ov[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) ov[e] = 0.f;
#pragma unroll
    for (int key = 0; key < BMAX; ++key) {
      if (key < kmax) {
        const float pk = __expf(sc[key] - m);
        l += pk;
#pragma unroll
        for (int e = 0; e < EPT; ++e) ov[e] += pk * s_v[key * (HD + 1) + e0 + e];
      }
    }
    const size_t prow = (size_t)item * a.R + rho;
    if (sub == 0) {
      a.part_ml[prow * 2 + 0] = m;
      a.part_ml[prow * 2 + 1] = l;
    }
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *reinterpret_cast<float4 *>(&a.part_o[prow * HD + e0 + e]) = make_float4(ov[e], ov[e + 1], ov[e + 2], ov[e + 3]);
  }
}

// Few-row shape (R <= 32, multi-head attention): the NW = 4 waves take pages w, w + 4,
// ..., operands straight from HBM, each wave with DEPTH pages in flight (a ring).  (Eight waves
// measured slower: with two workgroups per CU their registers spill; with one, on a grid
// of one item per CU (batch 1), attention took 18% longer.)  The pair's first item also attends
// the block's own keys: their loads are issued before the first pages', so the fp32
// block pass (block_item's arithmetic, into LDS) runs while the pages are in flight, and
// its state is merged after the waves' in the fixed order waves 0..NW-1, block.
template <int N, typename F>
TD_DEV void static_for(F &&f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// bf16 pages with one row tile fit two workgroups per CU (243 VGPRs when told so; left
// alone the compiler also took 32 AGPRs and one); the others need the whole register file.
template <typename T, int HD, int RT, int NW, int DEPTH>
__global__ __launch_bounds__(64 * NW, (sizeof(T) == 2 && RT == 1) ? 2 : 1) void attn_direct_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW, HC = HD / 32, OT = HD / 16, EPT = HD / 16, KPT = BMAX * HD / NT;
  constexpr int MERGE = (NW + 1) * RT * 16 * (HD + 2);   // waves' and the block's states
  constexpr int LDS = MERGE + block_item_lds<HD>();
  __shared__ float smem[LDS];
  float(*s_o)[RT * 16][HD] = reinterpret_cast<float(*)[RT * 16][HD]>(smem);
  float(*s_ml)[RT * 16][2] = reinterpret_cast<float(*)[RT * 16][2]>(smem + (NW + 1) * RT * 16 * HD);
  float *s_bk = smem + MERGE, *s_bv = s_bk + BMAX * (HD + 1);

  const AttnItem it = a.items[blockIdx.x];   // loaded together with the loop-exit flag
  if (a.done && *a.done) return;
  // A sequence whose block is fully adopted needs no attention.  Its flag is read with a
  // scalar load (nothing in the kernel writes it, and the kernel's start invalidates the
  // scalar cache), whose wait does not hold the vector loads back; the pages' items test
  // it once their first pages are requested.
  if (it.is_block == 1) {
    if (a.seq_done[it.seq]) return;
    block_item<HD, NT>(a, it, it.slot, smem);
    return;
  }
  const bool with_block = it.is_block == 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int npg = (nkeys + SUB - 1) / SUB;
  const size_t pstride = (size_t)a.Hkv * SUB * HD;   // elements between pages
  const T *Kp = reinterpret_cast<const T *>(a.kc) + ((size_t)it.page0 * a.Hkv + it.kvh) * SUB * HD;
  const T *Vp = reinterpret_cast<const T *>(a.vc) + ((size_t)it.page0 * a.Hkv + it.kvh) * HD * SUB;

  // Block keys/values (fp32, this thread's KPT elements) and the block pass's query
  // values (16 threads per row, EPT dimensions each): issued first.
  constexpr int BPASS = (RT * 16 + NT / 16 - 1) / (NT / 16);
  const int sub = threadIdx.x & 15, e0 = sub * EPT;
  const float *bbase = a.qkv + (size_t)it.seq * a.B * a.Nqkv;
  float bk[KPT], bv[KPT], bq[BPASS][EPT];
  if (with_block) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = threadIdx.x + NT * i, key = idx / HD, e = idx % HD;
      const int kk = key < a.B ? key : 0;
      bk[i] = bbase[(size_t)kk * a.Nqkv + (size_t)(a.H + it.kvh) * HD + e];
      bv[i] = bbase[(size_t)kk * a.Nqkv + (size_t)(a.H + a.Hkv + it.kvh) * HD + e];
    }
#pragma unroll
    for (int ps = 0; ps < BPASS; ++ps) {
      const int rho = ps * (NT / 16) + (threadIdx.x >> 4);
      const int rr = rho < a.R ? rho : 0;
      const float *q = bbase + (size_t)(rr % a.B) * a.Nqkv + (size_t)(it.kvh * a.G + rr / a.B) * HD + e0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) bq[ps][e] = q[e];
    }
  }

  float qraw[RT][HC][8];
  load_q_raw<HD, RT>(a, it, 0, g, l16, qraw);

  float m_run[RT], l_run[RT];
  f32x4_t o[RT][OT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[rt][t] = zero4();
  }

  AFrag<T> qf[RT][HC];                       // filled once the first pages are in flight
  Frag<T> kf[DEPTH][2][HC], vf[DEPTH][OT];   // [buffer] page operands
  auto fetch = [&](auto bufc, int pg) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    if (pg < npg) {
      const T *kp = Kp + (size_t)pg * pstride;
      const T *vp = Vp + (size_t)pg * pstride;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < HC; ++c) kf[b][h][c].load_nt(kp + kpos(c, h, l16) + g * 8);
#pragma unroll
      for (int t = 0; t < OT; ++t) vf[b][t].load_nt(vp + (16 * t + l16) * SUB + g * 8);
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
  const int pg0 = wave;
  __builtin_amdgcn_sched_barrier(0);   // the block and query loads stay ahead of the pages'
  static_for<DEPTH - 1>([&](auto sc) { fetch(sc, pg0 + decltype(sc)::value * NW); });
  __builtin_amdgcn_sched_barrier(0);
  if (a.seq_done[it.seq]) return;
  q_frags<T, HD, RT>(a, 0, l16, qraw, qf);

  if (with_block) {   // workgroup-uniform
    // The block pass: scores over the B block keys in fp32, one softmax, into slot NW.
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = threadIdx.x + NT * i, key = idx / HD, e = idx % HD;
      s_bk[key * (HD + 1) + e] = bk[i];
      s_bv[key * (HD + 1) + e] = bv[i];
    }
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < BPASS; ++ps) {
      const int rho = ps * (NT / 16) + (threadIdx.x >> 4);
      float sc[BMAX];
      float m = -INFINITY;
      const int kmax = a.causal ? min(a.B, rho % a.B + 1) : a.B;   // causal: block keys 0..p
#pragma unroll
      for (int key = 0; key < BMAX; ++key) {
        if (key < a.B) {
          float dsum = 0.f;
#pragma unroll
          for (int e = 0; e < EPT; ++e) dsum += bq[ps][e] * s_bk[key * (HD + 1) + e0 + e];
          sc[key] = key < kmax ? sum16(dsum) * a.scale : -INFINITY;
          m = fmaxf(m, sc[key]);
        }
      }
      float l = 0.f, ov[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) ov[e] = 0.f;
#pragma unroll
      for (int key = 0; key < BMAX; ++key) {
        if (key < kmax) {
          const float pk = __expf(sc[key] - m);
          l += pk;
#pragma unroll
          for (int e = 0; e < EPT; ++e) ov[e] += pk * s_bv[key * (HD + 1) + e0 + e];
        }
      }
      if (rho < RT * 16) {
        if (sub == 0) {
          s_ml[NW][rho][0] = m;
          s_ml[NW][rho][1] = l;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) s_o[NW][rho][e0 + e] = ov[e];
      }
    }
  }

  // Ring of DEPTH pages per wave: page pg + s * NW sits in buffer s; the page DEPTH - 1
  // steps ahead is requested before each page is consumed.
  for (int pg = pg0; pg < npg; pg += DEPTH * NW) {
    static_for<DEPTH>([&](auto sc) {
      constexpr int st = decltype(sc)::value;
      using Ahead = std::integral_constant<int, (st + DEPTH - 1) % DEPTH>;
      fetch(Ahead{}, pg + (st + DEPTH - 1) * NW);
      if (pg + st * NW < npg) consume(sc, pg + st * NW);
    });
  }

  // Merge the waves' states (wave order), then the block's, through LDS.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l_tot = sum_groups(l_run[rt]);
    const int rr = rt * 16 + l16;
    if (g == 0) {
      s_ml[wave][rr][0] = m_run[rt];
      s_ml[wave][rr][1] = l_tot;
    }
#pragma unroll
    for (int t = 0; t < OT; ++t) *reinterpret_cast<f32x4_t *>(&s_o[wave][rr][16 * t + 4 * g]) = o[rt][t];
  }
  __syncthreads();
  const int nst = with_block ? NW + 1 : NW;
  for (int rr = threadIdx.x >> 4; rr < RT * 16 && rr < a.R; rr += 4 * NW) {
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w <= NW; ++w)
      if (w < nst) Mx = fmaxf(Mx, s_ml[w][rr][0]);
    float L = 0.f, acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w <= NW; ++w) {
      if (w < nst) {
        const float mw = s_ml[w][rr][0];
        const float f = (mw == -INFINITY) ? 0.f : __expf(mw - Mx);
        L += s_ml[w][rr][1] * f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] += s_o[w][rr][e0 + e] * f;
      }
    }
    const size_t prow = (size_t)it.slot * a.R + rr;
    if (sub == 0) {
      a.part_ml[prow * 2 + 0] = Mx;
      a.part_ml[prow * 2 + 1] = L;
    }
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *reinterpret_cast<float4 *>(&a.part_o[prow * HD + e0 + e]) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
}

// Grouped-query shape (R > 32): eight waves (two per SIMD) share each page, wave w
// owning RTW 16-row tiles of the pair's query rows (RTW = 1: 128 rows per workgroup;
// more rows take several workgroups per item).  Pages reach LDS through a ring of
// DEPTH pages held in registers (every thread loads its share of page p + DEPTH while
// page p is multiplied), then one 16-byte store per chunk into the double-buffered,
// padded LDS stage of PPS = 2 pages (K in its page layout with 32-element rows, V^T
// rows); one barrier per two pages (one per page measured 11% slower, three 10%).  Each wave reads a page's K fragments from LDS once and reuses them for all of
// its row tiles; V fragments are read at their use.
template <typename T, int HD, int RTW>
__global__ __launch_bounds__(512) void attn_group_kernel(AttnArgs a) {
  constexpr int NW = 8, NT = 64 * NW, HC = HD / 32, OT = HD / 16;
  constexpr int PPS = 2;                   // pages per LDS stage (measured: 1 and 3 slower)
  constexpr int DEPTH = 2 * PPS;           // pages in flight in registers (two stages)
  constexpr int KR = 32 + Pad<T>::K;       // K row stride in LDS (elements)
  constexpr int VP = SUB + Pad<T>::V;      // V^T row stride in LDS (elements)
  constexpr int KCH = SUB * HD / 8;        // 8-element chunks of a K page (= of a V page)
  constexpr int CPT = (KCH + NT - 1) / NT; // chunks of each per thread
  constexpr int KBUF = HC * 2 * 16 * KR, VBUF = HD * VP;   // elements of one LDS page
  constexpr int BYTES_PAGES = DEPTH * (KBUF + VBUF) * (int)sizeof(T);   // two stages of PPS pages
  constexpr int BYTES_BLOCK = block_item_lds<HD>() * 4;
  constexpr int BYTES = BYTES_PAGES > BYTES_BLOCK ? BYTES_PAGES : BYTES_BLOCK;
  __shared__ __attribute__((aligned(16))) char smem[BYTES];
  T *s_k = reinterpret_cast<T *>(smem);          // [stage][page][KBUF]
  T *s_vt = s_k + DEPTH * KBUF;                  // [stage][page][VBUF]

  // Workgroup b takes row group b % YS of item b / YS: the row groups of an item are
  // neighbours in launch order, so its pages are read while still in the last-level cache.
  const int YS = (a.R + NW * RTW * 16 - 1) / (NW * RTW * 16);
  const int item = blockIdx.x / YS, ygrp = blockIdx.x % YS;
  const AttnItem it = a.items[item];   // loaded together with the loop-exit flag
  if (a.done && *a.done) return;
  if (a.seq_done[it.seq]) return;   // block fully adopted: no attention needed
  if (it.is_block) {
    if (ygrp == 0) block_item<HD, NT>(a, it, it.slot, reinterpret_cast<float *>(smem));
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int npg = (nkeys + SUB - 1) / SUB;
  const size_t pstride = (size_t)a.Hkv * SUB * HD;
  const T *Kp = reinterpret_cast<const T *>(a.kc) + ((size_t)it.page0 * a.Hkv + it.kvh) * SUB * HD;
  const T *Vp = reinterpret_cast<const T *>(a.vc) + ((size_t)it.page0 * a.Hkv + it.kvh) * HD * SUB;
  const int rt0 = (ygrp * NW + wave) * RTW;

  AFrag<T> qf[RTW][HC];
  load_q<T, HD, RTW>(a, it, rt0, g, l16, qf);
  float m_run[RTW], l_run[RTW];
  f32x4_t o[RTW][OT];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[rt][t] = zero4();
  }

  // Register ring: slot r holds this thread's chunks of one page.  Loads are
  // unconditional (pages past the end reread the last page) so that the waits before
  // each store are exact.
  constexpr int W = frag_words<T>();
  u32x4_t kreg[DEPTH][CPT][W], vreg[DEPTH][CPT][W];
  auto fetch = [&](auto slotc, int pg) __attribute__((always_inline)) {
    constexpr int r = decltype(slotc)::value;
    const size_t base = (size_t)min(pg, npg - 1) * pstride;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = min((int)threadIdx.x + NT * i, KCH - 1);
      const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(Kp + base + (size_t)c * 8);
      const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(Vp + base + (size_t)c * 8);
#pragma unroll
      for (int w = 0; w < W; ++w) {   // pages are read once per step: streaming loads
        kreg[r][i][w] = __builtin_nontemporal_load(kp + w);
        vreg[r][i][w] = __builtin_nontemporal_load(vp + w);
      }
    }
  };
  auto stash = [&](auto slotc, int buf, int kvalid) __attribute__((always_inline)) {
    constexpr int r = decltype(slotc)::value;
    T *sk = s_k + buf * KBUF;
    T *sv = s_vt + buf * VBUF;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + NT * i;
      if (c < KCH) {
        *reinterpret_cast<Frag<T> *>(&sk[(c >> 2) * KR + (c & 3) * 8]) = frag_of(kreg[r][i], T{});
        const int vrow = c / (SUB / 8), vpart = c % (SUB / 8);
        Frag<T> v = frag_of(vreg[r][i], T{});
        mask_v<T>(v, vpart, kvalid);
        *reinterpret_cast<Frag<T> *>(&sv[vrow * VP + vpart * 8]) = v;
      }
    }
  };
  auto compute = [&](int buf, int kvalid) __attribute__((always_inline)) {
    const T *sk = s_k + buf * KBUF;
    const T *sv = s_vt + buf * VBUF;
    Frag<T> kf[2][HC];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < HC; ++c) kf[h][c] = *reinterpret_cast<const Frag<T> *>(&sk[((c * 2 + h) * 16 + l16) * KR + g * 8]);
    // V fragments are read from LDS at their use (once per row tile): holding them too
    // would exceed the 256 registers of a wave at two waves per SIMD.
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
      PageMath<T, HD>::run([&](int h, int c) -> const Frag<T> & { return kf[h][c]; },
                           [&](int t) { return *reinterpret_cast<const Frag<T> *>(&sv[(16 * t + l16) * VP + g * 8]); },
                           qf[rt], a.scale, kvalid, g, m_run[rt], l_run[rt], o[rt]);
  };
  // PPS pages per stage and barrier: stage h multiplies pages p .. p + PPS - 1 from LDS
  // stage buffer h while the register slots of stage h (now free) take pages p + DEPTH ..,
  // and the pages held in the other stage's slots are staged into the other buffer.
  auto stage = [&](auto hc, int p) __attribute__((always_inline)) {
    constexpr int h = decltype(hc)::value;
    static_for<PPS>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      fetch(std::integral_constant<int, h * PPS + i>{}, p + i + DEPTH);
    });
#pragma unroll
    for (int i = 0; i < PPS; ++i)
      if (p + i < npg) compute(h * PPS + i, nkeys - (p + i) * SUB);
    static_for<PPS>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (p + PPS + i < npg)
        stash(std::integral_constant<int, (1 - h) * PPS + i>{}, (1 - h) * PPS + i, nkeys - (p + PPS + i) * SUB);
    });
    __syncthreads();
  };
  static_for<DEPTH>([&](auto ic) { fetch(ic, decltype(ic)::value); });
  static_for<PPS>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if (i < npg) stash(ic, i, nkeys - i * SUB);
  });
  __syncthreads();
  for (int p = 0; p < npg; p += DEPTH) {
    stage(std::integral_constant<int, 0>{}, p);
    if (p + PPS >= npg) break;
    stage(std::integral_constant<int, 1>{}, p + PPS);
  }
  float l_tot[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) l_tot[rt] = sum_groups(l_run[rt]);
  store_partial<HD, RTW>(a, it.slot, rt0, g, l16, m_run, l_tot, o);
}

// Merge of a pair's partials in item order (prefix runs, then the block), one thread
// per (query row, 8 output dimensions): online log-sum-exp over batches of partials
// loaded together.  Writes o (fp32, natural layout, optional) and the output
// projection's input in fragment layout.
template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a) {
  constexpr int BATCH = 16;
  const int pair = blockIdx.x;
  const int first = a.pair_first[pair], cnt = a.pair_count[pair];   // loaded with the exit flag
  if (a.done && *a.done) return;
  if (a.seq_done[pair / a.Hkv]) return;   // block fully adopted: rows not read again
  const int rho = blockIdx.y * 16 + (threadIdx.x >> 2);
  const int e0 = blockIdx.z * 32 + (threadIdx.x & 3) * 8;
  if (rho >= a.R) return;
  float M = -INFINITY, L = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < cnt; i0 += BATCH) {
    float mi[BATCH], li[BATCH], oi[BATCH][8];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const size_t prow = (size_t)(first + min(i0 + b, cnt - 1)) * a.R + rho;
      mi[b] = a.part_ml[prow * 2 + 0];
      li[b] = a.part_ml[prow * 2 + 1];
      load8f(a.part_o + prow * HD + e0, oi[b]);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (i0 + b < cnt && mi[b] != -INFINITY) {
        const float Mn = fmaxf(M, mi[b]);
        const float wo = (M == -INFINITY) ? 0.f : __expf(M - Mn);
        const float wn = __expf(mi[b] - Mn);
        L = L * wo + li[b] * wn;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] * wo + oi[b][e] * wn;
        M = Mn;
      }
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  const int seq = pair / a.Hkv, kvh = pair % a.Hkv;
  const int j = rho / a.B, p = rho % a.B;
  const int orow = seq * a.B + p, ocol = (kvh * a.G + j) * HD + e0;
  if (a.o) {
    float *out = a.o + (size_t)orow * a.ldo + ocol;
    *reinterpret_cast<float4 *>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4 *>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (a.o_afl) afl_put8<T>(a.o_afl, a.H * HD / 32, orow, ocol, acc);
}

template <typename T, int HD>
hipError_t launch_hd(const AttnArgs &a, hipStream_t s) {
  if (a.R <= 16) {
    hipLaunchKernelGGL((attn_direct_kernel<T, HD, 1, 4, DIRECT_DEPTH>), dim3(a.n_items), dim3(256), 0, s, a);
  } else if (a.R <= ATTN_FEW_ROWS) {
    hipLaunchKernelGGL((attn_direct_kernel<T, HD, 2, 4, DIRECT_DEPTH>), dim3(a.n_items), dim3(256), 0, s, a);
  } else {   // one 16-row tile per wave, 128 rows per workgroup (more would spill)
    hipLaunchKernelGGL((attn_group_kernel<T, HD, 1>), dim3(a.n_items * ((a.R + 127) / 128)), dim3(512), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_merge_kernel<T, HD>), dim3(a.n_pairs, (a.R + 15) / 16, HD / 32), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnArgs &a, hipStream_t s) {
  if (a.n_items <= 0 || a.n_pairs <= 0 || a.B > BMAX || a.seq_done == nullptr) return hipErrorInvalidValue;
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
