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
// (sequence, K/V head) pair; the pair's first item also takes the block's own keys (a
// pair with no prefix has one item of no pages).  Every
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
//     four-page register ring and the eight waves, each owning RTW 16-row tiles, read
//     it from there.
// Queries are fp32 activations; against bf16 keys each query fragment enters the MFMA
// as a bf16 high part plus a bf16 remainder, and the probabilities are split the same
// way for P.V, so q and P keep ~16 significant bits.  Key slots past the end of a
// sequence's last page are masked (scores to -inf, values to 0).
//
// The block's own keys: the B block keys/values are fp32 activations from the QKV
// projection.  Staged in LDS (values transposed), each split into a bf16 high part and
// remainder, they are one more page of the online softmax on the matrix cores
// (block_page).  For the frozen context tower's pass (causal) block query p sees block
// keys 0..p only; the prefix is always seen whole.
#include "td_device.h"
#include "td_kernels.h"

#include <type_traits>

namespace td {

namespace {

constexpr int SUB = KV_PAGE;   // keys per page
// Pages in flight per wave in the few-row kernel (measured: three were slower at every
// shape, batch 1 to 64 x 4096, with one row tile and with two).
constexpr int DIRECT_DEPTH = 2;
constexpr int BMAX = 32;       // largest block size

// Element offset, within a K page block, of MFMA row i of S^T half h, hd chunk c (32
// elements).  Row i of half h holds key 8 (i / 4) + 4 h + i % 4, so that lane group g
// receives the scores of keys 8g .. 8g+7.
TD_DEV int kpos(int c, int h, int i) { return ((c * 2 + h) * 16 + i) * 32; }

// A page fragment staged in LDS as frag_words<T>() planes of 64 lane-ordered 16-byte
// words (1 KiB per plane): every wave instruction that reads or writes it touches one
// contiguous KiB, which the LDS serves without bank conflicts.  (Rows padded to 80 bytes
// instead measured one conflict cycle per active cycle.)
TD_DEV void lds_frag_put(char *f, int lane, const Frag<bf16_t> &v) { reinterpret_cast<uint4 *>(f)[lane] = v.raw; }
TD_DEV void lds_frag_put(char *f, int lane, const Frag<float> &v) {
  reinterpret_cast<float4 *>(f)[lane] = v.lo;
  reinterpret_cast<float4 *>(f + 1024)[lane] = v.hi;
}
TD_DEV void lds_frag_get(const char *f, int lane, Frag<bf16_t> &v) { v.raw = reinterpret_cast<const uint4 *>(f)[lane]; }
TD_DEV void lds_frag_get(const char *f, int lane, Frag<float> &v) {
  v.lo = reinterpret_cast<const float4 *>(f)[lane];
  v.hi = reinterpret_cast<const float4 *>(f + 1024)[lane];
}

// Zero the value slots of a V^T fragment (keys 8g .. 8g+7 of the page) at or past kvalid.
template <typename T>
TD_DEV void mask_v(Frag<T> &f, int g, int kvalid) {
  if (8 * g + 8 <= kvalid) return;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (8 * g + j < kvalid) ? f.get(j) : 0.f;
  f.set8(v);
}

// The queries enter the page products pre-scaled by scale * log2(e), so that the scores
// and the running maxima of the prefix pages are in base-2 units and the probabilities
// are single exp2 instructions; a partial's maximum is turned back into natural units
// (times ln 2) where it leaves the kernel or meets the block pass's state.
constexpr float LOG2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;

// Online-softmax update of one 16-row tile with one page of 32 keys, from its scores
// S^T (lane group g holding keys 8g .. 8g + 7; vis(key): the key is visible to this
// lane's query row, at least one per row) and pv(pf, o), which adds V^T . P^T for the
// probability fragment pf into o.  The running state is rescaled only when the maximum
// of some row of the wave grew: the factor is exactly 1 for every other row, so skipping
// it changes no bit.
template <typename T, int OT, typename VIS, typename PV>
TD_DEV void softmax_page(const f32x4_t (&st)[2], int g, VIS &&vis, float &m_run, float &l_run, f32x4_t (&o)[OT],
                         PV &&pv) {
  float sc[8];
  float mx = -INFINITY;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = vis(8 * g + 4 * h + r) ? st[h][r] : -INFINITY;
      sc[4 * h + r] = v;
      mx = fmaxf(mx, v);
    }
  mx = max_groups(mx);
  // m_new is finite (a visible key per row), so exp2(-inf - m_new) = 0 covers both the
  // hidden keys and the first page (m_run = -inf).
  const float m_new = fmaxf(m_run, mx);
  float p[8], psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(sc[j] - m_new);
    psum += p[j];
  }
  if (__ballot(m_new > m_run)) {   // wave-uniform
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[t] *= alpha;
  }
  l_run += psum;
  m_run = m_new;
  AFrag<T> pf;
  pf.set8(p);
  pv(pf, o);
}

// A prefix page: S^T from the bf16 key fragments, P.V from the value fragments.  FULL:
// all SUB keys of the page are valid.
template <typename T, int HD>
struct PageMath {
  static constexpr int HC = HD / 32, OT = HD / 16;
  template <bool FULL, typename KF, typename VF>
  TD_DEV static void run(const KF &kfrag, const VF &vfrag, const AFrag<T> (&qf)[HC], int kvalid, int g,
                         float &m_run, float &l_run, f32x4_t (&o)[OT]) {
    f32x4_t st[2] = {zero4(), zero4()};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < HC; ++c) st[h] = mma_b(kfrag(h, c), qf[c], st[h]);
    softmax_page<T>(st, g, [&](int key) { return FULL || key < kvalid; }, m_run, l_run, o,
                    [&](const AFrag<T> &pf, f32x4_t(&oo)[OT]) {
#pragma unroll
                      for (int t = 0; t < OT; ++t) oo[t] = mma_b(vfrag(t), pf, oo[t]);
                    });
  }
};

// Product of two split operands: high x high + high x low + low x high (the dropped
// low x low term is below 2^-16 of the product); fp32 operands multiply as they are.
TD_DEV f32x4_t mma_ab(const AFrag<bf16_t> &a, const AFrag<bf16_t> &b, f32x4_t acc) {
  acc = mma(a.hi, b.hi, acc);
  acc = mma(a.hi, b.lo, acc);
  return mma(a.lo, b.hi, acc);
}
TD_DEV f32x4_t mma_ab(const AFrag<float> &a, const AFrag<float> &b, f32x4_t acc) { return mma(a.f, b.f, acc); }

// Row strides (floats) of the block's keys [BMAX][BKS] and transposed values [HD][BVS]
// staged in LDS: 16-byte aligned rows, so that a lane's eight consecutive elements are
// two 16-byte reads.
template <int HD> constexpr int bks() { return HD + 4; }
constexpr int BVS = BMAX + 4;
template <int HD> constexpr int block_page_lds() { return BMAX * bks<HD>() + HD * BVS; }   // floats

// The block's own nb keys as one more page of the online softmax, on the matrix cores:
// keys and values are fp32 activations, split into bf16 high and low parts (three
// products per operand pair) and multiplied against the pre-scaled queries.  MFMA row i
// of half h is key 8 (i / 4) + 4 h + i % 4, as in the prefix pages.  causal_p >= 0: the
// row sees block keys 0..causal_p only (the frozen context tower's pass).
template <typename T, int HD>
TD_DEV void block_page(const float *s_k, const float *s_vt, const AFrag<T> (&qf)[HD / 32], int nb, int causal_p, int g,
                       int l16, float &m_run, float &l_run, f32x4_t (&o)[HD / 16]) {
  constexpr int HC = HD / 32, OT = HD / 16;
  f32x4_t st[2] = {zero4(), zero4()};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float *kr = s_k + (8 * (l16 >> 2) + 4 * h + (l16 & 3)) * bks<HD>() + 8 * g;
#pragma unroll
    for (int c = 0; c < HC; ++c) {
      float v[8];
      const f32x4_t a = *reinterpret_cast<const f32x4_t *>(kr + 32 * c);
      const f32x4_t b = *reinterpret_cast<const f32x4_t *>(kr + 32 * c + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[4 + j] = b[j];
      }
      AFrag<T> kf;
      kf.set8(v);
      st[h] = mma_ab(kf, qf[c], st[h]);
    }
  }
  softmax_page<T>(st, g, [&](int key) { return key < nb && (causal_p < 0 || key <= causal_p); }, m_run, l_run, o,
                  [&](const AFrag<T> &pf, f32x4_t(&oo)[OT]) {
#pragma unroll
                    for (int t = 0; t < OT; ++t) {
                      const float *vr = s_vt + (16 * t + l16) * BVS + 8 * g;
                      float v[8];
                      const f32x4_t a = *reinterpret_cast<const f32x4_t *>(vr);
                      const f32x4_t b = *reinterpret_cast<const f32x4_t *>(vr + 4);
#pragma unroll
                      for (int j = 0; j < 4; ++j) {
                        v[j] = a[j];
                        v[4 + j] = b[j];
                      }
                      AFrag<T> vf;
                      vf.set8(v);
                      oo[t] = mma_ab(vf, pf, oo[t]);
                    }
                  });
}

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
  const float qs = a.scale * LOG2E;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const bool valid = (rt0 + rt) * 16 + l16 < a.R;
#pragma unroll
    for (int c = 0; c < HD / 32; ++c) {
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = valid ? v[rt][c][e] * qs : 0.f;
      qf[rt][c].set8(w);
    }
  }
}

template <typename T, int HD, int RT>
TD_DEV void load_q(const AttnArgs &a, const AttnItem &it, int rt0, int g, int l16, AFrag<T> (&qf)[RT][HD / 32]) {
  const float qs = a.scale * LOG2E;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = (rt0 + rt) * 16 + l16;
#pragma unroll
    for (int c = 0; c < HD / 32; ++c) {
      if (rho < a.R) {
        const int j = rho / a.B, p = rho % a.B;
        float v[8];
        load8f(a.qkv + (size_t)(it.seq * a.B + p) * a.Nqkv + (size_t)(it.kvh * a.G + j) * HD + c * 32 + g * 8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= qs;
        qf[rt][c].set8(v);
      } else {
        qf[rt][c].zero();
      }
    }
  }
}

// Partial state of rows (rt0 + rt) * 16 + l16 -> the item's slot (the maximum in natural
// units).
template <int HD, int RT>
TD_DEV void store_partial(const AttnArgs &a, int item, int rt0, int g, int l16, const float (&m_run)[RT],
                          const float (&l_tot)[RT], const f32x4_t (&o)[RT][HD / 16]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = (rt0 + rt) * 16 + l16;
    if (rho < a.R) {
      const size_t prow = (size_t)item * a.R + rho;
      if (g == 0) {
        a.part_ml[prow * 2 + 0] = m_run[rt] * LN2;
        a.part_ml[prow * 2 + 1] = l_tot[rt];
      }
#pragma unroll
      for (int t = 0; t < HD / 16; ++t)
        *reinterpret_cast<f32x4_t *>(&a.part_o[prow * HD + 16 * t + 4 * g]) = o[rt][t];
    }
  }
}

// Few-row shape (R <= 32, multi-head attention): the NW = 4 waves take pages w, w + 4,
// ..., operands straight from HBM, each wave with DEPTH pages in flight (a ring).  (Eight waves
// measured slower: with two workgroups per CU their registers spill; with one, on a grid
// of one item per CU (batch 1), attention took 18% longer.)  The pair's first item also attends
// the block's own keys: their loads are issued before the first pages', the keys and
// values are staged in LDS, and wave rt < RT takes them (block_page, on the matrix
// cores) as the first page of its row tile rt while its prefix pages are in flight.  (An
// fp32 pass over them on the VALU, 16 threads per row, took 15 us of the item's 49 at
// the batch-64 block-32 sweep, with the CU streaming no pages meanwhile.)
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
  constexpr int NT = 64 * NW, HC = HD / 32, OT = HD / 16, KPT = BMAX * HD / NT;
  // The states' rows are padded by 4 words, so that the 16 rows of an MFMA tile store
  // their 16-byte pieces into distinct banks.
  constexpr int HS = HD + 4;
  constexpr int MERGE = NW * RT * 16 * (HS + 2);   // the waves' states
  constexpr int LDS = MERGE + block_page_lds<HD>();
  __shared__ __attribute__((aligned(16))) float smem[LDS];
  float(*s_o)[RT * 16][HS] = reinterpret_cast<float(*)[RT * 16][HS]>(smem);
  float(*s_ml)[RT * 16][2] = reinterpret_cast<float(*)[RT * 16][2]>(smem + NW * RT * 16 * HS);
  float *s_bk = smem + MERGE, *s_bvt = s_bk + BMAX * bks<HD>();

  const AttnItem it = a.items[blockIdx.x];   // loaded together with the loop-exit flag
  if (a.done && *a.done) return;
  // A sequence whose block is fully adopted needs no attention.  Its flag is read with a
  // scalar load (nothing in the kernel writes it, and the kernel's start invalidates the
  // scalar cache), whose wait does not hold the vector loads back; the pages' items test
  // it once their first pages are requested.
  const bool with_block = it.is_block == 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int npg = (nkeys + SUB - 1) / SUB;
  const size_t pstride = (size_t)a.Hkv * SUB * HD;   // elements between pages
  const T *Kp = reinterpret_cast<const T *>(a.kc) + ((size_t)it.page0 * a.Hkv + it.kvh) * SUB * HD;
  const T *Vp = reinterpret_cast<const T *>(a.vc) + ((size_t)it.page0 * a.Hkv + it.kvh) * HD * SUB;

  // Block keys/values (fp32, this thread's KPT elements; slots past the block's B keys
  // read key 0, finite and never visible): issued first.
  const float *bbase = a.qkv + (size_t)it.seq * a.B * a.Nqkv;
  float bk[KPT], bv[KPT];
  if (with_block) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = threadIdx.x + NT * i, key = idx / HD, e = idx % HD;
      const int kk = key < a.B ? key : 0;
      bk[i] = bbase[(size_t)kk * a.Nqkv + (size_t)(a.H + it.kvh) * HD + e];
      bv[i] = bbase[(size_t)kk * a.Nqkv + (size_t)(a.H + a.Hkv + it.kvh) * HD + e];
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
    auto tiles = [&](auto fullc) __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        PageMath<T, HD>::template run<decltype(fullc)::value>(
            [&](int h, int c) -> const Frag<T> & { return kf[b][h][c]; },
            [&](int t) -> const Frag<T> & { return vf[b][t]; }, qf[rt], kvalid, g, m_run[rt], l_run[rt], o[rt]);
    };
    // Workgroup-uniform: only a sequence's last page is partial.  (fp32 pages keep the one
    // masked path: two copies of their page code overflow the register file.)
    if (sizeof(T) == 2 && kvalid >= SUB) {
      tiles(std::true_type{});
    } else {
#pragma unroll
      for (int t = 0; t < OT; ++t) mask_v<T>(vf[b][t], g, kvalid);
      tiles(std::false_type{});
    }
  };
  const int pg0 = wave;
  __builtin_amdgcn_sched_barrier(0);   // the block and query loads stay ahead of the pages'
  static_for<DEPTH - 1>([&](auto sc) { fetch(sc, pg0 + decltype(sc)::value * NW); });
  __builtin_amdgcn_sched_barrier(0);
  if (a.seq_done[it.seq]) return;
  q_frags<T, HD, RT>(a, 0, l16, qraw, qf);

  if (with_block) {   // workgroup-uniform
    // The block's keys (rows) and values (transposed) into LDS; wave rt < RT then takes
    // them as the first page of row tile rt, while its prefix pages are in flight.
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = threadIdx.x + NT * i, key = idx / HD, e = idx % HD;
      s_bk[key * bks<HD>() + e] = bk[i];
      s_bvt[e * BVS + key] = bv[i];
    }
    __syncthreads();
    if (wave < RT) {
      const int rho = wave * 16 + l16;
      static_for<RT>([&](auto rc) {   // register arrays indexed by constants only
        constexpr int rt = decltype(rc)::value;
        if (rt == wave)
          block_page<T, HD>(s_bk, s_bvt, qf[rt], a.B, a.causal ? rho % a.B : -1, g, l16, m_run[rt], l_run[rt], o[rt]);
      });
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

  // Merge the waves' states in wave order through LDS (the block's keys are in the states
  // of waves 0 .. RT - 1).
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l_tot = sum_groups(l_run[rt]);
    const int rr = rt * 16 + l16;
    if (g == 0) {
      s_ml[wave][rr][0] = m_run[rt] * LN2;
      s_ml[wave][rr][1] = l_tot;
    }
#pragma unroll
    for (int t = 0; t < OT; ++t) *reinterpret_cast<f32x4_t *>(&s_o[wave][rr][16 * t + 4 * g]) = o[rt][t];
  }
  __syncthreads();
  // Thread `sub` of a row merges the 16-byte pieces at words 4 sub + 64 k: the 16 threads
  // of the row read 256 consecutive bytes per piece.
  constexpr int KC = HD / 64;
  const int sub = threadIdx.x & 15;
  for (int rr = threadIdx.x >> 4; rr < RT * 16 && rr < a.R; rr += 4 * NW) {
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) Mx = fmaxf(Mx, s_ml[w][rr][0]);
    float L = 0.f;
    f32x4_t acc[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) acc[k] = zero4();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_ml[w][rr][0];
      const float f = (mw == -INFINITY) ? 0.f : __expf(mw - Mx);
      L += s_ml[w][rr][1] * f;
#pragma unroll
      for (int k = 0; k < KC; ++k) acc[k] += *reinterpret_cast<const f32x4_t *>(&s_o[w][rr][4 * sub + 64 * k]) * f;
    }
    if (a.single) {   // the pair's only item: the normalised output (the merge's arithmetic for one partial)
      const float inv = 1.0f / L;
      const int orow = it.seq * a.B + rr % a.B, ocol = (it.kvh * a.G + rr / a.B) * HD + 4 * sub;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const f32x4_t v = acc[k] * inv;
        const float vv[4] = {v[0], v[1], v[2], v[3]};
        if (a.o) *reinterpret_cast<f32x4_t *>(a.o + (size_t)orow * a.ldo + ocol + 64 * k) = v;
        if (a.o_afl) afl_put4<T>(a.o_afl, a.H * HD / 32, orow, ocol + 64 * k, vv);
      }
    } else {
      const size_t prow = (size_t)it.slot * a.R + rr;
      if (sub == 0) {
        a.part_ml[prow * 2 + 0] = Mx;
        a.part_ml[prow * 2 + 1] = L;
      }
#pragma unroll
      for (int k = 0; k < KC; ++k) *reinterpret_cast<f32x4_t *>(&a.part_o[prow * HD + 4 * sub + 64 * k]) = acc[k];
    }
  }
}

// Grouped-query shape (R > 32): eight waves (two per SIMD) share each page, wave w
// owning RTW 16-row tiles of the pair's query rows (RTW = 1: 128 rows per workgroup;
// more rows take several workgroups per item).  Pages reach LDS through a ring of
// DEPTH pages held in registers (every thread loads its share of page p + DEPTH while
// page p is multiplied), then stored into the double-buffered LDS stage of PPS = 2
// pages, each MFMA fragment of the page (16 K rows or V^T rows of 32 keys) in lane
// order: thread t of a wave loads the 8-element chunk that lane t reads, so that the
// stores and the reads are contiguous; one barrier per two pages (one per page measured 11% slower, three 10%).  The
// barrier waits for this wave's LDS operations only, not for the ring's page loads still
// in flight (a full fence would wait for those too: 216 -> 204 us per launch at the
// 4 x 65536 grouped-query workload).  Each wave reads a page's K fragments from LDS once
// and reuses them for all of its row tiles; V fragments are read at their use.  (Four
// waves of two row tiles each, one wave per SIMD, measured 281 us; four row tiles per
// wave spill.)  The pair's first item also takes the block's own keys: staged in LDS
// beside the pages' stages, they are every wave's first page (block_page), as in the
// few-row kernel.
template <typename T, int HD, int RTW>
__global__ __launch_bounds__(512) void attn_group_kernel(AttnArgs a) {
  constexpr int NW = 8, NT = 64 * NW, HC = HD / 32, OT = HD / 16;
  constexpr int PPS = 2;                   // pages per LDS stage (measured: 1 and 3 slower)
  constexpr int DEPTH = 2 * PPS;           // pages in flight in registers (two stages)
  constexpr int KCH = SUB * HD / 8;        // 8-element chunks of a K page (= of a V page)
  constexpr int CPT = (KCH + NT - 1) / NT; // chunks of each per thread
  constexpr int FB = frag_words<T>() * 1024;              // bytes of one staged fragment
  constexpr int KBUF = 2 * HC * FB, VBUF = OT * FB;       // bytes of one staged page
  constexpr int BYTES_PAGES = DEPTH * (KBUF + VBUF);      // two stages of PPS pages
  constexpr int BYTES_BLOCK = block_page_lds<HD>() * 4;
  // The block's keys get LDS of their own beside the stages; where both do not fit (fp32
  // pages at head size 128) they share the stages' first bytes and are used up before the
  // first pages are staged.
  constexpr bool SHARE = BYTES_PAGES + BYTES_BLOCK > 160 * 1024;
  constexpr int BYTES = SHARE ? (BYTES_PAGES > BYTES_BLOCK ? BYTES_PAGES : BYTES_BLOCK) : BYTES_PAGES + BYTES_BLOCK;
  constexpr int KPT = BMAX * HD / NT;      // block key / value elements per thread
  __shared__ __attribute__((aligned(16))) char smem[BYTES];
  char *s_k = smem;                              // [stage][page][fragment 2c + h][plane][lane]
  char *s_vt = smem + DEPTH * KBUF;              // [stage][page][fragment t][plane][lane]
  float *s_bk = reinterpret_cast<float *>(smem + (SHARE ? 0 : BYTES_PAGES)), *s_bvt = s_bk + BMAX * bks<HD>();

  // The row groups of an item run on one XCD, launched close together: workgroup b
  // (XCD b % 8 in the round-robin dispatch) takes row group (b / 8) % YS of item
  // 8 ((b / 8) / YS) + b % 8, so the later groups read the item's pages from that XCD's
  // L2.  The grid is rounded up to whole groups of 8 items.
  const int YS = (a.R + NW * RTW * 16 - 1) / (NW * RTW * 16);
  const int xslot = blockIdx.x >> 3;
  const int item = (xslot / YS) * 8 + (blockIdx.x & 7), ygrp = xslot % YS;
  if (item >= a.n_items) return;
  const AttnItem it = a.items[item];   // loaded together with the loop-exit flag
  if (a.done && *a.done) return;
  if (a.seq_done[it.seq]) return;   // block fully adopted: no attention needed
  const bool with_block = it.is_block == 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkeys = it.k_end - it.k_begin;
  const int npg = (nkeys + SUB - 1) / SUB;
  const size_t pstride = (size_t)a.Hkv * SUB * HD;
  const T *Kp = reinterpret_cast<const T *>(a.kc) + ((size_t)it.page0 * a.Hkv + it.kvh) * SUB * HD;
  const T *Vp = reinterpret_cast<const T *>(a.vc) + ((size_t)it.page0 * a.Hkv + it.kvh) * HD * SUB;
  const int rt0 = (ygrp * NW + wave) * RTW;

  float m_run[RTW], l_run[RTW];
  f32x4_t o[RTW][OT];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < OT; ++t) o[rt][t] = zero4();
  }
  // Block keys/values (fp32; slots past the block's B keys read key 0, never visible).
  const float *bbase = a.qkv + (size_t)it.seq * a.B * a.Nqkv;
  float bk[KPT], bv[KPT];
  if (with_block) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = threadIdx.x + NT * i, key = idx / HD, e = idx % HD;
      const int kk = key < a.B ? key : 0;
      bk[i] = bbase[(size_t)kk * a.Nqkv + (size_t)(a.H + it.kvh) * HD + e];
      bv[i] = bbase[(size_t)kk * a.Nqkv + (size_t)(a.H + a.Hkv + it.kvh) * HD + e];
    }
  }
  AFrag<T> qf[RTW][HC];
  load_q<T, HD, RTW>(a, it, rt0, g, l16, qf);
  // The block's keys as each wave's first page (its state is then merged with the
  // pages' in the same running softmax).
  auto block_first = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = threadIdx.x + NT * i, key = idx / HD, e = idx % HD;
      s_bk[key * bks<HD>() + e] = bk[i];
      s_bvt[e * BVS + key] = bv[i];
    }
  };
  auto block_pass = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int rho = (rt0 + rt) * 16 + l16;
      block_page<T, HD>(s_bk, s_bvt, qf[rt], a.B, a.causal ? rho % a.B : -1, g, l16, m_run[rt], l_run[rt], o[rt]);
    }
  };
  if (npg == 0) {   // no prefix pages (yet): the block's keys alone, or the empty state
    if (with_block) {
      block_first();
      __syncthreads();
      block_pass();
    }
    float l_tot[RTW];   // each lane group summed its own keys
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) l_tot[rt] = sum_groups(l_run[rt]);
    store_partial<HD, RTW>(a, it.slot, rt0, g, l16, m_run, l_tot, o);
    return;
  }

  // Register ring: slot r holds this thread's chunks of one page.  Loads are
  // unconditional (pages past the end reread the last page) so that the waits before
  // each store are exact.  Chunk index u = 64 f + lane of this thread (fragment f) takes
  // the page's chunk 64 f + 4 (lane % 16) + lane / 16: K row or V^T row lane % 16 of
  // the fragment, keys or dimensions 8 (lane / 16) .. + 7, the operand of that lane.
  constexpr int W = frag_words<T>();
  u32x4_t kreg[DEPTH][CPT][W], vreg[DEPTH][CPT][W];
  auto chunk_of = [](int u) { return (u & ~63) + 4 * (u & 15) + ((u >> 4) & 3); };
  auto fetch = [&](auto slotc, int pg) __attribute__((always_inline)) {
    constexpr int r = decltype(slotc)::value;
    const size_t base = (size_t)min(pg, npg - 1) * pstride;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = chunk_of(min((int)threadIdx.x + NT * i, KCH - 1));
      const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(Kp + base + (size_t)c * 8);
      const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(Vp + base + (size_t)c * 8);
#pragma unroll
      for (int w = 0; w < W; ++w) {   // plain loads: the item's other row groups re-read them
        kreg[r][i][w] = kp[w];
        vreg[r][i][w] = vp[w];
      }
    }
  };
  auto stash = [&](auto slotc, int buf, int kvalid) __attribute__((always_inline)) {
    constexpr int r = decltype(slotc)::value;
    char *sk = s_k + buf * KBUF;
    char *sv = s_vt + buf * VBUF;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int u = threadIdx.x + NT * i;
      if (u < KCH) {
        const int f = u >> 6, ln = u & 63;
        lds_frag_put(sk + f * FB, ln, frag_of(kreg[r][i], T{}));
        Frag<T> v = frag_of(vreg[r][i], T{});
        mask_v<T>(v, ln >> 4, kvalid);   // keys 8 (ln / 16) .. + 7 of the page
        lds_frag_put(sv + f * FB, ln, v);
      }
    }
  };
  auto compute = [&](int buf, int kvalid) __attribute__((always_inline)) {
    const char *sk = s_k + buf * KBUF;
    const char *sv = s_vt + buf * VBUF;
    Frag<T> kf[2][HC];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < HC; ++c) lds_frag_get(sk + (c * 2 + h) * FB, lane, kf[h][c]);
    // V fragments are read from LDS at their use (once per row tile): holding them too
    // would exceed the 256 registers of a wave at two waves per SIMD.
    auto tiles = [&](auto fullc) __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
        PageMath<T, HD>::template run<decltype(fullc)::value>(
            [&](int h, int c) -> const Frag<T> & { return kf[h][c]; },
            [&](int t) {
              Frag<T> v;
              lds_frag_get(sv + t * FB, lane, v);
              return v;
            },
            qf[rt],
            kvalid, g, m_run[rt], l_run[rt], o[rt]);
    };
    if (sizeof(T) == 2 && kvalid >= SUB)   // workgroup-uniform (fp32: one masked path, as above)
      tiles(std::true_type{});
    else
      tiles(std::false_type{});
  };
  // Barrier over LDS only: this wave's LDS reads and writes are complete (lgkmcnt 0), the
  // ring's global loads may stay in flight.
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
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
    lds_barrier();
  };
  static_for<DEPTH>([&](auto ic) { fetch(ic, decltype(ic)::value); });
  if (with_block) {   // workgroup-uniform
    block_first();
    if constexpr (SHARE) {
      __syncthreads();
      block_pass();
      __syncthreads();
    }
  }
  static_for<PPS>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if (i < npg) stash(ic, i, nkeys - i * SUB);
  });
  lds_barrier();
  if (!SHARE && with_block) block_pass();
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
hipError_t launch_hd(const AttnArgs &a, int part, hipStream_t s) {
  if (!(part & ATTN_SPLIT)) {
  } else if (a.R <= 16) {
    hipLaunchKernelGGL((attn_direct_kernel<T, HD, 1, 4, DIRECT_DEPTH>), dim3(a.n_items), dim3(256), 0, s, a);
  } else if (a.R <= ATTN_FEW_ROWS) {
    hipLaunchKernelGGL((attn_direct_kernel<T, HD, 2, 4, DIRECT_DEPTH>), dim3(a.n_items), dim3(256), 0, s, a);
  } else {   // one 16-row tile per wave, 128 rows per workgroup (more would spill)
    hipLaunchKernelGGL((attn_group_kernel<T, HD, 1>), dim3((a.n_items + 7) / 8 * 8 * ((a.R + 127) / 128)), dim3(512), 0,
                       s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(part & ATTN_MERGE) || a.single) return e;
  hipLaunchKernelGGL((attn_merge_kernel<T, HD>), dim3(a.n_pairs, (a.R + 15) / 16, HD / 32), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnArgs &a, int part, hipStream_t s) {
  if (a.n_items <= 0 || a.n_pairs <= 0 || a.B > BMAX || a.seq_done == nullptr) return hipErrorInvalidValue;
  if (a.single && (a.R > ATTN_FEW_ROWS || a.n_items != a.n_pairs)) return hipErrorInvalidValue;
  if (dtype == DT_BF16) {
    if (a.hd == 128) return launch_hd<bf16_t, 128>(a, part, s);
    if (a.hd == 64) return launch_hd<bf16_t, 64>(a, part, s);
  } else {
    if (a.hd == 128) return launch_hd<float, 128>(a, part, s);
    if (a.hd == 64) return launch_hd<float, 64>(a, part, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace td
