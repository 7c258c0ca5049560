// Host runtime behind td.h: validation, workspace, weight packing, split-K planning,
// and the launch sequence of one denoising step / one block loop on the ctx's stream.
#include "../../include/td.h"
#include "td_internal.h"
#include "td_kernels.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

using namespace td;

namespace {

thread_local std::string g_create_error;

// Projection ids of the profiling tags of TD_PROF_GEMM.
enum { PROJ_QKV = 0, PROJ_OUT = 1, PROJ_UP = 2, PROJ_DOWN = 3, PROJ_ROUTER = 4 };

struct GemmPlan {
  int nt = 1, nw = 4;
  bool tile = false;   // many rows: the tiled MFMA kernel
  int splits = 1;      // tiled kernel: K split (partials summed by a second kernel)
};

}  // namespace

// Per-layer weights of one tower (packed).
struct Layers {
  std::vector<void *> attn_norm, mlp_norm, wqkv, wo, w1, w2;
};

struct td_ctx {
  td_config cfg{};
  int dev = 0;
  hipStream_t stream = nullptr;
  std::string err;
  int elt = 4;

  // weights (ctx-owned, packed)
  void *tok_emb = nullptr, *pos_emb = nullptr, *final_norm = nullptr, *lm_head = nullptr;
  Layers layers;
  // frozen context tower (td_set_context_tower)
  void *ctx_tok_emb = nullptr, *ctx_final_norm = nullptr, *ctx_lm_head = nullptr;
  Layers context;
  uint8_t *ar_committed = nullptr;   // [max_batch] adoption flags of an AR step
  int *zero_flag = nullptr;          // a loop-exit flag that stays 0 (the context pass)
  int *zero_seq = nullptr;           // [max_batch] finished-sequence flags that stay 0
  const int *gemm_done = nullptr;    // flag the layer GEMMs test; nullptr: the step's

  // adoption rule (td_set_commit_rule)
  int rule = RULE_THRESHOLD, min_adopt = 1;

  // mixture-of-experts MLP of the denoiser (td_set_moe)
  bool moe = false;
  td_moe_config moe_cfg{};
  int moe_Epad = 0, moe_max_tiles = 0, moe_cap_rows = 0;
  std::vector<void *> moe_router, moe_w1, moe_w2;   // packed per layer; w1/w2: routed then shared experts
  float *moe_scores = nullptr, *moe_gates = nullptr, *moe_rs = nullptr, *moe_y = nullptr;
  int *moe_experts = nullptr, *moe_slot_pos = nullptr, *moe_src_row = nullptr, *moe_n_tiles = nullptr;
  int4 *moe_tiles = nullptr;
  void *moe_u = nullptr;             // GELU outputs of the sorted rows, fragment layout
  long long *moe_stats = nullptr;    // launches, active experts
  GemmPlan p_router;

  // workspace
  int Mmax = 0, Nqkv = 0;
  float *x = nullptr, *ssq = nullptr, *conf_row = nullptr;
  VStat *vpart = nullptr;
  float *qkv = nullptr;          // q | k | v of the block rows (fp32)
  // GEMM inputs in fragment layout: ah = x * (gain of the next RMSNorm), ao = attention
  // output, au = GELU output of the MLP up projection.
  void *ah = nullptr, *ao = nullptr, *au = nullptr;
  int *arg_row = nullptr;
  int *state_ints = nullptr;    // rowlist | rowpos | act_rows | n_rows, done, t, err, n_act
  StepState st{};
  GemmPlan p_qkv, p_wo, p_w1, p_w2, p_lm;

  // prefix binding
  int n_seqs = 0;
  std::vector<int64_t> lengths, caps;   // tokens and reserved pages of each bound sequence
  int *seq_lp_d = nullptr;              // device [2][max_batch]: lengths, first pages
  std::vector<const void *> kc, vc;
  AttnItem *items_d = nullptr;
  int *pair_first_d = nullptr, *pair_count_d = nullptr;
  // Appending tokens (td_append_block, td_ar_step) extends each pair's last prefix item on
  // the device (grow_idx_d: its index in items_d, or -1 if the pair has none); the host
  // follows the lengths and rebuilds the list only when such an item has grown past
  // twice the chunk size.
  int *grow_idx_d = nullptr;
  std::vector<int> grow_len;            // tokens of each pair's growing item
  std::vector<char> grow_ok;            // the pair has an item that can grow
  int chunk = 0;                        // tokens per split-K item of the binding
  int n_items = 0, n_pairs = 0;
  bool attn_single = false;   // every pair has one attention item (few-row path): no merge launch
  size_t items_cap = 0, pairs_cap = 0;
  float *att_o = nullptr, *att_ml = nullptr;
  float *part = nullptr;     // split-K partial products
  size_t part_cap = 0;       // floats
  size_t part_need = 0;      // floats the bound batch's GEMM plans use
  size_t att_cap_rows = 0;   // capacity in partial rows (items * R)

  // td_generate_block's issue window (td_set_issue_window): steps enqueued beyond the
  // last one the device has reported finished; 0 = the whole loop at once.
  int issue_window = 0;
  unsigned *host_progress = nullptr;   // coherent pinned word written by the commit
  unsigned gen = 0;                    // tag of the current windowed td_generate_block call
  bool progress_armed = false;         // steps enqueued now report progress

  // profiling: event pairs around the launches of the kernel classes in prof_mask, each
  // pair tagged kind | sub << 8 | layer << 16
  unsigned prof_mask = 0;
  int prof_layer = 0;                 // layer of the launches being enqueued
  int prof_only_layer = -1;           // >= 0: per-layer classes bracketed on this layer only
  long prof_open[TD_PROF_KINDS] = {}; // slot of the open bracket of each kind, or -1
  std::vector<hipEvent_t> ev_start, ev_stop;
  std::vector<int32_t> ev_tag;
  size_t prof_n = 0;
};

namespace {

td_status fail(td_ctx *c, td_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  else g_create_error = buf;
  return s;
}

#define TD_HIP(c, expr)                                                                        \
  do {                                                                                         \
    hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess) return fail((c), TD_EDEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

template <typename P>
td_status dmalloc(td_ctx *c, P **p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) bytes = 256;
  hipError_t e = hipMalloc((void **)p, bytes);
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
    return fail(c, TD_ENOMEM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  if (e != hipSuccess) return fail(c, TD_EDEVICE, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  return TD_OK;
}

#define TD_TRY(expr)            \
  do {                          \
    td_status s_ = (expr);      \
    if (s_ != TD_OK) return s_; \
  } while (0)

bool finite(float v) { return std::isfinite(v); }

td_status validate_config(const td_config *cfg) {
  if (!cfg) return fail(nullptr, TD_EINVAL, "cfg is NULL");
  const td_config &c = *cfg;
  if (c.dtype != TD_F32 && c.dtype != TD_BF16) return fail(nullptr, TD_EINVAL, "dtype must be TD_F32 or TD_BF16");
  if (c.n_layers < 1 || c.n_layers > 1024) return fail(nullptr, TD_EINVAL, "n_layers must be in [1, 1024]");
  if (c.d_model < 64 || c.d_model % 64) return fail(nullptr, TD_EINVAL, "d_model must be a positive multiple of 64");
  if (c.d_ff < 64 || c.d_ff % 64) return fail(nullptr, TD_EINVAL, "d_ff must be a positive multiple of 64");
  if (c.vocab < 64 || c.vocab % 64) return fail(nullptr, TD_EINVAL, "vocab must be a positive multiple of 64");
  if (c.head_dim != 64 && c.head_dim != 128) return fail(nullptr, TD_EINVAL, "head_dim must be 64 or 128");
  if (c.n_heads < 1 || c.n_kv_heads < 1 || c.n_heads % c.n_kv_heads)
    return fail(nullptr, TD_EINVAL, "n_heads must be a positive multiple of n_kv_heads");
  if (c.block_size != 1 && c.block_size != 8 && c.block_size != 16 && c.block_size != 32)
    return fail(nullptr, TD_EINVAL, "block_size must be 1, 8, 16 or 32");
  if (c.max_batch < 1 || (int64_t)c.max_batch * c.block_size > (1 << 20))
    return fail(nullptr, TD_EINVAL, "max_batch must be in [1, 2^20 / block_size]");
  if (c.max_prefix_tokens < 0 || c.max_prefix_tokens > ((int64_t)1 << 40))
    return fail(nullptr, TD_EINVAL, "max_prefix_tokens out of range");
  if (!finite(c.rms_eps) || c.rms_eps <= 0.f) return fail(nullptr, TD_EINVAL, "rms_eps must be finite and > 0");
  if ((int64_t)c.n_heads * c.head_dim > (1 << 20)) return fail(nullptr, TD_EINVAL, "n_heads * head_dim too large");
  return TD_OK;
}

td_status validate_weights(const td_config &c, const td_weights *w, bool context = false) {
  if (!w) return fail(nullptr, TD_EINVAL, "weights is NULL");
  if (!w->tok_emb || (!context && (!w->pos_emb || !w->final_norm || !w->lm_head)))
    return fail(nullptr, TD_EINVAL, "a global weight pointer is NULL");
  // The denoiser may leave both MLP arrays NULL: its MLP is then a mixture of experts
  // (td_set_moe); the context tower always has a dense MLP.
  const bool no_mlp = !context && !w->w1 && !w->w2;
  const void *const *lists[] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->mlp_norm, w->w1, w->w2};
  for (int k = 0; k < 8; ++k) {
    const void *const *l = lists[k];
    if (k >= 6 && no_mlp) continue;
    if (!l) return fail(nullptr, TD_EINVAL, "a per-layer weight array is NULL");
    for (int i = 0; i < c.n_layers; ++i)
      if (!l[i]) return fail(nullptr, TD_EINVAL, "per-layer weight pointer %d is NULL", i);
  }
  return TD_OK;
}

// Layer projections (bf16): each activation fragment a wave loads feeds NT
// column tiles, and the L2 -> CU traffic of the activations (2 KiB per k-tile per wave)
// is what bounds these kernels besides the weight stream, so outputs of more than 256
// column tiles take two tiles per workgroup (4 waves along K); narrower outputs keep one
// tile per workgroup (every CU busy) with 16 waves along K (8 with four row tiles, for
// the register file).  Each wave keeps >= 2 k-tiles.
GemmPlan plan_gemm(int M, int N, int K, bool vstat, int dtype) {
  GemmPlan p;
  if (gemm_tile_supported(dtype == TD_BF16 ? DT_BF16 : DT_F32, M, N, K)) {
    p.tile = true;
    p.splits = vstat ? 1 : gemm_tile_splits(M, N, K);
    return p;
  }
  if (vstat) {
    // At most 16 rows of a bf16 tower with d <= 2048: the activations staged in LDS, 16
    // waves x 2 column tiles per workgroup.  Otherwise one row tile: 8 waves x 2 column
    // tiles; four row tiles need more registers per k-tile: 4 waves x 4 column tiles.
    if (M <= 16 && K <= 2048 && N % 512 == 0 && dtype == TD_BF16) {
      p.nw = 16;
      p.nt = 2;
      return p;
    }
    p.nw = M <= 16 && N % 256 == 0 ? 8 : 4;
    p.nt = M <= 16 ? (N % 256 == 0 ? 2 : 1) : (N % 256 == 0 ? 4 : (N % 128 == 0 ? 2 : 1));
  } else {
    const int KT = K / 32, tiles = N / 16;
    const int pairs = tiles / 2;
    if (dtype == TD_BF16 && tiles % 2 == 0 && (pairs > 128 || KT >= 2 * 64)) {
      // Two column tiles per wave, four waves.  Few column pairs over a deep K (the MLP
      // down projection) split K over up to 256 workgroups, at least 64 k-tiles each:
      // each CU then streams a short run of K and re-reads that much of the
      // activations instead of all of it, and a second kernel sums the partials.
      // (Measured: the extra launch costs more than it saves for shallower K.)
      // Two to four row tiles (17-64 rows) re-read the activations once per column
      // tile a wave owns, four times the weight bytes at two tiles: four column tiles
      // per wave over eight waves halve that (measured 15% less GEMM time at 64 rows).
      p.nt = (M > 16 && M <= 64 && tiles % 4 == 0) ? 4 : 2;
      p.nw = p.nt == 4 ? 8 : 4;
      const int groups = tiles / p.nt;
      if (groups <= 128)
        while (groups * p.splits < 256 && KT / (2 * p.splits) >= 64) p.splits *= 2;
    } else {
      p.nt = 1;
      p.nw = tiles <= 256 ? (M <= 16 ? 16 : 8) : 4;
    }
    while (p.nw > 4 && KT / p.nw < 2) p.nw /= 2;
  }
  return p;
}

// Upper bound on the 16-row tiles of the expert-sorted rows of M token rows: the routed
// experts' rows, each nonempty expert padded by at most 15, plus every shared expert's M.
int moe_max_tiles(int M, const td_moe_config &mc) {
  const int64_t mk = (int64_t)M * mc.top_k;
  const int64_t routed = (mk + 15 * std::min<int64_t>(mc.n_experts, mk) + 15) / 16;
  return (int)(routed + (int64_t)mc.n_shared * ((M + 15) / 16));
}

// Prefix keys per split-K item: a multiple of the page size (at least eight pages)
// chosen from the whole batch's prefix keys summed over K/V heads.  Multi-head items
// (memory-bound) aim at about two workgroups per CU: each item's start (its first loads,
// the block's keys) leaves its CU partly idle, while the ragged ends of the pairs still
// spread over the last round (longest first).  Measured against about four per CU:
// attention per block 47.1 -> 45.2 ms at the batch-64 block-32 sweep (two row tiles, one
// workgroup per CU; one item per pair there), 23.1 -> 22.5 ms at block 16, 19.9 ms at
// the ragged batch of 32 either way; six per CU was slower everywhere.  Grouped-query items
// (matrix-core-bound pages, split into row groups of 128 query rows) aim at about one
// workgroup per CU, counting the row groups (measured: more items were slower).
int chunk_keys(int64_t total_pair_keys, int R) {
  const int64_t row_groups = R <= ATTN_FEW_ROWS ? 1 : (R + 127) / 128;
  const int64_t target = R <= ATTN_FEW_ROWS ? 512 : std::max<int64_t>(1, 256 / row_groups);
  int64_t tc = (total_pair_keys + target - 1) / target;
  tc = (tc + KV_PAGE - 1) / KV_PAGE * KV_PAGE;
  return (int)std::min<int64_t>(std::max<int64_t>(tc, 8 * KV_PAGE), (int64_t)1 << 30);
}

constexpr size_t PROF_MAX = 65536;

// Opens (start) or closes the bracket of one launch of class `kind`; sub tells the
// launches of a class apart (the layer projections).
td_status prof_mark(td_ctx *c, int kind, bool start, int sub = 0) {
  if (!(c->prof_mask & (1u << kind))) return TD_OK;
  const bool per_layer = kind == TD_PROF_GEMM || kind == TD_PROF_ATTENTION || kind == TD_PROF_ATTN_MERGE ||
                         kind == TD_PROF_MOE;
  if (per_layer && c->prof_only_layer >= 0 && c->prof_layer != c->prof_only_layer) return TD_OK;
  if (start) {
    c->prof_open[kind] = -1;
    if (c->prof_n >= PROF_MAX) return TD_OK;
    if (c->ev_start.size() <= c->prof_n) {
      // Timing-only events: no system-scope fence, which would write back and invalidate
      // the L2 around every timed launch and slow the next kernel.
      hipEvent_t a, b;
      TD_HIP(c, hipEventCreateWithFlags(&a, hipEventDisableSystemFence));
      TD_HIP(c, hipEventCreateWithFlags(&b, hipEventDisableSystemFence));
      c->ev_start.push_back(a);
      c->ev_stop.push_back(b);
      c->ev_tag.push_back(0);
    }
    TD_HIP(c, hipEventRecord(c->ev_start[c->prof_n], c->stream));
    c->ev_tag[c->prof_n] = kind | (sub << 8) | (c->prof_layer << 16);
    c->prof_open[kind] = (long)c->prof_n++;
  } else {
    const long slot = c->prof_open[kind];
    if (slot < 0) return TD_OK;
    TD_HIP(c, hipEventRecord(c->ev_stop[slot], c->stream));
    c->prof_open[kind] = -1;
  }
  return TD_OK;
}

td_status enqueue_attention(td_ctx *c, int layer, const float *qkv, float *o, void *o_afl, const int *done,
                            bool causal = false) {
  const td_config &g = c->cfg;
  AttnArgs a{};
  a.B = g.block_size;
  a.H = g.n_heads;
  a.Hkv = g.n_kv_heads;
  a.hd = g.head_dim;
  a.Nqkv = c->Nqkv;
  a.G = g.n_heads / g.n_kv_heads;
  a.R = a.G * a.B;
  a.qkv = qkv;
  a.kc = c->kc[layer];
  a.vc = c->vc[layer];
  a.items = c->items_d;
  a.n_items = c->n_items;
  a.pair_first = c->pair_first_d;
  a.pair_count = c->pair_count_d;
  a.n_pairs = c->n_pairs;
  a.part_o = c->att_o;
  a.part_ml = c->att_ml;
  a.o = o;
  a.ldo = g.n_heads * g.head_dim;
  a.o_afl = o_afl;
  a.scale = 1.0f / std::sqrt((float)g.head_dim);
  a.done = done;
  a.causal = causal ? 1 : 0;
  // The denoiser's step skips finished sequences (one sequence: the step's own flag does);
  // other passes skip nothing (flags that stay 0).
  a.seq_done = done && c->n_seqs > 1 ? c->st.seq_done : c->zero_seq;
  a.single = c->attn_single ? 1 : 0;
  TD_TRY(prof_mark(c, TD_PROF_ATTENTION, true));
  TD_HIP(c, launch_attention(g.dtype, a, ATTN_SPLIT, c->stream));
  TD_TRY(prof_mark(c, TD_PROF_ATTENTION, false));
  if (!a.single) {   // pairs of one item normalise their output themselves
    TD_TRY(prof_mark(c, TD_PROF_ATTN_MERGE, true));
    TD_HIP(c, launch_attention(g.dtype, a, ATTN_MERGE, c->stream));
    TD_TRY(prof_mark(c, TD_PROF_ATTN_MERGE, false));
  }
  return TD_OK;
}

// One weight-streaming GEMM.  A: fragment-layout input; norm: A holds x * gain of an
// RMSNorm whose row scale comes from the partial sums of squares in c->ssq.
td_status enqueue_gemm(td_ctx *c, int epi, bool norm, int M, int N, int K, const void *A, const void *Wp,
                       const GemmPlan &p, float *out, void *out_afl, const void *gain_next,
                       const GemmArgs *extra = nullptr, int prof_sub = 0) {
  GemmArgs a{};
  if (extra) a = *extra;
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  if (norm) {
    a.ssq = c->ssq;
    a.norm_nparts = c->cfg.d_model / 16;
    a.ld_ssq = M;
    a.norm_eps = c->cfg.rms_eps;
  }
  a.Wp = Wp;
  a.nt = p.nt;
  a.nw = p.nw;
  a.out = out;
  a.ldo = N;
  a.out_afl = out_afl;
  a.gain_next = gain_next;
  a.ssq_out = c->ssq;
  a.done = c->gemm_done ? c->gemm_done : c->st.done;
  a.splits = epi == EPI_VSTAT ? 1 : p.splits;
  a.part = c->part;
  a.part_cap = c->part_need;
  // A denoising step over several sequences computes only the rows of the sequences that
  // still have a masked position (a finished sequence's rows are never read again); the
  // context pass (its own loop-exit flag) computes every row.  A projection already split
  // in K (the MLP down projection) grows its split on the device once those rows get few:
  // its reduction is launched anyway.  (Growing the others too needs a reduction launch
  // after each of them in every step; at the batch-64 block-32 sweep those launches, idle
  // at full batch, cost 2.3 ms per block, about what their late steps saved.)
  if (p.tile && epi != EPI_VSTAT && !c->gemm_done && c->n_seqs > 1 && !a.rowlist) {
    a.rowlist = c->st.act_rows;
    a.n_rows = c->st.n_act;
    a.dyn = p.splits > 1 ? 1 : 0;
  }
  if (p.tile) {
    if (epi != EPI_VSTAT) TD_TRY(prof_mark(c, TD_PROF_GEMM, true, prof_sub));
    TD_HIP(c, launch_gemm_tile(epi, norm, a, c->stream));
    if (epi != EPI_VSTAT) TD_TRY(prof_mark(c, TD_PROF_GEMM, false));
  } else if (epi == EPI_VSTAT) {
    TD_HIP(c, launch_gemm(c->cfg.dtype, epi, norm, a, c->stream));
  } else {
    TD_TRY(prof_mark(c, TD_PROF_GEMM, true, prof_sub));
    TD_HIP(c, launch_gemm_wk(c->cfg.dtype, epi, norm, a, c->stream));
    TD_TRY(prof_mark(c, TD_PROF_GEMM, false));
  }
  return TD_OK;
}

td_status enqueue_head_commit(td_ctx *c, const void *head, int *tokens, uint8_t *committed, const float *inv_temp,
                              float gamma, int rule, int min_adopt, uint8_t *newly, float *conf_out, int *argmax_out,
                              float *logits, int *steps, int8_t *commit_step);

// The mixture-of-experts MLP of layer l over M rows: router scores (a weight-streaming
// GEMM over the normed input c->ah with its row scale), routing and the expert-sorted
// tile table, the expert up and down projections, then the gated sum into the residual
// stream, which leaves x, its partial sums of squares and x * gain_after in fragment
// layout exactly as the dense MLP's down projection does.
td_status enqueue_moe(td_ctx *c, int l, int M, const void *gain_after) {
  const td_config &g = c->cfg;
  const td_moe_config &mc = c->moe_cfg;
  const int d = g.d_model;
  TD_TRY(enqueue_gemm(c, EPI_STORE, true, M, c->moe_Epad, d, c->ah, c->moe_router[l], c->p_router, c->moe_scores,
                      nullptr, nullptr, nullptr, PROJ_ROUTER));
  MoeRoute r{};
  r.M = M;
  r.E = mc.n_experts;
  r.Epad = c->moe_Epad;
  r.top_k = mc.top_k;
  r.n_shared = mc.n_shared;
  r.d = d;
  r.scores = c->moe_scores;
  r.ssq = c->ssq;
  r.eps = g.rms_eps;
  r.experts = c->moe_experts;
  r.gates = c->moe_gates;
  r.rs = c->moe_rs;
  r.slot_pos = c->moe_slot_pos;
  r.src_row = c->moe_src_row;
  r.tiles = c->moe_tiles;
  r.n_tiles = c->moe_n_tiles;
  r.stats = c->moe_stats;
  // Rows of finished sequences are skipped with more than one sequence bound (one
  // sequence: the step's own flag ends the loop).
  r.seq_done = c->n_seqs > 1 ? c->st.seq_done : c->zero_seq;
  r.B = g.block_size;
  r.done = c->st.done;
  TD_HIP(c, launch_moe_route(r, c->stream));
  const int NE = mc.n_experts + mc.n_shared;
  const int tiles = moe_max_tiles(M, mc);
  MoeGemm up{};
  up.N = mc.d_expert;
  up.K = d;
  up.A = c->ah;
  up.src_row = c->moe_src_row;
  up.rs = c->moe_rs;
  up.Wp = c->moe_w1[l];
  up.tiles = c->moe_tiles;
  up.n_tiles = c->moe_n_tiles;
  up.max_tiles = tiles;
  up.out_afl = c->moe_u;
  up.done = c->st.done;
  MoeGemm dn = up;
  dn.N = d;
  dn.K = mc.d_expert;
  dn.A = c->moe_u;
  dn.src_row = nullptr;
  dn.rs = nullptr;
  dn.Wp = c->moe_w2[l];
  dn.out_afl = nullptr;
  dn.out = c->moe_y;
  (void)NE;
  TD_TRY(prof_mark(c, TD_PROF_MOE, true, 0));
  TD_HIP(c, launch_moe_gemm(g.dtype, true, up, c->stream));
  TD_TRY(prof_mark(c, TD_PROF_MOE, false));
  TD_TRY(prof_mark(c, TD_PROF_MOE, true, 1));
  TD_HIP(c, launch_moe_gemm(g.dtype, false, dn, c->stream));
  TD_TRY(prof_mark(c, TD_PROF_MOE, false));
  MoeCombine cb{};
  cb.M = M;
  cb.d = d;
  cb.top_k = mc.top_k;
  cb.n_shared = mc.n_shared;
  cb.slot_pos = c->moe_slot_pos;
  cb.gates = c->moe_gates;
  cb.y = c->moe_y;
  cb.x = c->x;
  cb.out_afl = c->ah;
  cb.gain_next = gain_after;
  cb.ssq_out = c->ssq;
  cb.seq_done = r.seq_done;
  cb.B = g.block_size;
  cb.done = c->st.done;
  TD_HIP(c, launch_moe_combine(g.dtype, cb, c->stream));
  return TD_OK;
}

td_status enqueue_step(td_ctx *c, int *tokens, uint8_t *committed, const float *inv_temp, float gamma,
                       uint8_t *newly, float *conf_out, int *argmax_out, float *logits, int *steps,
                       int8_t *commit_step) {
  const td_config &g = c->cfg;
  const int M = c->n_seqs * g.block_size;
  const int d = g.d_model, Hd = g.n_heads * g.head_dim;
  TD_TRY(prof_mark(c, TD_PROF_STEP, true));
  c->prof_layer = 0;
  TD_TRY(prof_mark(c, TD_PROF_EMBED, true));
  TD_HIP(c, launch_embed(g.dtype, tokens, c->tok_emb, c->pos_emb, c->layers.attn_norm[0], c->x, c->ssq, c->ah, M,
                         g.block_size, d, g.vocab, c->st, c->stream));
  TD_TRY(prof_mark(c, TD_PROF_EMBED, false));
  for (int l = 0; l < g.n_layers; ++l) {
    c->prof_layer = l;
    const void *gain_after = l + 1 < g.n_layers ? c->layers.attn_norm[l + 1] : c->final_norm;
    TD_TRY(enqueue_gemm(c, EPI_STORE, true, M, c->Nqkv, d, c->ah, c->layers.wqkv[l], c->p_qkv, c->qkv, nullptr, nullptr,
                        nullptr, PROJ_QKV));
    TD_TRY(enqueue_attention(c, l, c->qkv, nullptr, c->ao, c->st.done));
    TD_TRY(enqueue_gemm(c, EPI_RESID, false, M, d, Hd, c->ao, c->layers.wo[l], c->p_wo, c->x, c->ah, c->layers.mlp_norm[l],
                        nullptr, PROJ_OUT));
    if (c->moe) {
      TD_TRY(enqueue_moe(c, l, M, gain_after));
    } else {
      TD_TRY(enqueue_gemm(c, EPI_GELU, true, M, g.d_ff, d, c->ah, c->layers.w1[l], c->p_w1, nullptr, c->au, nullptr,
                          nullptr, PROJ_UP));
      TD_TRY(enqueue_gemm(c, EPI_RESID, false, M, d, g.d_ff, c->au, c->layers.w2[l], c->p_w2, c->x, c->ah, gain_after,
                          nullptr, PROJ_DOWN));
    }
  }
  c->prof_layer = 0;
  TD_TRY(enqueue_head_commit(c, c->lm_head, tokens, committed, inv_temp, gamma, c->rule, c->min_adopt, newly, conf_out,
                             argmax_out, logits, steps, commit_step));
  TD_TRY(prof_mark(c, TD_PROF_STEP, false));
  return TD_OK;
}

// The LM head (head: packed [vocab][d]) with the fused vocabulary statistics over the rows
// still masked, then the merge and the adoption rule.  The head's input is c->ah, the
// last residual update's x * final gain, with its sums of squares in c->ssq.
td_status enqueue_head_commit(td_ctx *c, const void *head, int *tokens, uint8_t *committed, const float *inv_temp,
                              float gamma, int rule, int min_adopt, uint8_t *newly, float *conf_out, int *argmax_out,
                              float *logits, int *steps, int8_t *commit_step) {
  const td_config &g = c->cfg;
  const int M = c->n_seqs * g.block_size;
  const int d = g.d_model;
  GemmArgs lm{};
  lm.rowlist = c->st.rowlist;
  lm.rowpos = c->st.rowpos;
  lm.n_rows = c->st.n_rows;
  lm.inv_temp = inv_temp;
  lm.vpart = c->vpart;
  lm.logits = logits;
  TD_TRY(prof_mark(c, TD_PROF_LMHEAD, true));
  TD_TRY(enqueue_gemm(c, EPI_VSTAT, true, M, g.vocab, d, c->ah, head, c->p_lm, nullptr, nullptr, nullptr, &lm));
  TD_TRY(prof_mark(c, TD_PROF_LMHEAD, false));
  CommitArgs ca{};
  ca.V = g.vocab;
  ca.B = g.block_size;
  ca.n = c->n_seqs;
  ca.nslices = c->p_lm.tile ? gemm_tile_slices(g.vocab) : lmhead_slices(g.vocab, c->p_lm.nt, c->p_lm.nw);
  ca.vpart = c->vpart;
  ca.conf_row = c->conf_row;
  ca.arg_row = c->arg_row;
  ca.tokens = tokens;
  ca.committed = committed;
  ca.gamma = gamma;
  ca.rule = rule;
  ca.min_adopt = min_adopt;
  ca.newly = newly;
  ca.conf_out = conf_out;
  ca.argmax_out = argmax_out;
  ca.steps = steps;
  ca.commit_step = commit_step;
  ca.st = c->st;
  ca.host_progress = c->progress_armed ? c->host_progress : nullptr;
  ca.gen = c->gen;
  TD_TRY(prof_mark(c, TD_PROF_COMMIT, true));
  TD_HIP(c, launch_merge_commit(ca, M, c->stream));
  TD_TRY(prof_mark(c, TD_PROF_COMMIT, false));
  return TD_OK;
}

// The frozen context tower over the bound batch's block tokens (committed ids): embedding
// without a position table, then per layer the fused QKV projection, attention that is
// causal inside the block and sees the whole cached prefix, the append of this layer's
// K/V to its cache at each sequence's current length, and the residual MLP.  The last
// layer stops after its K/V, unless `full` (AR decoding): then it completes and leaves
// x * final gain in c->ah for the head.  The layer GEMMs test a flag that stays 0 (the
// step's flag says the block is done).
td_status enqueue_context_pass(td_ctx *c, const int32_t *tokens, bool full = false) {
  const td_config &g = c->cfg;
  const int M = c->n_seqs * g.block_size;
  const int d = g.d_model, Hd = g.n_heads * g.head_dim;
  StepState st = c->st;
  st.done = c->zero_flag;
  TD_HIP(c, launch_embed(g.dtype, tokens, c->ctx_tok_emb, nullptr, c->context.attn_norm[0], c->x, c->ssq, c->ah, M,
                         g.block_size, d, g.vocab, st, c->stream));
  c->gemm_done = c->zero_flag;
  td_status s = TD_OK;
  for (int l = 0; l < g.n_layers && s == TD_OK; ++l) {
    s = enqueue_gemm(c, EPI_STORE, true, M, c->Nqkv, d, c->ah, c->context.wqkv[l], c->p_qkv, c->qkv, nullptr,
                     nullptr);
    const bool last = l + 1 == g.n_layers && !full;   // full: through the last layer (AR decoding)
    if (s == TD_OK && !last) s = enqueue_attention(c, l, c->qkv, nullptr, c->ao, nullptr, true);
    if (s == TD_OK) {
      const hipError_t e = launch_kv_append(g.dtype, c->qkv, c->Nqkv, g.n_heads, g.n_kv_heads, g.head_dim,
                                            const_cast<void *>(c->kc[l]), const_cast<void *>(c->vc[l]), c->seq_lp_d,
                                            c->seq_lp_d + c->n_seqs, c->n_seqs, g.block_size, c->stream);
      if (e != hipSuccess) s = fail(c, TD_EDEVICE, "K/V append launch failed: %s", hipGetErrorString(e));
    }
    if (s == TD_OK && !last) {
      s = enqueue_gemm(c, EPI_RESID, false, M, d, Hd, c->ao, c->context.wo[l], c->p_wo, c->x, c->ah,
                       c->context.mlp_norm[l]);
      if (s == TD_OK)
        s = enqueue_gemm(c, EPI_GELU, true, M, g.d_ff, d, c->ah, c->context.w1[l], c->p_w1, nullptr, c->au, nullptr);
      if (s == TD_OK)
        s = enqueue_gemm(c, EPI_RESID, false, M, d, g.d_ff, c->au, c->context.w2[l], c->p_w2, c->x, c->ah,
                         l + 1 < g.n_layers ? c->context.attn_norm[l + 1] : c->ctx_final_norm);
    }
  }
  c->gemm_done = nullptr;
  return s;
}

td_status check_ctx(td_ctx *c) {
  if (!c) return fail(nullptr, TD_EINVAL, "ctx is NULL");
  return TD_OK;
}

td_status check_mlp(td_ctx *c) {
  if (!c->moe && (c->layers.w1.empty() || !c->layers.w1[0]))
    return fail(c, TD_EINVAL, "the denoiser has no MLP weights: pass w1/w2 to td_create or call td_set_moe");
  return TD_OK;
}

td_status check_bound(td_ctx *c) {
  if (c->n_seqs <= 0) return fail(c, TD_EINVAL, "no prefix bound: call td_set_prefix first");
  TD_HIP(c, hipSetDevice(c->dev));
  return TD_OK;
}

void free_moe(td_ctx *c) {
  auto f = [](void *p) {
    if (p) (void)hipFree(p);
  };
  for (auto *v : {&c->moe_router, &c->moe_w1, &c->moe_w2}) {
    for (void *p : *v) f(p);
    v->clear();
  }
  f(c->moe_scores); f(c->moe_gates); f(c->moe_rs); f(c->moe_y); f(c->moe_experts); f(c->moe_slot_pos);
  f(c->moe_src_row); f(c->moe_n_tiles); f(c->moe_tiles); f(c->moe_u); f(c->moe_stats);
  c->moe_scores = c->moe_gates = c->moe_rs = c->moe_y = nullptr;
  c->moe_experts = c->moe_slot_pos = c->moe_src_row = c->moe_n_tiles = nullptr;
  c->moe_tiles = nullptr;
  c->moe_u = nullptr;
  c->moe_stats = nullptr;
  c->moe = false;
}

void free_all(td_ctx *c) {
  auto f = [](void *p) {
    if (p) (void)hipFree(p);
  };
  f(c->tok_emb); f(c->pos_emb); f(c->final_norm); f(c->lm_head);
  for (Layers *t : {&c->layers, &c->context})
    for (auto *v : {&t->attn_norm, &t->mlp_norm, &t->wqkv, &t->wo, &t->w1, &t->w2})
      for (void *p : *v) f(p);
  f(c->ctx_tok_emb); f(c->ctx_final_norm); f(c->ctx_lm_head); f(c->ar_committed); f(c->st.seq_done); f(c->zero_seq); f(c->zero_flag); f(c->seq_lp_d);
  f(c->x); f(c->ssq); f(c->conf_row); f(c->vpart); f(c->qkv); f(c->ah); f(c->ao); f(c->au);
  f(c->arg_row); f(c->state_ints); f(c->items_d); f(c->pair_first_d);
  f(c->pair_count_d); f(c->grow_idx_d); f(c->att_o); f(c->att_ml); f(c->part);
  free_moe(c);
  for (hipEvent_t e : c->ev_start) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->ev_stop) (void)hipEventDestroy(e);
  if (c->host_progress) (void)hipHostFree(c->host_progress);
  c->host_progress = nullptr;
}

// Per-layer weights of a tower, packed into MFMA tiles (W_q, W_k, W_v fused).
td_status pack_layers(td_ctx *c, const td_weights &w, Layers &t) {
  const td_config &g = c->cfg;
  const size_t e = c->elt, d = g.d_model, F = g.d_ff, L = g.n_layers;
  const size_t Hd = (size_t)g.n_heads * g.head_dim, KVd = (size_t)g.n_kv_heads * g.head_dim;
  t.attn_norm.assign(L, nullptr); t.mlp_norm.assign(L, nullptr); t.wqkv.assign(L, nullptr);
  t.wo.assign(L, nullptr); t.w1.assign(L, nullptr); t.w2.assign(L, nullptr);
  for (size_t l = 0; l < L; ++l) {
    TD_TRY(dmalloc(c, &t.attn_norm[l], d * e));
    TD_TRY(dmalloc(c, &t.mlp_norm[l], d * e));
    TD_TRY(dmalloc(c, &t.wqkv[l], (size_t)c->Nqkv * d * e));
    TD_TRY(dmalloc(c, &t.wo[l], d * Hd * e));
    if (w.w1) {
      TD_TRY(dmalloc(c, &t.w1[l], F * d * e));
      TD_TRY(dmalloc(c, &t.w2[l], d * F * e));
    }
    TD_HIP(c, hipMemcpyAsync(t.attn_norm[l], w.attn_norm[l], d * e, hipMemcpyDeviceToDevice, c->stream));
    TD_HIP(c, hipMemcpyAsync(t.mlp_norm[l], w.mlp_norm[l], d * e, hipMemcpyDeviceToDevice, c->stream));
    char *qkv = (char *)t.wqkv[l];
    TD_HIP(c, launch_pack_weight(g.dtype, w.wq[l], qkv, (int)Hd, (int)d, c->stream));
    TD_HIP(c, launch_pack_weight(g.dtype, w.wk[l], qkv + Hd * d * e, (int)KVd, (int)d, c->stream));
    TD_HIP(c, launch_pack_weight(g.dtype, w.wv[l], qkv + (Hd + KVd) * d * e, (int)KVd, (int)d, c->stream));
    TD_HIP(c, launch_pack_weight(g.dtype, w.wo[l], t.wo[l], (int)d, (int)Hd, c->stream));
    if (w.w1) {
      TD_HIP(c, launch_pack_weight(g.dtype, w.w1[l], t.w1[l], (int)F, (int)d, c->stream));
      TD_HIP(c, launch_pack_weight(g.dtype, w.w2[l], t.w2[l], (int)d, (int)F, c->stream));
    }
  }
  return TD_OK;
}

td_status create_impl(td_ctx *c, const td_config &g, const td_weights &w) {
  TD_HIP(c, hipGetDevice(&c->dev));
  TD_HIP(c, td::noalloc_scratch_init());   // the allocation-free step's array on this device
  c->elt = g.dtype == TD_BF16 ? 2 : 4;
  const size_t e = c->elt;
  const size_t d = g.d_model, F = g.d_ff, V = g.vocab;
  const size_t Hd = (size_t)g.n_heads * g.head_dim, KVd = (size_t)g.n_kv_heads * g.head_dim;
  c->Nqkv = (int)(Hd + 2 * KVd);
  c->Mmax = g.max_batch * g.block_size;
  const size_t M = c->Mmax;

  // Packed weights.
  TD_TRY(dmalloc(c, &c->tok_emb, (V + 1) * d * e));
  TD_TRY(dmalloc(c, &c->pos_emb, (size_t)g.block_size * d * e));
  TD_TRY(dmalloc(c, &c->final_norm, d * e));
  TD_TRY(dmalloc(c, &c->lm_head, V * d * e));
  TD_HIP(c, hipMemcpyAsync(c->tok_emb, w.tok_emb, (V + 1) * d * e, hipMemcpyDeviceToDevice, c->stream));
  TD_HIP(c, hipMemcpyAsync(c->pos_emb, w.pos_emb, (size_t)g.block_size * d * e, hipMemcpyDeviceToDevice, c->stream));
  TD_HIP(c, hipMemcpyAsync(c->final_norm, w.final_norm, d * e, hipMemcpyDeviceToDevice, c->stream));
  TD_HIP(c, launch_pack_weight(g.dtype, w.lm_head, c->lm_head, (int)V, (int)d, c->stream));
  TD_TRY(pack_layers(c, w, c->layers));

  // Workspace sized for max_batch.
  TD_TRY(dmalloc(c, &c->x, M * d * 4));
  TD_TRY(dmalloc(c, &c->ssq, (d / 16) * M * 4));
  TD_TRY(dmalloc(c, &c->qkv, M * c->Nqkv * 4));
  TD_TRY(dmalloc(c, &c->ah, afl_bytes((int)M, (int)d)));
  TD_TRY(dmalloc(c, &c->ao, afl_bytes((int)M, (int)Hd)));
  TD_TRY(dmalloc(c, &c->au, afl_bytes((int)M, (int)F)));
  // Rows past the live count are read as padding by the GEMMs: keep them finite.
  TD_HIP(c, hipMemsetAsync(c->ah, 0, afl_bytes((int)M, (int)d), c->stream));
  TD_HIP(c, hipMemsetAsync(c->ao, 0, afl_bytes((int)M, (int)Hd), c->stream));
  TD_HIP(c, hipMemsetAsync(c->au, 0, afl_bytes((int)M, (int)F), c->stream));
  TD_TRY(dmalloc(c, &c->conf_row, M * 4));
  TD_TRY(dmalloc(c, &c->arg_row, M * 4));
  TD_TRY(dmalloc(c, &c->vpart, M * (V / 16) * sizeof(VStat)));   // up to one group per 16 columns
  TD_TRY(dmalloc(c, &c->seq_lp_d, 2 * (size_t)g.max_batch * sizeof(int)));
  TD_TRY(dmalloc(c, &c->ar_committed, M));
  TD_TRY(dmalloc(c, &c->st.seq_done, g.max_batch * sizeof(int)));
  TD_HIP(c, hipMemsetAsync(c->st.seq_done, 0, g.max_batch * sizeof(int), c->stream));
  TD_TRY(dmalloc(c, &c->zero_seq, g.max_batch * sizeof(int)));
  TD_HIP(c, hipMemsetAsync(c->zero_seq, 0, g.max_batch * sizeof(int), c->stream));
  TD_TRY(dmalloc(c, &c->zero_flag, sizeof(int)));
  TD_HIP(c, hipMemsetAsync(c->zero_flag, 0, sizeof(int), c->stream));
  TD_TRY(dmalloc(c, &c->state_ints, (3 * M + 8) * sizeof(int)));
  TD_HIP(c, hipMemsetAsync(c->state_ints, 0, (3 * M + 8) * sizeof(int), c->stream));
  int *si = c->state_ints;
  c->st.rowlist = si;
  c->st.rowpos = si + M;
  c->st.act_rows = si + 2 * M;
  c->st.n_rows = si + 3 * M;
  c->st.done = si + 3 * M + 1;
  c->st.t = si + 3 * M + 2;
  c->st.err = si + 3 * M + 3;
  c->st.n_act = si + 3 * M + 4;
  TD_HIP(c, hipStreamSynchronize(c->stream));
  return TD_OK;
}

}  // namespace

// ---------------------------------------------------------------- steps on caller-side scratch

namespace td {

// The partial-result buffers of one step over the bound batch, carved from `base`
// (256-byte aligned pieces): the vocabulary statistics of every (row, column group), the
// per-row confidences and predictions, the attention items' partial states and the
// K-split partial products.  Returns the bytes needed; fills *out only when they fit.
int ctx_device(const td_ctx *c) { return c->dev; }

size_t carve_step_scratch(const td_ctx *c, char *base, size_t bytes, StepScratch *out) {
  const td_config &g = c->cfg;
  const size_t M = (size_t)c->n_seqs * g.block_size;
  const size_t nslices = c->p_lm.tile ? gemm_tile_slices(g.vocab) : lmhead_slices(g.vocab, c->p_lm.nt, c->p_lm.nw);
  const size_t R = (size_t)(g.n_heads / g.n_kv_heads) * g.block_size;
  const size_t rows = (size_t)c->n_items * R;
  const size_t sizes[6] = {M * nslices * sizeof(VStat), M * 4, M * 4, rows * g.head_dim * 4, rows * 8,
                           c->part_need * 4};
  size_t off[6], total = 0;
  for (int i = 0; i < 6; ++i) {
    off[i] = total;
    total += (sizes[i] + 255) / 256 * 256;
  }
  if (out && base && total <= bytes) {
    out->vpart = reinterpret_cast<VStat *>(base + off[0]);
    out->conf_row = reinterpret_cast<float *>(base + off[1]);
    out->arg_row = reinterpret_cast<int *>(base + off[2]);
    out->att_o = reinterpret_cast<float *>(base + off[3]);
    out->att_ml = reinterpret_cast<float *>(base + off[4]);
    out->part = sizes[5] ? reinterpret_cast<float *>(base + off[5]) : nullptr;
  }
  return total;
}

// td_denoise_step with the step's partial results in caller-side device scratch
// [scratch, scratch + bytes) instead of the ctx's own buffers.  Nothing is allocated:
// profiling brackets (whose events are created on first use) are not recorded.
td_status denoise_step_on_scratch(td_ctx *c, int32_t *tokens, uint8_t *committed, const float *inv_temp, float gamma,
                                  uint8_t *newly, float *conf_out, int32_t *argmax_out, float *logits_out,
                                  char *scratch, size_t bytes) {
  TD_TRY(check_ctx(c));
  TD_TRY(check_mlp(c));
  if (!tokens || !committed) return fail(c, TD_EINVAL, "tokens and committed must not be NULL");
  if (!finite(gamma)) return fail(c, TD_EINVAL, "gamma must be finite");
  if (c->n_seqs <= 0) return fail(c, TD_EINVAL, "no prefix bound: call td_set_prefix first");
  StepScratch sc{};
  const size_t need = carve_step_scratch(c, scratch, bytes, &sc);
  if (!scratch || need > bytes)
    return fail(c, TD_EINVAL, "the bound batch needs %zu bytes of step scratch; the allocation-free step holds %zu",
                need, bytes);
  TD_TRY(check_bound(c));
  const StepScratch own{c->vpart, c->conf_row, c->arg_row, c->att_o, c->att_ml, c->part};
  const unsigned mask = c->prof_mask;
  c->prof_mask = 0;
  c->vpart = sc.vpart;
  c->conf_row = sc.conf_row;
  c->arg_row = sc.arg_row;
  c->att_o = sc.att_o;
  c->att_ml = sc.att_ml;
  c->part = sc.part;
  const int M = c->n_seqs * c->cfg.block_size;
  td_status st = TD_OK;
  const hipError_t e = launch_prep(tokens, committed, M, c->cfg.block_size, c->cfg.vocab, c->st, c->stream);
  if (e != hipSuccess) st = fail(c, TD_EDEVICE, "launch_prep: %s", hipGetErrorString(e));
  if (st == TD_OK)
    st = enqueue_step(c, tokens, committed, inv_temp, gamma, newly, conf_out, argmax_out, logits_out, nullptr, nullptr);
  c->vpart = own.vpart;
  c->conf_row = own.conf_row;
  c->arg_row = own.arg_row;
  c->att_o = own.att_o;
  c->att_ml = own.att_ml;
  c->part = own.part;
  c->prof_mask = mask;
  return st;
}

}  // namespace td

extern "C" {

td_status td_create(const td_config *cfg, const td_weights *w, void *stream, td_ctx **out) {
  g_create_error.clear();
  if (!out) return fail(nullptr, TD_EINVAL, "out is NULL");
  *out = nullptr;
  TD_TRY(validate_config(cfg));
  TD_TRY(validate_weights(*cfg, w));
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev <= 0)
    return fail(nullptr, TD_EDEVICE, "no HIP device available (%s)", hipGetErrorString(e));
  td_ctx *c = new (std::nothrow) td_ctx();
  if (!c) return fail(nullptr, TD_ENOMEM, "host allocation failed");
  c->cfg = *cfg;
  c->stream = (hipStream_t)stream;
  td_status s = create_impl(c, *cfg, *w);
  if (s != TD_OK) {
    g_create_error = c->err;
    (void)hipStreamSynchronize(c->stream);
    free_all(c);
    delete c;
    return s;
  }
  *out = c;
  return TD_OK;
}

// Binds caches whose sequence i holds len[i] tokens in cap[i] reserved pages, the pages
// of sequence i starting after those of sequences 0..i-1.
static td_status bind_impl(td_ctx *c, int32_t n_seqs, const int64_t *len, const int64_t *cap,
                    const void *const *k_cache_host, const void *const *v_cache_host) {
  const td_config &g = c->cfg;
  int64_t total = 0, pages = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (len[i] < 0 || len[i] > (int64_t)1 << 30) return fail(c, TD_EINVAL, "length of sequence %d out of range", i);
    if (cap[i] < (len[i] + KV_PAGE - 1) / KV_PAGE)
      return fail(c, TD_EINVAL, "sequence %d: %lld tokens do not fit %lld pages", i, (long long)len[i],
                  (long long)cap[i]);
    total += len[i];
    pages += cap[i];
  }
  if (total > g.max_prefix_tokens)
    return fail(c, TD_ENOMEM, "sum of prefix lengths %lld exceeds max_prefix_tokens %lld", (long long)total,
                (long long)g.max_prefix_tokens);
  if (pages > ((int64_t)1 << 31) - 1) return fail(c, TD_EINVAL, "too many cache pages");
  for (int l = 0; l < g.n_layers; ++l)
    if (pages > 0 && (!k_cache_host[l] || !v_cache_host[l]))
      return fail(c, TD_EINVAL, "cache pointer of layer %d is NULL", l);
  TD_HIP(c, hipSetDevice(c->dev));
  TD_HIP(c, hipStreamSynchronize(c->stream));   // previous work may still read the old binding

  std::vector<int64_t> off(n_seqs + 1, 0);
  for (int i = 0; i < n_seqs; ++i) off[i + 1] = off[i] + len[i];
  const int G = g.n_heads / g.n_kv_heads, R = G * g.block_size;
  const int tc = chunk_keys(off[n_seqs] * g.n_kv_heads, R);
  // The pair's first item also takes the block's keys (no item of its own, so the item
  // count is the prefix pages' alone: a block-only item made a second round of
  // workgroups at batch 1).
  std::vector<AttnItem> items;
  std::vector<int> pfirst, pcount, grow_slot;
  std::vector<int> grow_len;
  int64_t page_base = 0;   // first cache page of sequence i
  for (int i = 0; i < n_seqs; ++i) {
    const int64_t P = off[i + 1] - off[i];
    for (int h = 0; h < g.n_kv_heads; ++h) {
      pfirst.push_back((int)items.size());
      // A pair with no prefix gets one item of no pages, which appended tokens extend.
      if (P == 0) items.push_back(AttnItem{i, h, 0, 0, 2, 0, page_base});
      for (int64_t k0 = 0; k0 < P; k0 += tc)
        items.push_back(AttnItem{i, h, (int)k0, (int)std::min<int64_t>(P, k0 + tc), k0 == 0 ? 2 : 0, 0,
                                 page_base + k0 / KV_PAGE});
      const bool has_prefix_item = (int)items.size() > pfirst.back();
      grow_slot.push_back(has_prefix_item ? (int)items.size() - 1 : -1);
      grow_len.push_back(has_prefix_item ? items.back().k_end - items.back().k_begin : 0);
      pcount.push_back((int)items.size() - pfirst.back());
    }
    page_base += cap[i];
  }
  if (items.size() > ((size_t)1 << 28)) return fail(c, TD_EINVAL, "too many attention work items");
  // Slots in pair order (the merge reads them so); launch order longest first, ties in
  // slot order: workgroups start roughly in launch order, so the short ragged ends of
  // the pairs fill the last wave instead of trailing it (largest-first list scheduling).
  for (size_t k = 0; k < items.size(); ++k) items[k].slot = (int)k;
  std::stable_sort(items.begin(), items.end(), [](const AttnItem &x, const AttnItem &y) {
    return x.k_end - x.k_begin > y.k_end - y.k_begin;
  });
  std::vector<int> at_slot(items.size()), grow_idx(grow_slot.size());
  for (size_t k = 0; k < items.size(); ++k) at_slot[items[k].slot] = (int)k;
  for (size_t p = 0; p < grow_slot.size(); ++p) grow_idx[p] = grow_slot[p] >= 0 ? at_slot[grow_slot[p]] : -1;
  auto grow = [&](auto **p, size_t &cap, size_t need, size_t elt) -> td_status {
    if (need <= cap) return TD_OK;
    if (*p) TD_HIP(c, hipFree(*p));
    *p = nullptr;
    cap = 0;
    TD_TRY(dmalloc(c, p, need * elt));
    cap = need;
    return TD_OK;
  };
  size_t cap_items = c->items_cap;
  TD_TRY(grow(&c->items_d, cap_items, items.size(), sizeof(AttnItem)));
  c->items_cap = cap_items;
  size_t cap_pairs = c->pairs_cap, cap_pairs2 = c->pairs_cap, cap_pairs3 = c->pairs_cap;
  TD_TRY(grow(&c->pair_first_d, cap_pairs, pfirst.size(), sizeof(int)));
  TD_TRY(grow(&c->pair_count_d, cap_pairs2, pcount.size(), sizeof(int)));
  TD_TRY(grow(&c->grow_idx_d, cap_pairs3, grow_idx.size(), sizeof(int)));
  c->pairs_cap = std::min(cap_pairs, std::min(cap_pairs2, cap_pairs3));
  const size_t rows = items.size() * (size_t)R;
  size_t cap_o = c->att_cap_rows, cap_ml = c->att_cap_rows;
  TD_TRY(grow(&c->att_o, cap_o, rows, (size_t)g.head_dim * 4));
  TD_TRY(grow(&c->att_ml, cap_ml, rows, 8));
  c->att_cap_rows = std::min(cap_o, cap_ml);
  TD_HIP(c, hipMemcpy(c->items_d, items.data(), items.size() * sizeof(AttnItem), hipMemcpyHostToDevice));
  TD_HIP(c, hipMemcpy(c->pair_first_d, pfirst.data(), pfirst.size() * sizeof(int), hipMemcpyHostToDevice));
  TD_HIP(c, hipMemcpy(c->pair_count_d, pcount.data(), pcount.size() * sizeof(int), hipMemcpyHostToDevice));
  TD_HIP(c, hipMemcpy(c->grow_idx_d, grow_idx.data(), grow_idx.size() * sizeof(int), hipMemcpyHostToDevice));
  {  // GEMM plans for this batch size
    const int M = n_seqs * g.block_size;
    const int d = g.d_model, F = g.d_ff, Hd = g.n_heads * g.head_dim;
    c->p_qkv = plan_gemm(M, c->Nqkv, d, false, g.dtype);
    c->p_wo = plan_gemm(M, d, Hd, false, g.dtype);
    c->p_w1 = plan_gemm(M, F, d, false, g.dtype);
    c->p_w2 = plan_gemm(M, d, F, false, g.dtype);
    c->p_lm = plan_gemm(M, g.vocab, d, true, g.dtype);
    size_t need = 0;   // floats of split-K partials
    c->p_router = plan_gemm(M, std::max(c->moe_Epad, 32), d, false, g.dtype);
    const GemmPlan *plans[] = {&c->p_qkv, &c->p_wo, &c->p_w1, &c->p_w2, &c->p_router};
    const int widths[] = {c->Nqkv, d, F, d, c->moe_Epad};
    const size_t Mpad = (size_t)(M + 127) / 128 * 128;   // the tiled kernel's rows, whole tiles
    for (int i = 0; i < 5; ++i) {
      if (plans[i]->splits > 1) need = std::max(need, (size_t)plans[i]->splits * Mpad * widths[i]);
      // A split tiled layer GEMM of a batched step grows its split at few live rows (up
      // to the workspace: here at least 1024 rows' worth of partials at its width).
      if (i < 4 && plans[i]->tile && plans[i]->splits > 1 && n_seqs > 1)
        need = std::max(need, (size_t)1024 * widths[i]);
    }
    TD_TRY(grow(&c->part, c->part_cap, need, sizeof(float)));
    c->part_need = need;
  }
  {  // per-sequence length and first page for the K/V append
    std::vector<int> lp(2 * n_seqs);
    int64_t pb = 0;
    for (int i = 0; i < n_seqs; ++i) {
      lp[i] = (int)len[i];
      lp[n_seqs + i] = (int)pb;
      pb += cap[i];
    }
    TD_HIP(c, hipMemcpy(c->seq_lp_d, lp.data(), lp.size() * sizeof(int), hipMemcpyHostToDevice));
  }
  c->lengths.assign(len, len + n_seqs);
  c->caps.assign(cap, cap + n_seqs);
  c->kc.assign(k_cache_host, k_cache_host + g.n_layers);
  c->vc.assign(v_cache_host, v_cache_host + g.n_layers);
  c->n_items = (int)items.size();
  c->n_pairs = (int)pfirst.size();
  c->attn_single = R <= ATTN_FEW_ROWS && items.size() == pfirst.size();
  c->n_seqs = n_seqs;
  c->grow_len = grow_len;
  c->grow_ok.assign(grow_idx.size(), 0);
  for (size_t p = 0; p < grow_idx.size(); ++p) c->grow_ok[p] = grow_idx[p] >= 0;
  c->chunk = tc;
  return TD_OK;
}

// Every bound sequence grew by `add` tokens (appended to the caches by the work already
// enqueued).  Extends each pair's last prefix item and the device lengths with one small
// kernel, without waiting; rebuilds the binding (which waits for the stream) only when a
// pair has no item that can grow or an item would exceed twice the chunk size.
static td_status advance_binding(td_ctx *c, int add) {
  bool rebuild = false;
  for (size_t p = 0; p < c->grow_len.size(); ++p) {
    if (!c->grow_ok[p] || c->grow_len[p] + add > 2 * c->chunk) rebuild = true;
  }
  std::vector<int64_t> len = c->lengths;
  for (auto &v : len) v += add;
  if (rebuild) {
    const std::vector<int64_t> cap = c->caps;
    const std::vector<const void *> kc = c->kc, vc = c->vc;
    return bind_impl(c, c->n_seqs, len.data(), cap.data(), kc.data(), vc.data());
  }
  TD_HIP(c, launch_advance(c->items_d, c->grow_idx_d, c->n_pairs, c->seq_lp_d, c->n_seqs, add, c->stream));
  for (auto &v : c->grow_len) v += add;
  c->lengths = len;
  return TD_OK;
}

td_status td_set_prefix(td_ctx *c, int32_t n_seqs, const int64_t *off, const void *const *k_cache_host,
                        const void *const *v_cache_host) {
  TD_TRY(check_ctx(c));
  const td_config &g = c->cfg;
  if (n_seqs < 1 || n_seqs > g.max_batch) return fail(c, TD_EINVAL, "n_seqs must be in [1, max_batch=%d]", g.max_batch);
  if (!off || !k_cache_host || !v_cache_host) return fail(c, TD_EINVAL, "NULL offsets or cache array");
  if (off[0] != 0) return fail(c, TD_EINVAL, "prefix_offsets[0] must be 0");
  std::vector<int64_t> len(n_seqs), cap(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    if (off[i + 1] < off[i]) return fail(c, TD_EINVAL, "prefix_offsets must be non-decreasing");
    len[i] = off[i + 1] - off[i];
    cap[i] = (len[i] + KV_PAGE - 1) / KV_PAGE;
  }
  return bind_impl(c, n_seqs, len.data(), cap.data(), k_cache_host, v_cache_host);
}

td_status td_bind_cache(td_ctx *c, int32_t n_seqs, const int64_t *lengths_host, const int64_t *page_capacity_host,
                        const void *const *k_cache_host, const void *const *v_cache_host) {
  TD_TRY(check_ctx(c));
  const td_config &g = c->cfg;
  if (n_seqs < 1 || n_seqs > g.max_batch) return fail(c, TD_EINVAL, "n_seqs must be in [1, max_batch=%d]", g.max_batch);
  if (!lengths_host || !page_capacity_host || !k_cache_host || !v_cache_host)
    return fail(c, TD_EINVAL, "NULL lengths, capacities or cache array");
  return bind_impl(c, n_seqs, lengths_host, page_capacity_host, k_cache_host, v_cache_host);
}

td_status td_denoise_step(td_ctx *c, int32_t *tokens, uint8_t *committed, const float *inv_temp, float gamma,
                          uint8_t *newly, float *conf_out, int32_t *argmax_out, float *logits_out) {
  TD_TRY(check_ctx(c));
  TD_TRY(check_mlp(c));
  if (!tokens || !committed) return fail(c, TD_EINVAL, "tokens and committed must not be NULL");
  if (!finite(gamma)) return fail(c, TD_EINVAL, "gamma must be finite");
  TD_TRY(check_bound(c));
  const int M = c->n_seqs * c->cfg.block_size;
  TD_HIP(c, launch_prep(tokens, committed, M, c->cfg.block_size, c->cfg.vocab, c->st, c->stream));
  return enqueue_step(c, tokens, committed, inv_temp, gamma, newly, conf_out, argmax_out, logits_out, nullptr,
                      nullptr);
}

// Spins on the progress word until the current call's first `need` steps have finished
// on the device (returns 0) or its batch is adopted (1); -1 after a second without
// either (the stream may be waiting on work the caller enqueues later).
static int wait_progress(const td_ctx *c, int need) {
  const auto t0 = std::chrono::steady_clock::now();
  for (unsigned it = 0;; ++it) {
    const unsigned w = __atomic_load_n(c->host_progress, __ATOMIC_ACQUIRE);
    if ((w >> 8) == c->gen) {
      if (w & 1u) return 1;
      if ((int)((w >> 1) & 127u) >= need) return 0;
    }
    if ((it & 1023u) == 1023u && std::chrono::steady_clock::now() - t0 > std::chrono::seconds(1)) return -1;
  }
}

td_status td_generate_block(td_ctx *c, int32_t *tokens, uint8_t *committed, const float *inv_temp, float gamma,
                            int32_t *steps, int8_t *commit_step) {
  TD_TRY(check_ctx(c));
  TD_TRY(check_mlp(c));
  if (!tokens || !committed) return fail(c, TD_EINVAL, "tokens and committed must not be NULL");
  if (!finite(gamma)) return fail(c, TD_EINVAL, "gamma must be finite");
  TD_TRY(check_bound(c));
  const td_config &g = c->cfg;
  TD_HIP(c, launch_init_block(tokens, committed, commit_step, steps, c->n_seqs, g.block_size, g.vocab, c->st,
                              c->stream));
  // With an issue window W, step s is enqueued once the device has finished step s - W
  // (so W - 1 steps stay queued behind the running one), and no step is enqueued once
  // the device reports the batch adopted: the launches that would only test the loop-exit
  // flag are never issued.  The loop's decisions stay on the device either way.
  const int W = c->issue_window;
  bool wait = W > 0 && c->host_progress;
  if (wait) {
    c->gen = (c->gen + 1) & 0xFFFFFFu;
    if (c->gen == 0) c->gen = 1;
  }
  c->progress_armed = wait;
  td_status st = TD_OK;
  for (int s = 0; s < g.block_size && st == TD_OK; ++s) {
    if (wait && s >= W) {
      const int r = wait_progress(c, s - W + 1);
      if (r > 0) break;
      if (r < 0) wait = false;   // issue the rest at once
    }
    st = enqueue_step(c, tokens, committed, inv_temp, gamma, nullptr, nullptr, nullptr, nullptr, steps, commit_step);
  }
  c->progress_armed = false;
  return st;
}

td_status td_set_issue_window(td_ctx *c, int32_t steps_ahead) {
  TD_TRY(check_ctx(c));
  if (steps_ahead < 0) return fail(c, TD_EINVAL, "steps_ahead must be >= 0");
  if (steps_ahead > 0 && !c->host_progress) {
    TD_HIP(c, hipSetDevice(c->dev));
    void *p = nullptr;
    const hipError_t e = hipHostMalloc(&p, 256, hipHostMallocCoherent);
    if (e != hipSuccess) return fail(c, TD_ENOMEM, "hipHostMalloc(256, coherent) failed: %s", hipGetErrorString(e));
    std::memset(p, 0, 256);
    c->host_progress = static_cast<unsigned *>(p);
  }
  c->issue_window = steps_ahead;
  return TD_OK;
}

td_status td_set_commit_rule(td_ctx *c, int32_t rule, int32_t min_adopt) {
  TD_TRY(check_ctx(c));
  if (rule == TD_RULE_LEFT_TO_RIGHT) {
    c->rule = RULE_LEFT_TO_RIGHT;
    c->min_adopt = 1;
    return TD_OK;
  }
  if (rule != TD_RULE_THRESHOLD) return fail(c, TD_EINVAL, "unknown commit rule %d", rule);
  if (min_adopt < 1 || min_adopt > c->cfg.block_size)
    return fail(c, TD_EINVAL, "min_adopt must be in [1, block_size=%d]", c->cfg.block_size);
  c->rule = RULE_THRESHOLD;
  c->min_adopt = min_adopt;
  return TD_OK;
}

td_status td_set_context_tower(td_ctx *c, const td_weights *w) {
  TD_TRY(check_ctx(c));
  if (validate_weights(c->cfg, w, true) != TD_OK) return fail(c, TD_EINVAL, "%s", g_create_error.c_str());
  TD_HIP(c, hipSetDevice(c->dev));
  TD_HIP(c, hipStreamSynchronize(c->stream));   // a previous context tower may still be in use
  auto f = [](void *p) {
    if (p) (void)hipFree(p);
  };
  for (auto *v : {&c->context.attn_norm, &c->context.mlp_norm, &c->context.wqkv, &c->context.wo, &c->context.w1,
                  &c->context.w2}) {
    for (void *p : *v) f(p);
    v->clear();
  }
  f(c->ctx_tok_emb); f(c->ctx_final_norm); f(c->ctx_lm_head);
  c->ctx_tok_emb = c->ctx_final_norm = c->ctx_lm_head = nullptr;
  const size_t e = c->elt, d = c->cfg.d_model, V = c->cfg.vocab;
  TD_TRY(dmalloc(c, &c->ctx_tok_emb, (V + 1) * d * e));
  TD_HIP(c, hipMemcpyAsync(c->ctx_tok_emb, w->tok_emb, (V + 1) * d * e, hipMemcpyDeviceToDevice, c->stream));
  if (w->final_norm && w->lm_head) {   // a head of its own: AR decoding (td_ar_step)
    TD_TRY(dmalloc(c, &c->ctx_final_norm, d * e));
    TD_TRY(dmalloc(c, &c->ctx_lm_head, V * d * e));
    TD_HIP(c, hipMemcpyAsync(c->ctx_final_norm, w->final_norm, d * e, hipMemcpyDeviceToDevice, c->stream));
    TD_HIP(c, launch_pack_weight(c->cfg.dtype, w->lm_head, c->ctx_lm_head, (int)V, (int)d, c->stream));
  }
  TD_TRY(pack_layers(c, *w, c->context));
  TD_HIP(c, hipStreamSynchronize(c->stream));
  return TD_OK;
}

td_status td_append_block(td_ctx *c, const int32_t *tokens) {
  TD_TRY(check_ctx(c));
  if (!tokens) return fail(c, TD_EINVAL, "tokens must not be NULL");
  if (!c->ctx_tok_emb) return fail(c, TD_EINVAL, "no context tower: call td_set_context_tower first");
  TD_TRY(check_bound(c));
  const int B = c->cfg.block_size;
  std::vector<int64_t> len = c->lengths;
  for (int i = 0; i < c->n_seqs; ++i) {
    if (len[i] + B > c->caps[i] * KV_PAGE)
      return fail(c, TD_EINVAL, "sequence %d: no room for %d more tokens (%lld tokens, %lld pages)", i, B,
                  (long long)len[i], (long long)c->caps[i]);
    len[i] += B;
  }
  TD_TRY(enqueue_context_pass(c, tokens));
  return advance_binding(c, B);
}

td_status td_ar_step(td_ctx *c, int32_t *tokens) {
  TD_TRY(check_ctx(c));
  if (!tokens) return fail(c, TD_EINVAL, "tokens must not be NULL");
  if (c->cfg.block_size != 1) return fail(c, TD_EINVAL, "AR decoding needs a ctx created with block_size 1");
  if (!c->ctx_lm_head) return fail(c, TD_EINVAL, "no context tower with an LM head: call td_set_context_tower");
  TD_TRY(check_bound(c));
  std::vector<int64_t> len = c->lengths;
  for (int i = 0; i < c->n_seqs; ++i) {
    if (len[i] + 1 > c->caps[i] * KV_PAGE)
      return fail(c, TD_EINVAL, "sequence %d: no room for another token (%lld tokens, %lld pages)", i,
                  (long long)len[i], (long long)c->caps[i]);
    len[i] += 1;
  }
  const td_config &g = c->cfg;
  TD_TRY(enqueue_context_pass(c, tokens, true));
  // Every row masked, then the head and the adoption rule at gamma 0: each row adopts its
  // prediction, the lowest id of its largest logit.
  TD_HIP(c, launch_init_block(tokens, c->ar_committed, nullptr, nullptr, c->n_seqs, 1, g.vocab, c->st, c->stream));
  TD_TRY(enqueue_head_commit(c, c->ctx_lm_head, tokens, c->ar_committed, nullptr, 0.f, RULE_THRESHOLD, 1, nullptr,
                             nullptr, nullptr, nullptr, nullptr, nullptr));
  return advance_binding(c, 1);
}

static td_status set_moe_impl(td_ctx *c, const td_moe_config &m, const td_moe_weights &w) {
  const td_config &g = c->cfg;
  const size_t e = c->elt, d = g.d_model, de = m.d_expert, L = g.n_layers;
  const size_t E = m.n_experts, S = m.n_shared, NE = E + S;
  c->moe_cfg = m;
  c->moe_Epad = (m.n_experts + 31) / 32 * 32;
  c->moe_max_tiles = moe_max_tiles(c->Mmax, m);
  c->moe_cap_rows = 16 * c->moe_max_tiles;
  const size_t Ep = c->moe_Epad, M = c->Mmax, cap = c->moe_cap_rows;
  c->moe_router.assign(L, nullptr);
  c->moe_w1.assign(L, nullptr);
  c->moe_w2.assign(L, nullptr);
  void *tmp = nullptr;   // the router padded to Epad rows of zeros
  TD_TRY(dmalloc(c, &tmp, Ep * d * e));
  td_status st = TD_OK;
  for (size_t l = 0; l < L && st == TD_OK; ++l) {
    st = [&]() -> td_status {
      TD_TRY(dmalloc(c, &c->moe_router[l], Ep * d * e));
      TD_TRY(dmalloc(c, &c->moe_w1[l], NE * de * d * e));
      TD_TRY(dmalloc(c, &c->moe_w2[l], NE * d * de * e));
      TD_HIP(c, hipMemsetAsync(tmp, 0, Ep * d * e, c->stream));
      TD_HIP(c, hipMemcpyAsync(tmp, w.router[l], E * d * e, hipMemcpyDeviceToDevice, c->stream));
      TD_HIP(c, launch_pack_weight(g.dtype, tmp, c->moe_router[l], (int)Ep, (int)d, c->stream));
      // Expert e's rows of a per-layer [E * rows][cols] matrix pack to one contiguous block.
      TD_HIP(c, launch_pack_weight(g.dtype, w.w1[l], c->moe_w1[l], (int)(E * de), (int)d, c->stream));
      TD_HIP(c, launch_pack_weight(g.dtype, w.w2[l], c->moe_w2[l], (int)(E * d), (int)de, c->stream));
      if (S) {
        TD_HIP(c, launch_pack_weight(g.dtype, w.shared_w1[l], (char *)c->moe_w1[l] + E * de * d * e, (int)(S * de),
                                     (int)d, c->stream));
        TD_HIP(c, launch_pack_weight(g.dtype, w.shared_w2[l], (char *)c->moe_w2[l] + E * d * de * e, (int)(S * d),
                                     (int)de, c->stream));
      }
      TD_HIP(c, hipStreamSynchronize(c->stream));   // tmp is reused by the next layer
      return TD_OK;
    }();
  }
  (void)hipFree(tmp);
  TD_TRY(st);
  TD_TRY(dmalloc(c, &c->moe_scores, M * Ep * 4));
  TD_TRY(dmalloc(c, &c->moe_experts, M * m.top_k * 4));
  TD_TRY(dmalloc(c, &c->moe_gates, M * m.top_k * 4));
  TD_TRY(dmalloc(c, &c->moe_rs, M * 4));
  TD_TRY(dmalloc(c, &c->moe_slot_pos, M * (m.top_k + S) * 4));
  TD_TRY(dmalloc(c, &c->moe_src_row, cap * 4));
  TD_TRY(dmalloc(c, &c->moe_tiles, (size_t)c->moe_max_tiles * sizeof(int4)));
  TD_TRY(dmalloc(c, &c->moe_n_tiles, 4));
  TD_TRY(dmalloc(c, &c->moe_u, afl_bytes((int)cap, (int)de)));
  TD_TRY(dmalloc(c, &c->moe_y, cap * d * 4));
  TD_TRY(dmalloc(c, &c->moe_stats, 2 * sizeof(long long)));
  // The grouped GEMMs read tile entries and sorted rows beyond the live ones before they
  // test the live count: zeroed entries (expert 0, row 0) keep those reads in bounds.
  TD_HIP(c, hipMemsetAsync(c->moe_src_row, 0, cap * 4, c->stream));
  TD_HIP(c, hipMemsetAsync(c->moe_tiles, 0, (size_t)c->moe_max_tiles * sizeof(int4), c->stream));
  TD_HIP(c, hipMemsetAsync(c->moe_n_tiles, 0, 4, c->stream));
  TD_HIP(c, hipMemsetAsync(c->moe_u, 0, afl_bytes((int)cap, (int)de), c->stream));
  TD_HIP(c, hipMemsetAsync(c->moe_stats, 0, 2 * sizeof(long long), c->stream));
  TD_HIP(c, hipStreamSynchronize(c->stream));
  return TD_OK;
}

td_status td_set_moe(td_ctx *c, const td_moe_config *mc, const td_moe_weights *w) {
  TD_TRY(check_ctx(c));
  if (!mc || !w) return fail(c, TD_EINVAL, "MoE config and weights must not be NULL");
  const td_moe_config m = *mc;
  if (m.n_experts < 1 || m.n_experts > MOE_MAX_EXPERTS)
    return fail(c, TD_EINVAL, "n_experts must be in [1, %d]", MOE_MAX_EXPERTS);
  if (m.top_k < 1 || m.top_k > MOE_MAX_TOP_K || m.top_k > m.n_experts)
    return fail(c, TD_EINVAL, "top_k must be in [1, min(%d, n_experts)]", MOE_MAX_TOP_K);
  if (m.n_shared < 0 || m.n_shared > MOE_MAX_SHARED)
    return fail(c, TD_EINVAL, "n_shared must be in [0, %d]", MOE_MAX_SHARED);
  if (m.d_expert < 64 || m.d_expert % 64 || m.d_expert > (1 << 20))
    return fail(c, TD_EINVAL, "d_expert must be a positive multiple of 64");
  {  // the packed expert matrices are addressed with 32-bit row counts
    const int64_t NE = (int64_t)m.n_experts + m.n_shared;
    if (NE * m.d_expert > INT32_MAX || NE * c->cfg.d_model > INT32_MAX)
      return fail(c, TD_EUNSUPPORTED, "experts x width too large");
  }
  const void *const *lists[] = {w->router, w->w1, w->w2, w->shared_w1, w->shared_w2};
  for (int k = 0; k < 5; ++k) {
    if (k >= 3 && m.n_shared == 0) continue;
    if (!lists[k]) return fail(c, TD_EINVAL, "a per-layer MoE weight array is NULL");
    for (int l = 0; l < c->cfg.n_layers; ++l)
      if (!lists[k][l]) return fail(c, TD_EINVAL, "MoE weight pointer of layer %d is NULL", l);
  }
  TD_HIP(c, hipSetDevice(c->dev));
  TD_HIP(c, hipStreamSynchronize(c->stream));   // earlier steps may still read the old experts
  free_moe(c);
  td_status s = set_moe_impl(c, m, *w);
  if (s == TD_OK && c->n_seqs > 0) {   // the router's GEMM plan for the bound batch
    const int M = c->n_seqs * c->cfg.block_size;
    c->p_router = plan_gemm(M, c->moe_Epad, c->cfg.d_model, false, c->cfg.dtype);
    const size_t need = c->p_router.splits > 1 ? (size_t)c->p_router.splits * ((size_t)(M + 127) / 128 * 128) * c->moe_Epad : 0;
    c->part_need = std::max(c->part_need, need);
    if (need > c->part_cap) {
      if (c->part) (void)hipFree(c->part);
      c->part = nullptr;
      c->part_cap = 0;
      s = dmalloc(c, &c->part, need * sizeof(float));
      if (s == TD_OK) c->part_cap = need;
    }
  }
  if (s != TD_OK) {
    (void)hipStreamSynchronize(c->stream);
    free_moe(c);
    return s;
  }
  c->moe = true;
  return TD_OK;
}

td_status td_moe_stats(td_ctx *c, int64_t *launches, int64_t *active) {
  TD_TRY(check_ctx(c));
  if (!c->moe) return fail(c, TD_EINVAL, "no mixture of experts set: call td_set_moe first");
  if (!launches || !active) return fail(c, TD_EINVAL, "output pointers must not be NULL");
  TD_HIP(c, hipSetDevice(c->dev));
  TD_HIP(c, hipStreamSynchronize(c->stream));
  long long v[2] = {0, 0};
  TD_HIP(c, hipMemcpy(v, c->moe_stats, sizeof v, hipMemcpyDeviceToHost));
  TD_HIP(c, hipMemset(c->moe_stats, 0, sizeof v));
  *launches = v[0];
  *active = v[1];
  return TD_OK;
}

td_status td_debug_attention(td_ctx *c, int32_t layer, const void *qkv, void *o) {
  TD_TRY(check_ctx(c));
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, TD_EINVAL, "layer out of range");
  if (!qkv || !o) return fail(c, TD_EINVAL, "qkv and o must not be NULL");
  TD_TRY(check_bound(c));
  return enqueue_attention(c, layer, (const float *)qkv, (float *)o, nullptr, nullptr);
}

td_status td_sync(td_ctx *c) {
  TD_TRY(check_ctx(c));
  TD_HIP(c, hipSetDevice(c->dev));
  TD_HIP(c, hipStreamSynchronize(c->stream));
  int err = 0;
  TD_HIP(c, hipMemcpy(&err, c->st.err, sizeof(int), hipMemcpyDeviceToHost));
  if (err) {
    const int zero = 0;
    TD_HIP(c, hipMemcpy(c->st.err, &zero, sizeof(int), hipMemcpyHostToDevice));
    return fail(c, TD_EDEVICE, "device-side input error %d: %s", err,
                (err & 1) ? "token/committed state invalid (a token outside [0, vocab], or [MASK] not exactly at "
                            "uncommitted positions)"
                          : "token id outside [0, vocab]");
  }
  return TD_OK;
}

td_status td_profile_begin(td_ctx *c, int32_t kinds_mask) {
  TD_TRY(check_ctx(c));
  if (kinds_mask & ~((1 << TD_PROF_KINDS) - 1)) return fail(c, TD_EINVAL, "unknown profiling kinds in mask 0x%x", kinds_mask);
  c->prof_mask = (unsigned)kinds_mask & ~1u;   // bit 0 (TD_PROF_OFF) brackets nothing
  for (long &o : c->prof_open) o = -1;
  return TD_OK;
}

td_status td_profile_layer(td_ctx *c, int32_t layer) {
  TD_TRY(check_ctx(c));
  if (layer < -1 || layer >= c->cfg.n_layers) return fail(c, TD_EINVAL, "layer must be in [-1, n_layers)");
  c->prof_only_layer = layer;
  return TD_OK;
}

int32_t td_profile_end(td_ctx *c, float *ms_out, int32_t *tags_out, int32_t max) {
  if (!c) return -1;
  if (hipStreamSynchronize(c->stream) != hipSuccess) return -1;
  const size_t n = c->prof_n;
  c->prof_n = 0;
  c->prof_mask = 0;
  for (size_t i = 0; i < n && (int64_t)i < max; ++i) {
    float ms = 0.f;
    if (ms_out) {
      if (hipEventElapsedTime(&ms, c->ev_start[i], c->ev_stop[i]) != hipSuccess) return -1;
      ms_out[i] = ms;
    }
    if (tags_out) tags_out[i] = c->ev_tag[i];
  }
  return (int32_t)n;
}

int32_t td_kernels_per_step(const td_ctx *c) {
  if (!c) return -1;
  // prep/init, embed; per layer the projections (a K-split one adds its reduction),
  // attention and its merge, and the MLP or the mixture of experts (router GEMM, routing
  // and bucketing in one launch up to 64 rows, else two, the expert up and down
  // projections, the combine); the LM head and the merge + commit (two launches above
  // COMMIT_SMALL_ROWS rows).
  auto gemm = [](const GemmPlan &p) { return 1 + (p.splits > 1 ? 1 : 0); };
  const int M = std::max(1, c->n_seqs) * c->cfg.block_size;
  int layer = gemm(c->p_qkv) + 2 + gemm(c->p_wo);
  layer += c->moe ? gemm(c->p_router) + (M <= 64 ? 1 : 2) + 3 : gemm(c->p_w1) + gemm(c->p_w2);
  return 2 + layer * c->cfg.n_layers + 2 + (M > COMMIT_SMALL_ROWS ? 1 : 0);
}

void td_destroy(td_ctx *c) {
  if (!c) return;
  (void)hipSetDevice(c->dev);
  (void)hipStreamSynchronize(c->stream);
  free_all(c);
  delete c;
}

const char *td_last_error(const td_ctx *c) { return c ? c->err.c_str() : g_create_error.c_str(); }

const char *td_version(void) { return "td 0.1 (gfx950)"; }

}  // extern "C"
