// Host-side launch interface of the gfx950 kernels (internal to libtd).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace td {

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };
enum Epi { EPI_STORE = 0, EPI_GELU = 1, EPI_RESID = 2, EPI_VSTAT = 3 };

// Softmax statistics of a set of scaled logits: max, sum of exp(s - max), lowest index
// of the max.
struct VStat {
  float m, s;
  int a;
};

// ---------------------------------------------------------------- packing
// W [N][K] row-major -> 16x32 MFMA tiles, tile (nt, kt) at ((nt * K/32 + kt) * 64 + lane) * 8,
// lane l holding W[16 nt + l%16][32 kt + 8 (l/16) .. +8].
hipError_t launch_pack_weight(int dtype, const void *W, void *Wp, int N, int K, hipStream_t s);

// ---------------------------------------------------------------- activations in fragment layout
// Activation matrices that feed a GEMM are stored by their producer in MFMA A-fragment
// order ("AFL"): fragment (mt, kt, lane) is 32 bytes at ((mt * K/32 + kt) * 64 + lane) * 32
// and holds row 16 mt + lane % 16, columns 32 kt + 8 (lane / 16) .. +8, as 8 bf16 high
// parts then 8 bf16 remainders (bf16 towers) or as 8 fp32 values (fp32 towers): 4 bytes
// per element either way.  Rows are padded to a multiple of 64 (the widest row tile).
inline size_t afl_bytes(int rows, int K) { return (size_t)((rows + 63) / 64 * 64) * K * 4; }

// ---------------------------------------------------------------- GEMM (weight streaming)
struct GemmArgs {
  int M, N, K;             // M: row capacity (grid); the live count is *n_rows when n_rows != nullptr
  const void *A;           // activations [M][K] in fragment layout
  // RMSNorm (NORM variants): A holds x * gain; the row scale 1/sqrt(mean(x^2) + eps)
  // comes from the producer's partial sums of squares and multiplies the accumulator.
  const float *ssq;        // [norm_nparts][ld_ssq]
  int norm_nparts, ld_ssq;
  float norm_eps;
  const int *rowlist;      // optional row gather: GEMM row r is activation row rowlist[r]
  const int *rowpos;       // VSTAT, few-row kernel: position of each row in the row list, or -1
  const int *n_rows;       // optional live row count (device)
  const void *Wp;          // packed weight [N][K]
  int nt;                  // 16-column tiles per wave (launch_gemm: 1, 2, 4, 8) or per workgroup (launch_gemm_wk: 1, 2, 4)
  int nw;                  // waves per workgroup (launch_gemm: 4, 8; launch_gemm_wk: 4, 8, 16)
  float *out; int ldo;     // STORE: fp32 [M][ldo]; RESID: x [M][ldo], updated in place
  void *out_afl;           // GELU: gelu(y) [M][N] in fragment layout; RESID: x * gain_next, same layout
  const void *gain_next;   // RESID: [N] gain of the RMSNorm that consumes the updated x
  float *ssq_out;          // RESID: [N/16][M] partial sums of squares of the updated rows
  const float *inv_temp;   // VSTAT: [rows] inverse temperature, or nullptr (1)
  VStat *vpart;            // VSTAT: [row index][grid.x] statistics of each column group
  float *logits;           // VSTAT: optional capture [rows][N] of the raw logits
  const int *done;         // skip the launch when *done != 0 (required: read before the operands)
  int splits;              // K split over this many workgroups (1: none; not VSTAT)
  float *part;             // K-split partial products, fp32 (workspace): [splits][M][N] for the
                           // weight-streaming kernels, [S][live tiles * tile_rows][N] for the tiled one
  int dyn;                 // tiled layer GEMM over live rows (*n_rows): the K split grows on the
                           // device when the live row tiles fill less than one workgroup per CU;
                           // split_reduce then sums the partials (it does nothing when none grew)
  int tile_rows;           // tiled kernel: rows per workgroup tile (set by launch_gemm_tile)
  size_t part_cap;         // floats of `part` a grown split may use
};
// The LM head (EPI_VSTAT): nw waves x nt column tiles per workgroup, each wave streaming
// its own columns over the whole K range.
hipError_t launch_gemm(int dtype, int epi, bool norm, const GemmArgs &a, hipStream_t s);
// Column groups of the LM head, i.e. vocabulary-statistics triples per row.
int lmhead_slices(int N, int nt, int nw);
// Many rows (bf16, M >= 128, N % 128 == 0, K % 32 == 0): 128 x 128 tiles through
// double-buffered LDS, every epilogue (VSTAT: one statistics triple per 128 columns).
// With a.splits > 1 (not VSTAT) the K range is split over that many workgroups, which
// store fp32 partials to a.part, and a second kernel sums them in split order and
// applies the epilogue.
bool gemm_tile_supported(int dtype, int M, int N, int K);
int gemm_tile_slices(int N);
int gemm_tile_splits(int M, int N, int K);   // splits that give the grid ~2 workgroups per CU
hipError_t launch_gemm_tile(int epi, bool norm, const GemmArgs &a, hipStream_t s);
// Sum of a.splits fp32 partials part[split][M][N] in split order, then the row scale and
// the epilogue (STORE, GELU or RESID) of the projection.
hipError_t launch_split_reduce(int epi, bool norm, const GemmArgs &a, hipStream_t s);
// One 16-column tile per workgroup, its nw waves splitting K with all weights in flight;
// used for the layer projections (STORE, GELU, RESID).
hipError_t launch_gemm_wk(int dtype, int epi, bool norm, const GemmArgs &a, hipStream_t s);

// ---------------------------------------------------------------- attention
// Prefix K/V cache pages: 32 tokens per page; page p of K/V head h is one contiguous
// block of 32 * hd elements.  V is transposed, [hd][32 tokens]: element (slot, e) at
//   ((p * Hkv + h) * hd + e) * 32 + slot.
// K is [hd / 32][2][16][32]: element (slot, e) at
//   ((p * Hkv + h) * 32 * hd) + ((e / 32) * 2 + hf) * 512 + i * 32 + e % 32,
// with hf = (slot / 4) % 2 and i = (slot / 8) * 4 + slot % 4 (the row of the key in the
// MFMA operand of its half of the page).
// Sequence i owns pages [page_off[i], page_off[i] + ceil(P_i / 32)); token t is in page
// page_off[i] + t / 32, slot t % 32.
constexpr int KV_PAGE = 32;

// Query rows per (seq, kv head) pair up to which attention takes the few-row path (four
// waves per item straight from HBM); more rows take the grouped-query path.
constexpr int ATTN_FEW_ROWS = 32;


// One split-K work item of a (seq, kv head) pair: prefix tokens [k_begin, k_end)
// (k_begin a multiple of the page size, first page page0 of the cache) and/or the
// block's own keys.  The slots of a pair's items are consecutive; the items array is in
// launch order.  is_block:
//   0  prefix keys only;
//   2  prefix keys and the block's keys (the pair's first item; the prefix range is
//      empty when the sequence has no prefix).
struct AttnItem {
  int seq, kvh;            // sequence and key/value head
  int k_begin, k_end;      // prefix key range (token index within the sequence)
  int is_block;            // 0 or 2 as above
  int slot;                // partial-state slot: the item's index in (pair, key range) order
  int64_t page0;           // cache page holding token k_begin (prefix items)
};
struct AttnArgs {
  int B, H, Hkv, hd, Nqkv, G, R;   // R = G * B query rows per (seq, kv head)
  int causal;                      // 1: block query p sees block keys 0..p only (context tower)
  const int *seq_done;             // [n] 1: the sequence's block is fully adopted, skip it (never null)
  const float *qkv;                // [n*B][Nqkv]: q | k_block | v_block (fp32)
  const void *kc, *vc;             // prefix cache pages (layout above)
  const AttnItem *items; int n_items;
  const int *pair_first, *pair_count;   // item range of each (seq, kv head) pair
  int n_pairs;
  float *part_o;                   // [n_items][R][hd] partial outputs (unnormalised)
  float *part_ml;                  // [n_items][R][2] partial max and sum of exp
  float *o; int ldo;               // optional output [n*B][ldo] (fp32, natural layout)
  void *o_afl;                     // optional output [n*B][H*hd] in fragment layout
  float scale;                     // 1 / sqrt(hd)
  const int *done;
  int single;                      // 1: every pair has one item (few-row path): the items write
                                   // the normalised output (o, o_afl) themselves, no merge runs
};
// part: ATTN_SPLIT (the split-K items), ATTN_MERGE (the merge of their partials; nothing
// when a.single), or both.
enum { ATTN_SPLIT = 1, ATTN_MERGE = 2 };
hipError_t launch_attention(int dtype, const AttnArgs &a, int part, hipStream_t s);

// ---------------------------------------------------------------- embedding, step control
struct StepState {                 // device-resident loop state owned by the ctx
  int *rowlist;                    // [M] rows (seq*B + p) still masked, ascending
  int *rowpos;                     // [M] index of each row in rowlist, or -1
  int *n_rows;                     // number of masked rows
  int *act_rows;                   // [M] rows of the sequences that still have a masked position, ascending
  int *n_act;                      // number of such rows (the layer GEMMs' live rows)
  int *done;                       // 1 when no row is masked
  int *t;                          // step counter of td_generate_block
  int *err;                        // device-side input error flags
  int *seq_done;                   // [n] 1 when the sequence has no masked position left
};
hipError_t launch_prep(const int *tokens, const uint8_t *committed, int M, int B, int V, StepState st, hipStream_t s);
hipError_t launch_init_block(int *tokens, uint8_t *committed, int8_t *commit_step, int *steps, int n, int B,
                             int V, StepState st, hipStream_t s);
// x = E[token] + Pos[position] (fp32), partial sums of squares per 16 columns, and
// x * gain (the first RMSNorm's gain) in fragment layout.
hipError_t launch_embed(int dtype, const int *tokens, const void *E, const void *Pos, const void *gain, float *x,
                        float *ssq, void *x_afl, int M, int B, int d, int V, StepState st, hipStream_t s);

// ---------------------------------------------------------------- vocab merge + commit
enum { RULE_THRESHOLD = 0, RULE_LEFT_TO_RIGHT = 1 };   // = td_commit_rule
struct CommitArgs {
  int V, B, n, nslices;
  int rule, min_adopt;             // adoption rule (td_set_commit_rule)
  const VStat *vpart;              // [row index][nslices]
  float *conf_row; int *arg_row;   // [M] per-row results (indexed by position in rowlist)
  int *tokens; uint8_t *committed;
  float gamma;
  uint8_t *newly;                  // nullable [n*B]
  float *conf_out; int *argmax_out;   // nullable [n*B]
  int *steps; int8_t *commit_step; // nullable
  StepState st;
  // Nullable: a word in coherent pinned host memory that the commit overwrites with
  // (gen << 8) | (steps finished << 1) | adopted, for a host issuing the loop's steps a
  // few at a time.
  unsigned *host_progress; unsigned gen;
};
// Up to COMMIT_SMALL_ROWS rows one launch merges and commits; more rows take two.
constexpr int COMMIT_SMALL_ROWS = 128;
hipError_t launch_merge_commit(const CommitArgs &a, int max_rows, hipStream_t s);
// K/V of the block rows of qkv ([n*B][Nqkv] fp32: q | k | v) appended to one layer's cache
// (layout above; bf16 caches round to nearest even): row seq*B + p is token
// seq_len[seq] + p of sequence seq, whose pages start at seq_page[seq].
// Every bound sequence grew by `add` appended tokens: items[grow_idx[p]].k_end += add for
// each pair p with grow_idx[p] >= 0, and seq_len[s] += add for each sequence.
hipError_t launch_advance(AttnItem *items, const int *grow_idx, int n_pairs, int *seq_len, int n_seqs, int add,
                          hipStream_t s);
hipError_t launch_kv_append(int dtype, const float *qkv, int Nqkv, int H, int Hkv, int hd, void *kc, void *vc,
                            const int *seq_len, const int *seq_page, int n, int B, hipStream_t s);

// ---------------------------------------------------------------- mixture of experts
// Routing, expert-grouped weight streaming and the gated sum of a mixture-of-experts MLP
// (see k_moe.hip).  Experts 0 .. E-1 are routed, E .. E+n_shared-1 shared.  Expert-sorted
// rows: every expert's rows form a segment padded to a multiple of 16, so each 16-row
// tile belongs to one expert.
constexpr int MOE_MAX_EXPERTS = 256, MOE_MAX_TOP_K = 8, MOE_MAX_SHARED = 4;
struct MoeRoute {
  int M, E, Epad, top_k, n_shared, d;
  const float *scores;        // [M][Epad] router scores (fp32, row scale applied)
  const float *ssq;           // [d/16][M] partial sums of squares of the MLP input rows
  float eps;                  // RMSNorm epsilon
  int *experts;               // [M][top_k] chosen experts by rank
  float *gates;               // [M][top_k]
  float *rs;                  // [M] RMSNorm row scale of each row
  int *slot_pos;              // [M][top_k + n_shared] sorted row of each (row, slot)
  int *src_row;               // [cap_rows] token row of each sorted row (padding: row 0)
  int4 *tiles;                // [max_tiles] (expert, first sorted row, live rows, 0)
  int *n_tiles;               // tiles in use
  long long *stats;           // [2] launches, sum of active experts
  const int *seq_done;        // [M / B] 1: the sequence's block is adopted, its rows are not routed
  int B;                      // rows per sequence
  const int *done;
};
hipError_t launch_moe_route(const MoeRoute &a, hipStream_t s);   // route + bucket (two kernels)
struct MoeGemm {
  int N, K;                   // per expert: Y[rows][N] = A[rows][K] * W_e[N][K]^T
  const void *A;              // W1: the MLP input x * gain in fragment layout, gathered by
                              // src_row; W2: the sorted GELU output in fragment layout
  const int *src_row;         // W1 only
  const float *rs;            // W1 only: row scales, indexed by token row
  const void *Wp;             // packed experts, expert e at e * N * K elements
  const int4 *tiles; const int *n_tiles; int max_tiles;
  void *out_afl;              // W1: gelu(y) of the sorted rows in fragment layout (all 16 rows of a tile)
  float *out;                 // W2: y of the sorted rows, fp32 [cap_rows][N] (live rows)
  const int *done;
};
hipError_t launch_moe_gemm(int dtype, bool up, const MoeGemm &a, hipStream_t s);
struct MoeCombine {
  int M, d, top_k, n_shared;
  const int *slot_pos; const float *gates; const float *y;
  float *x;                   // [M][d] residual stream, updated in place
  void *out_afl;              // x * gain_next in fragment layout
  const void *gain_next;      // [d]
  float *ssq_out;             // [d/16][M]
  const int *seq_done; int B; // rows of adopted sequences are left as they are
  const int *done;
};
hipError_t launch_moe_combine(int dtype, const MoeCombine &a, hipStream_t s);

}  // namespace td
