/*
 * td.h — C ABI of the block-diffusion denoising step on MI355X (gfx950).
 *
 * The operation.  A block of B positions, each holding a vocabulary token or the
 * [MASK] token (id == vocab), is refined by a denoiser tower whose block queries
 * attend, in one softmax, over the frozen context tower's cached prefix keys/values
 * and bidirectionally over the block's own keys (poko-everyday.com Nemotron-TwoTower
 * news item, section 技術/ビジネス面).  An LM head and a vocabulary softmax give each
 * masked position a confidence (largest probability of its logits scaled by the
 * position's inverse temperature) and a prediction (lowest id of the largest logit).
 * Masked positions whose confidence is at least gamma are adopted; if none is, the
 * single most confident masked position is; the rest stay [MASK], and the loop
 * repeats until the block has no [MASK] left (PredNext "人工知能は拡散言語モデルの夢を
 * 見るか？", section 拡散言語モデルで推論するには, steps 1-5; dzen.guru "NVIDIA
 * Nemotron 70B генерирует текст…", section "Как попробовать?": block 16, threshold 0.8).
 *
 * Conventions.
 *  - Every buffer pointer is a DEVICE pointer unless its name ends in _host.
 *  - All calls enqueue work on the stream given to td_create and return without
 *    waiting, except where a call's comment says it waits (the binding and setup
 *    calls, td_moe_stats, td_generate_block under an issue window, and td_append_block /
 *    td_ar_step when they rebuild the work lists); results are valid once that stream
 *    has synchronised (td_sync).
 *  - A ctx is bound to one device and one stream and is not thread-safe.
 *  - Every call returns td_status; no C++ exception crosses the ABI.  Arguments are
 *    validated on the host before anything is enqueued (TD_EINVAL, nothing runs).
 *    Asynchronous device faults and device-side input errors (a token id outside
 *    [0, vocab]) surface as TD_EDEVICE from td_sync or a later call; the message is
 *    in td_last_error.
 *  - Layouts are row-major.  bf16 is stored as IEEE bfloat16 (uint16 bit pattern).
 */
#ifndef TD_H
#define TD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct td_ctx td_ctx;

typedef enum {
  TD_OK = 0,
  TD_EINVAL = 1,        /* bad argument; nothing was enqueued */
  TD_ENOMEM = 2,        /* device allocation failed or capacity exceeded */
  TD_EDEVICE = 3,       /* HIP runtime / device error, or a device-side input error */
  TD_EUNSUPPORTED = 4   /* valid but unsupported shape */
} td_status;

typedef enum { TD_F32 = 0, TD_BF16 = 1 } td_dtype;

/* Tower shape and capacity.  Supported: head_dim in {64, 128}; block_size in {8, 16, 32}
 * (and 1, one row per sequence: the ctx for AR decoding, td_ar_step);
 * n_heads % n_kv_heads == 0; d_model, d_ff, vocab multiples of 64; n_heads*head_dim a
 * multiple of 64.  dtype is the storage type of weights and prefix K/V.  Activations
 * (the residual stream, normed inputs, q/k/v, attention output, MLP activation) and all
 * accumulators and softmax statistics are fp32 either way; against bf16 weights an
 * activation enters the bf16 matrix cores as a bf16 high part plus a bf16 remainder. */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab;
  int32_t block_size;          /* B, positions per block */
  int32_t max_batch;           /* capacity: sequences per call */
  int64_t max_prefix_tokens;   /* capacity: sum of prefix lengths over the batch */
  int32_t dtype;               /* td_dtype */
  float rms_eps;               /* RMSNorm epsilon (1e-6 in the synthetic towers) */
} td_config;

/* Tower weights, DEVICE pointers in the config's dtype, row-major [out][in].
 * Per-layer entries are HOST arrays of n_layers device pointers.  td_create copies
 * and repacks every weight into ctx-owned memory; the caller may free its copies once
 * the stream has synchronised after td_create. */
typedef struct {
  const void *tok_emb;                 /* [vocab+1][d]; row `vocab` embeds [MASK] */
  const void *pos_emb;                 /* [B][d]; learned row per block position */
  const void *const *attn_norm;        /* L x [d] RMSNorm gains before attention */
  const void *const *wq;               /* L x [n_heads*head_dim][d] */
  const void *const *wk;               /* L x [n_kv_heads*head_dim][d] */
  const void *const *wv;               /* L x [n_kv_heads*head_dim][d] */
  const void *const *wo;               /* L x [d][n_heads*head_dim] */
  const void *const *mlp_norm;         /* L x [d] RMSNorm gains before the MLP */
  const void *const *w1;               /* L x [d_ff][d]   (u = gelu_erf(h W1^T)) */
  const void *const *w2;               /* L x [d][d_ff]   (x += u W2^T)
                                        * w1 and w2 may both be NULL in td_create for a
                                        * denoiser whose MLP is a mixture of experts
                                        * (td_set_moe before the first step). */
  const void *final_norm;              /* [d] */
  const void *lm_head;                 /* [vocab][d], untied; never predicts [MASK] */
} td_weights;

/* Create a ctx on the current HIP device for the denoiser tower of the two-tower model
 * (poko-everyday.com Nemotron-TwoTower news item, section 技術/ビジネス面: a diffusion
 * tower that reads the context tower's cache).  `stream` is a hipStream_t (NULL = default
 * stream).  Validates cfg/w (TD_EINVAL), allocates the workspace for max_batch and
 * max_prefix_tokens (TD_ENOMEM), packs the weights (TD_EDEVICE on runtime failure,
 * e.g. no device).  On failure *out is NULL and the message is in td_last_error(NULL). */
td_status td_create(const td_config *cfg, const td_weights *w, void *stream, td_ctx **out);

/* Prefix K/V cache layout (per layer, config dtype): pages of TD_KV_PAGE = 32 tokens.
 * Page p of K/V head h is one contiguous block of 32 * head_dim elements:
 *   V, transposed [head_dim][32 tokens]: token slot s, dimension e at
 *       ((p * n_kv_heads + h) * head_dim + e) * 32 + s
 *   K, [head_dim / 32][2][16][32]: slot s, dimension e at
 *       (p * n_kv_heads + h) * 32 * head_dim + ((e / 32) * 2 + (s / 4) % 2) * 512
 *       + ((s / 8) * 4 + s % 4) * 32 + e % 32
 *     (keys grouped by halves of the page in the row order of the attention kernel's
 *     matrix-core operand, so every operand load is one contiguous KiB).
 * Sequence i owns ceil(P_i / 32) consecutive pages starting at page
 * sum_{j<i} ceil(P_j / 32); its token t is in slot t % 32 of its page t / 32.  Slots
 * past P_i in its last page are never used (they may hold anything). */
#define TD_KV_PAGE 32

/* Bind the frozen context tower's prefix K/V for a batch of n_seqs sequences.
 * prefix_offsets_host[n_seqs+1]: P_i = off[i+1] - off[i] is sequence i's prefix length;
 * off[0] == 0, non-decreasing, off[n] <= max_prefix_tokens; a prefix may be empty.
 * k_cache_host / v_cache_host: HOST arrays of n_layers DEVICE pointers, layer l of the
 * context tower feeding denoiser layer l, each holding sum_i ceil(P_i / 32) pages in the
 * layout above.  The caches are BORROWED: they must stay valid and unchanged until the
 * next td_set_prefix or td_destroy.  Builds the split-K work list (host) and may grow
 * the ctx's attention workspace. */
td_status td_set_prefix(td_ctx *ctx, int32_t n_seqs, const int64_t *prefix_offsets_host,
                        const void *const *k_cache_host, const void *const *v_cache_host);

/* Bind caches with room to grow (multi-block generation): sequence i holds
 * lengths_host[i] tokens in page_capacity_host[i] reserved pages (32 tokens each,
 * lengths_host[i] <= 32 * page_capacity_host[i]); its pages start after the reserved
 * pages of sequences 0..i-1, in the layout above.  td_set_prefix is this call with no
 * room (page_capacity = ceil(length / 32)).  Same ownership, errors and workspace
 * growth as td_set_prefix. */
td_status td_bind_cache(td_ctx *ctx, int32_t n_seqs, const int64_t *lengths_host, const int64_t *page_capacity_host,
                        const void *const *k_cache_host, const void *const *v_cache_host);

/* The frozen context tower that writes the cache: the causal tower whose cached K/V the
 * denoiser reads (poko-everyday.com Nemotron-TwoTower news item, section 技術/ビジネス面;
 * dzen.guru, section "Что нового": frozen).  Same shapes and storage dtype as the
 * denoiser; tok_emb [vocab+1][d] and every per-layer pointer are read, pos_emb is
 * ignored (may be NULL), final_norm [d] and lm_head [vocab][d] are optional (both or
 * neither; needed by td_ar_step).  The tower has no position table:
 * its causal mask orders the tokens.  Device pointers, copied and packed into the ctx
 * (the caller may free them afterwards); a later call replaces the tower.
 * Errors: TD_EINVAL for a NULL pointer, TD_ENOMEM. */
td_status td_set_context_tower(td_ctx *ctx, const td_weights *w);

/* One step of AR decoding with the context tower (dzen.guru, section "Что нового": the
 * classic autoregressive mode of the same model; read as the context tower used as an AR
 * model with a final norm and LM head of its own, given to td_set_context_tower):
 * tokens [n] in/out.  In: each sequence's current token (a vocabulary id).  The full
 * tower runs over it, attending to the sequence's cached prefix and itself; its K/V of
 * every layer are appended to the caches (as td_append_block does for a block of one),
 * the bound lengths advance by 1, and tokens receives the prediction: the lowest id of
 * the largest logit (greedy).  Needs a ctx created with block_size 1, a context tower
 * with final_norm and lm_head, and a binding with room for one more token per sequence;
 * otherwise TD_EINVAL and nothing is enqueued.  Returns without waiting, like
 * td_append_block (the same work-list growth and rebuild rule, for one token). */
td_status td_ar_step(td_ctx *ctx, int32_t *tokens);

/* Append a committed block to the prefix (the loop of multi-block generation): run the
 * context tower over tokens [n][B] (committed vocabulary ids, e.g. the output of
 * td_generate_block) -- every block query attends to its sequence's whole cached prefix
 * and causally to the block's earlier positions -- and write each layer's K/V of the B
 * tokens into that layer's cache at positions length .. length+B-1 (bf16 towers round
 * to nearest even), then advance every bound length by B and rebuild the work lists.
 * The next td_generate_block then continues after the appended block.  Needs
 * td_set_context_tower and a binding with room for B more tokens per sequence
 * (td_bind_cache); otherwise TD_EINVAL and nothing is enqueued.  Returns without waiting:
 * each (sequence, K/V head)'s last split-K item of the prefix is extended on the device.
 * Only when such an item would exceed twice the binding's chunk size (or a pair has no
 * prefix item to extend) are the work lists rebuilt on the host, which waits for the
 * stream. */
td_status td_append_block(td_ctx *ctx, const int32_t *tokens);

/* Mixture-of-experts MLP of the denoiser (dzen.guru, section "Что нового": the tower's
 * MoE layers activate 6 of 128 experts plus 2 shared ones per token).  Readings: a
 * router row per expert scores the normed MLP input h2 (the same RMSNorm as the dense
 * MLP); each token takes the top_k experts of largest fp32 score (lowest expert id on
 * ties) with gates = softmax over the chosen scores; every expert, routed or shared, is
 * an ungated GELU MLP of width d_expert; shared experts apply to every token with weight
 * 1:  x += sum_j gate_j * gelu(h2 W1_{e_j}^T) W2_{e_j}^T + sum_s gelu(h2 S1_s^T) S2_s^T.
 * Supported: 1 <= n_experts <= 256, 1 <= top_k <= min(8, n_experts), 0 <= n_shared <= 4,
 * d_expert a positive multiple of 64. */
typedef struct {
  int32_t n_experts, top_k, n_shared, d_expert;
} td_moe_config;

/* Expert weights, DEVICE pointers in the config's dtype; every entry is a HOST array of
 * n_layers device pointers.  Experts of one layer are contiguous: expert e of w1 starts
 * at element e * d_expert * d, of w2 at e * d * d_expert. */
typedef struct {
  const void *const *router;      /* L x [n_experts][d] */
  const void *const *w1;          /* L x [n_experts][d_expert][d] */
  const void *const *w2;          /* L x [n_experts][d][d_expert] */
  const void *const *shared_w1;   /* L x [n_shared][d_expert][d]; NULL when n_shared == 0 */
  const void *const *shared_w2;   /* L x [n_shared][d][d_expert]; NULL when n_shared == 0 */
} td_moe_weights;

/* Replace the MLP of every denoiser layer with the mixture of experts above (a later
 * call replaces it again).  The weights are copied and packed into the ctx (the caller
 * may free them once the stream has synchronised); the workspace for max_batch rows is
 * allocated here.  The context tower keeps its dense MLP.  Routing, the expert
 * products and their gated sum all run on the device inside every later step.
 * Errors: TD_EINVAL (NULL pointer, shape outside the supported ranges), TD_EUNSUPPORTED
 * ((n_experts + n_shared) * max(d_expert, d_model) beyond 2^31 - 1), TD_ENOMEM. */
td_status td_set_moe(td_ctx *ctx, const td_moe_config *cfg, const td_moe_weights *w);

/* Expert counters of the MoE layers since the previous call (then reset): the number of
 * expert-layer launches that ran (a layer of a step whose block was not yet adopted) and
 * the sum over them of the distinct experts, routed plus shared, that held at least one
 * token: the expert weights read per launch are active / launches experts' W1 and W2.
 * With more than one sequence bound, the rows of a sequence whose block is already
 * adopted are not routed (they are not read again) and count for no expert.
 * Waits for the stream.  Errors: TD_EINVAL (no MoE set, NULL pointer). */
td_status td_moe_stats(td_ctx *ctx, int64_t *launches_host, int64_t *active_experts_host);

/* One denoising step over the bound batch: one forward pass of the denoiser over every
 * position of the block, the confidence and prediction of each masked position, and the
 * adoption of those at or above gamma (the single most confident one if none is); the
 * rest stay [MASK] (PredNext "人工知能は拡散言語モデルの夢を見るか？", section
 * 拡散言語モデルで推論するには, steps 2-4).  A finished sequence (no masked position)
 * is left unchanged.
 *  tokens     int32 [n][B] in/out: a token id, or vocab ([MASK]) exactly where
 *             committed == 0.
 *  committed  uint8 [n][B] in/out.
 *  inv_temp   fp32 [n][B] per-position logit inverse temperature, or NULL (all 1).
 *  gamma      adoption threshold (finite; <= 0 adopts every masked position, > 1 adopts
 *             exactly one per sequence with a masked position).
 *  newly_committed  uint8 [n][B] or NULL: 1 where this step adopted the position.
 *  conf_out   fp32 [n][B] or NULL: confidence of each position masked on entry
 *             (unchanged elsewhere).
 *  argmax_out int32 [n][B] or NULL: prediction of each position masked on entry.
 *  logits_out fp32 [n][B][vocab] or NULL: debug capture of the raw logits (before the
 *             inverse temperature) of positions masked on entry. */
td_status td_denoise_step(td_ctx *ctx, int32_t *tokens, uint8_t *committed, const float *inv_temp,
                          float gamma, uint8_t *newly_committed, float *conf_out, int32_t *argmax_out,
                          float *logits_out);

/* Allocation-free step, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): td_denoise_step,
 * same arguments and results, whose partial results -- the vocabulary statistics of
 * every (row, column group), the per-row confidences and predictions, the attention
 * items' partial states and the K-split partial products -- live in a file-scope device
 * array of TD_NOALLOC_SCRATCH_MB MiB instead of buffers of the ctx.  The call makes no
 * hipMalloc, hipFree or other allocating call (profiling brackets are not recorded by
 * it).  Each device holds one such array, from the first td_create on it until the
 * process ends; every call on a device uses that device's array and leaves its contents
 * behind (each step writes every part it reads first), so calls that overlap on one GPU
 * -- ctxs on different streams -- race.  Errors: as td_denoise_step, and TD_EINVAL when
 * the bound batch needs more than the array holds (about 12 B per row and vocabulary
 * column group, plus (head_dim + 2) * 4 B per attention query row and split-K item, plus
 * the K-split partials). */
#define TD_NOALLOC_SCRATCH_MB 64
td_status td_denoise_step_noalloc(td_ctx *ctx, int32_t *tokens, uint8_t *committed, const float *inv_temp,
                                  float gamma, uint8_t *newly_committed, float *conf_out, int32_t *argmax_out,
                                  float *logits_out);

/* The whole block loop on the device (PredNext, section 拡散言語モデルで推論するには,
 * steps 1-5: start from an all-[MASK] block and repeat the step until no [MASK] is left;
 * dzen.guru, section "Как попробовать?": blocks of 16 at threshold 0.8), with no host
 * round-trip at the default issue window 0 (td_set_issue_window; W > 0 paces it from the
 * host polling a pinned progress word): sets tokens to [MASK]
 * and committed to 0, then runs at most B steps; each sequence's loop ends when its
 * block is fully committed (a finished sequence is left unchanged).
 *  steps        int32 [n] or NULL: steps in which the sequence still had a masked position.
 *  commit_step  int8 [n][B] or NULL: step index at which each position was adopted. */
td_status td_generate_block(td_ctx *ctx, int32_t *tokens, uint8_t *committed, const float *inv_temp,
                            float gamma, int32_t *steps, int8_t *commit_step);

/* Issue window of td_generate_block.  0 (the default): the call enqueues all B steps and
 * returns at once; steps after the batch is adopted still launch and return on the
 * device's loop-exit flag (a few microseconds per launch).  steps_ahead = W > 0: the call
 * enqueues step s only once the device has finished step s - W, and enqueues no step
 * once the device reports the whole batch adopted; it then returns when the last step
 * it needs is enqueued, close to the end of the block.  The device writes its progress
 * to a word of coherent pinned host memory (allocated here, owned by the ctx) that the
 * calling thread polls; results are identical for every W.  If the device reports
 * nothing for a second (e.g. the stream waits on an event the caller records later),
 * the call enqueues the remaining steps at once.  W = 2 keeps one step queued behind the
 * running one.  Errors: TD_EINVAL (steps_ahead < 0), TD_ENOMEM. */
td_status td_set_issue_window(td_ctx *ctx, int32_t steps_ahead);

/* Adoption rules for td_set_commit_rule. */
typedef enum {
  TD_RULE_THRESHOLD = 0,     /* conf >= gamma, plus the min_adopt most confident */
  TD_RULE_LEFT_TO_RIGHT = 1  /* the lowest masked position, one per step */
} td_commit_rule;

/* Choose the adoption rule of every later td_denoise_step / td_generate_block on this
 * ctx (the default is TD_RULE_THRESHOLD with min_adopt 1, the rule described at the top).
 *  TD_RULE_THRESHOLD: adopt the masked positions whose confidence is at least gamma,
 *    together with the min_adopt most confident masked positions (lowest position on
 *    ties; every masked position if fewer remain).  PredNext, section
 *    拡散言語モデルで推論するには, step 3 names forcing the top few positions as an
 *    alternative to the threshold; min_adopt = 1 is the single-position fallback, and
 *    gamma > 1 with min_adopt = k adopts exactly k per step.
 *  TD_RULE_LEFT_TO_RIGHT: adopt only the lowest masked position of each sequence (its
 *    prediction), one per step, B steps per block: the mock-AR mode of dzen.guru, section
 *    "Что нового" (one token per step through the diffusion tower), read as
 *    autoregressive order.  gamma and min_adopt are ignored.
 *  min_adopt: 1 .. block_size (TD_RULE_THRESHOLD); any value for TD_RULE_LEFT_TO_RIGHT.
 * Errors: TD_EINVAL for an unknown rule or min_adopt outside 1 .. block_size. */
td_status td_set_commit_rule(td_ctx *ctx, int32_t rule, int32_t min_adopt);

/* Debug hook: run the layer-`layer` attention (prefix split-K + in-block keys + merge)
 * on caller-provided projections qkv [n*B][(n_heads + 2*n_kv_heads)*head_dim] (q, then
 * k, then v of the block; fp32, the precision the step carries activations in) and
 * write o [n*B][n_heads*head_dim] (fp32). */
td_status td_debug_attention(td_ctx *ctx, int32_t layer, const void *qkv, void *o);

/* Wait for the ctx's stream; report asynchronous device errors and device-side input
 * errors recorded since the last td_sync. */
td_status td_sync(td_ctx *ctx);

/* Kernel classes for td_profile_begin (bit k of its mask brackets class k). */
typedef enum {
  TD_PROF_OFF = 0,
  TD_PROF_LMHEAD = 1,     /* LM head + fused vocab statistics (one launch per step) */
  TD_PROF_GEMM = 2,       /* each layer projection, with its K-split reduction when split: 4 L per
                           * step (tag sub 0 fused QKV, 1 output, 2 MLP up, 3 MLP down, 4 MoE router) */
  TD_PROF_ATTENTION = 3,  /* the split-K attention items (prefix pages and block keys), L per step */
  TD_PROF_STEP = 4,       /* one whole step, embedding to commit */
  TD_PROF_MOE = 5,        /* the expert up (sub 0) and down (sub 1) projections, 2 L per step */
  TD_PROF_ATTN_MERGE = 6, /* the merge of the attention partials, L per step */
  TD_PROF_COMMIT = 7,     /* vocabulary merge + adoption rule (one or two launches per step) */
  TD_PROF_EMBED = 8,      /* the embedding (one launch per step) */
  TD_PROF_KINDS = 9
} td_prof_kind;

/* Profiling: from now on bracket every launch of the kernel classes in kinds_mask
 * (bit k = class k; 0 stops recording) with a pair of HIP events on the ctx's stream, at
 * most 65536 brackets (later launches are not recorded).  Errors: TD_EINVAL for bits
 * past TD_PROF_KINDS. */
td_status td_profile_begin(td_ctx *ctx, int32_t kinds_mask);

/* Bracket the per-layer classes (projections, attention, merge, experts) on one layer
 * only (layer in [0, n_layers)), or on every layer (-1, the default): fewer events on the
 * stream where they would perturb short launches.  Errors: TD_EINVAL (layer out of range,
 * NULL ctx). */
td_status td_profile_layer(td_ctx *ctx, int32_t layer);

/* Wait for the stream, write the duration in ms of each bracketed launch, in launch order,
 * to ms_out_host[0 .. min(count, max)) and its tag (class | sub << 8 | layer << 16) to
 * tags_out_host (either may be NULL), and return the number recorded (or -1 on error);
 * then clear the record and stop recording.  Launches skipped on the device because the
 * block was already committed are included (they take a few microseconds). */
int32_t td_profile_end(td_ctx *ctx, float *ms_out_host, int32_t *tags_out_host, int32_t max);

/* Number of kernels one td_denoise_step enqueues on the bound batch (for profiling and
 * launch accounting; before a binding, for one sequence with the creation-time plans). */
int32_t td_kernels_per_step(const td_ctx *ctx);

/* Measurement helper, not part of the step: the chip's own ceilings, to report achieved
 * rates against measured as well as published peaks.  On the current device and the
 * given stream (a hipStream_t, NULL = default), waiting for it; best of five launches
 * each.
 *  hbm_read_gbs      a read stream over buf: every 16-byte word read once (streaming loads);
 *  copy_gbs          a copy of the first half of buf into the second, bytes read + written;
 *  mfma_bf16_tflops  loops of bf16 matrix-core products (16x16x32 and 32x32x16, the better
 *                    of the two), operands in registers, no memory traffic, four waves per
 *                    SIMD.
 * buf: DEVICE scratch of `bytes` bytes (>= 68 MiB, 16-byte aligned; use well over the
 * 256 MiB last-level cache for an HBM figure), overwritten.  Errors: TD_EINVAL (NULL
 * pointer, buffer too small or misaligned), TD_EDEVICE (a runtime error). */
td_status td_measure_peaks(void *buf, int64_t bytes, void *stream, double *hbm_read_gbs, double *copy_gbs,
                           double *mfma_bf16_tflops);

void td_destroy(td_ctx *ctx);                  /* NULL-safe; waits for the stream */
const char *td_last_error(const td_ctx *ctx);  /* ctx == NULL: this thread's last create error */
const char *td_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TD_H */
