// Argument validation of the C ABI on the host, for a sanitizer (ASan + UBSan) build of
// the host runtime: every entry point given a NULL ctx or invalid arguments must return
// its error code, write its message, and touch no memory it does not own.  With no device,
// a valid td_create must fail with TD_EDEVICE and leave *out NULL.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/td.h"

static int g_fail = 0, g_checks = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    ++g_checks;                                                      \
    if (!(cond)) {                                                   \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

static td_config base_cfg() {
  td_config c{};
  c.n_layers = 2;
  c.d_model = 256;
  c.n_heads = 4;
  c.n_kv_heads = 4;
  c.head_dim = 64;
  c.d_ff = 1024;
  c.vocab = 4096;
  c.block_size = 16;
  c.max_batch = 1;
  c.max_prefix_tokens = 128;
  c.dtype = TD_F32;
  c.rms_eps = 1e-6f;
  return c;
}

static void expect_create_einval(const td_config &c, const td_weights *w) {
  td_ctx *ctx = reinterpret_cast<td_ctx *>(0x1);
  CHECK(td_create(&c, w, nullptr, &ctx) == TD_EINVAL);
  CHECK(ctx == nullptr);
  CHECK(std::strlen(td_last_error(nullptr)) > 0);
}

int main() {
  CHECK(std::strncmp(td_version(), "td ", 3) == 0);

  // td_create: argument checks
  td_config c = base_cfg();
  td_weights none{};
  CHECK(td_create(&c, &none, nullptr, nullptr) == TD_EINVAL);
  expect_create_einval(c, nullptr);
  expect_create_einval(c, &none);
  CHECK(std::strstr(td_last_error(nullptr), "NULL") != nullptr);
  {
    td_ctx *ctx = nullptr;
    CHECK(td_create(nullptr, &none, nullptr, &ctx) == TD_EINVAL && ctx == nullptr);
  }
  const td_config bad[] = {
      [] { auto x = base_cfg(); x.head_dim = 96; return x; }(),
      [] { auto x = base_cfg(); x.block_size = 12; return x; }(),
      [] { auto x = base_cfg(); x.n_heads = 6; return x; }(),
      [] { auto x = base_cfg(); x.d_model = 100; return x; }(),
      [] { auto x = base_cfg(); x.vocab = 1000; return x; }(),
      [] { auto x = base_cfg(); x.dtype = 7; return x; }(),
      [] { auto x = base_cfg(); x.max_batch = 0; return x; }(),
      [] { auto x = base_cfg(); x.max_batch = 1 << 30; return x; }(),
      [] { auto x = base_cfg(); x.rms_eps = NAN; return x; }(),
      [] { auto x = base_cfg(); x.rms_eps = -1.f; return x; }(),
      [] { auto x = base_cfg(); x.n_layers = 0; return x; }(),
      [] { auto x = base_cfg(); x.max_prefix_tokens = -1; return x; }(),
      [] { auto x = base_cfg(); x.d_ff = 0; return x; }(),
  };
  for (const td_config &b : bad) expect_create_einval(b, &none);

  // A structurally valid config and non-NULL (never dereferenced on the host) weights.
  const void *fake[2] = {reinterpret_cast<void *>(16), reinterpret_cast<void *>(16)};
  td_weights w{};
  w.tok_emb = w.pos_emb = w.final_norm = w.lm_head = fake[0];
  w.attn_norm = w.wq = w.wk = w.wv = w.wo = w.mlp_norm = w.w1 = w.w2 = fake;
  {
    // one per-layer pointer NULL
    const void *holes[2] = {fake[0], nullptr};
    td_weights w2 = w;
    w2.wk = holes;
    expect_create_einval(c, &w2);
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    td_ctx *ctx = reinterpret_cast<td_ctx *>(0x1);
    CHECK(td_create(&c, &w, nullptr, &ctx) == TD_EDEVICE);
    CHECK(ctx == nullptr);
    CHECK(std::strstr(td_last_error(nullptr), "device") != nullptr);
  }

  // Every entry point with a NULL ctx.
  int64_t off[2] = {0, 0};
  CHECK(td_set_prefix(nullptr, 1, off, nullptr, nullptr) == TD_EINVAL);
  CHECK(td_bind_cache(nullptr, 1, off, off, nullptr, nullptr) == TD_EINVAL);
  CHECK(td_set_context_tower(nullptr, &w) == TD_EINVAL);
  CHECK(td_ar_step(nullptr, nullptr) == TD_EINVAL);
  CHECK(td_append_block(nullptr, nullptr) == TD_EINVAL);
  td_moe_config mc{8, 2, 1, 64};
  td_moe_weights mw{};
  CHECK(td_set_moe(nullptr, &mc, &mw) == TD_EINVAL);
  int64_t n = 0, act = 0;
  CHECK(td_moe_stats(nullptr, &n, &act) == TD_EINVAL);
  CHECK(td_denoise_step(nullptr, nullptr, nullptr, nullptr, 0.8f, nullptr, nullptr, nullptr, nullptr) == TD_EINVAL);
  CHECK(td_generate_block(nullptr, nullptr, nullptr, nullptr, 0.8f, nullptr, nullptr) == TD_EINVAL);
  CHECK(td_set_issue_window(nullptr, 2) == TD_EINVAL);
  CHECK(td_set_commit_rule(nullptr, 0, 1) == TD_EINVAL);
  CHECK(td_debug_attention(nullptr, 0, nullptr, nullptr) == TD_EINVAL);
  CHECK(td_sync(nullptr) == TD_EINVAL);
  CHECK(td_profile_begin(nullptr, 1 << TD_PROF_GEMM) == TD_EINVAL);
  CHECK(td_profile_layer(nullptr, 0) == TD_EINVAL);
  float ms[4];
  int32_t tags[4];
  CHECK(td_profile_end(nullptr, ms, tags, 4) == -1);
  CHECK(td_kernels_per_step(nullptr) == -1);
  CHECK(std::strstr(td_last_error(nullptr), "ctx is NULL") != nullptr);
  td_destroy(nullptr);

  std::printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
