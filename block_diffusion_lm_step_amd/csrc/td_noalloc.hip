// The allocation-free step: td_denoise_step with its partial results (vocabulary
// statistics, per-row confidences and predictions, attention partial states, K-split
// partial products) in a file-scope device array instead of buffers the ctx allocates,
// for callers that cannot allocate.  The array is SCRATCH_BYTES on every device the
// library runs on, resolved to a device address once per device by td_create (with that
// device current), and held until the process ends.  Calls on one device share it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/td.h"
#include "td_internal.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)TD_NOALLOC_SCRATCH_MB << 20;
static __device__ __align__(256) char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_scratch[MAX_DEVICES];   // device address of `scratch` on each device (null: not resolved)

}  // namespace

namespace td {

hipError_t noalloc_scratch_init() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev]) return hipSuccess;
  void *ptr = nullptr;
  e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch[dev] = ptr;
  return hipSuccess;
}

}  // namespace td

extern "C" td_status td_denoise_step_noalloc(td_ctx *ctx, int32_t *tokens, uint8_t *committed, const float *inv_temp,
                                             float gamma, uint8_t *newly_committed, float *conf_out,
                                             int32_t *argmax_out, float *logits_out) {
  void *ptr = nullptr;
  if (ctx) {
    const int dev = td::ctx_device(ctx);
    std::lock_guard<std::mutex> lock(g_mu);
    if (dev >= 0 && dev < MAX_DEVICES) ptr = g_scratch[dev];
  }
  // A ctx exists only after td_create resolved the array on its device, so ptr is null
  // only for a NULL ctx (rejected inside with TD_EINVAL).
  return td::denoise_step_on_scratch(ctx, tokens, committed, inv_temp, gamma, newly_committed, conf_out, argmax_out,
                                     logits_out, static_cast<char *>(ptr), ptr ? SCRATCH_BYTES : 0);
}
