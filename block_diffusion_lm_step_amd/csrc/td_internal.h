// Internal interface between the host runtime (td_api.cpp) and the allocation-free step
// (td_noalloc.hip); not part of the C ABI.
#pragma once
#include <stddef.h>

#include "../../include/td.h"
#include "td_kernels.h"

namespace td {

// Partial-result buffers of one step (see carve_step_scratch).
struct StepScratch {
  VStat *vpart;
  float *conf_row;
  int *arg_row;
  float *att_o, *att_ml;
  float *part;
};

size_t carve_step_scratch(const td_ctx *c, char *base, size_t bytes, StepScratch *out);
td_status denoise_step_on_scratch(td_ctx *c, int32_t *tokens, uint8_t *committed, const float *inv_temp, float gamma,
                                  uint8_t *newly, float *conf_out, int32_t *argmax_out, float *logits_out,
                                  char *scratch, size_t bytes);
// Resolves, once per device and with that device current, the device address of the
// allocation-free step's scratch array (td_noalloc.hip); called by td_create.
hipError_t noalloc_scratch_init();
int ctx_device(const td_ctx *c);

}  // namespace td
