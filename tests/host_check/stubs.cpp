// Host-only stand-ins for the kernel launchers and planning helpers of the gfx950 kernel
// files, so that the host runtime (td_api.cpp) links into a sanitizer build without device
// code.  Every launcher reports an error: the harness only exercises paths that validate
// arguments and fail before anything would run on a device.
#include "../../block_diffusion_lm_step_amd/csrc/td_internal.h"
#include "../../block_diffusion_lm_step_amd/csrc/td_kernels.h"

namespace td {

hipError_t launch_pack_weight(int, const void *, void *, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm(int, int, bool, const GemmArgs &, hipStream_t) { return hipErrorNoDevice; }
int lmhead_slices(int N, int nt, int nw) { return N / (16 * nt * nw); }
bool gemm_tile_supported(int, int, int, int) { return false; }
int gemm_tile_slices(int N) { return N / 128; }
int gemm_tile_splits(int, int, int) { return 1; }
hipError_t launch_gemm_tile(int, bool, const GemmArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_split_reduce(int, bool, const GemmArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm_wk(int, int, bool, const GemmArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attention(int, const AttnArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prep(const int *, const uint8_t *, int, int, int, StepState, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_init_block(int *, uint8_t *, int8_t *, int *, int, int, int, StepState, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_embed(int, const int *, const void *, const void *, const void *, float *, float *, void *, int, int,
                        int, int, StepState, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_merge_commit(const CommitArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_append(int, const float *, int, int, int, int, void *, void *, const int *, const int *, int, int,
                            hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_moe_route(const MoeRoute &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_moe_gemm(int, bool, const MoeGemm &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_moe_combine(int, const MoeCombine &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_advance(AttnItem *, const int *, int, int *, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch_init() { return hipErrorNoDevice; }

}  // namespace td
