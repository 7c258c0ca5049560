// The chip's own ceilings, measured on it: a read stream over device memory, a copy, and
// loops of bf16 matrix-core products with no memory traffic.  Used to report the rates of
// the step's kernels against measured as well as published peaks; not part of the step.
#include "../../include/td.h"
#include "td_device.h"

#include <hip/hip_runtime.h>

#include <algorithm>

namespace {

constexpr int PEAK_GRID = 2048, PEAK_THREADS = 256;

// Every 16-byte word of src[0 .. n16) read once with streaming loads, four in flight per
// thread, folded with XOR so no load is dead; one word per thread to sink.
__global__ __launch_bounds__(PEAK_THREADS) void read_stream_kernel(const u32x4_t *src, size_t n16, u32x4_t *sink) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * PEAK_THREADS;
  size_t i = (size_t)blockIdx.x * PEAK_THREADS + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = acc;
}

__global__ __launch_bounds__(PEAK_THREADS) void copy_kernel(const u32x4_t *src, u32x4_t *dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * PEAK_THREADS;
  size_t i = (size_t)blockIdx.x * PEAK_THREADS + threadIdx.x;
  for (; i + stride < n16; i += 2 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
  }
  if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// CHAINS independent accumulators per wave, operands in registers, derived from the
// thread index so nothing folds at compile time.  Two chains: with four 16x16x32 chains
// the compiler moves accumulator registers inside the loop (measured: 1.34 PFLOP/s
// against 2.0-2.2 with one or two chains at three or four waves per SIMD).
template <int CHAINS>
__global__ __launch_bounds__(PEAK_THREADS) void mfma16_loop_kernel(int iters, float *sink) {
  Frag<bf16_t> a, b;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (float)((threadIdx.x + j) & 7) * 0.125f;
  a.set8(v);
  b.set8(v);
  f32x4_t acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = zero4();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.vec(), b.vec(), acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = s;
}

template <int CHAINS>
__global__ __launch_bounds__(PEAK_THREADS) void mfma32_loop_kernel(int iters, float *sink) {
  Frag<bf16_t> a, b;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (float)((threadIdx.x + j) & 7) * 0.125f;
  a.set8(v);
  b.set8(v);
  f32x16_t acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.vec(), b.vec(), acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = s;
}

// Best duration in ms of `reps` launches made by `launch`, each bracketed by events.
template <typename F>
hipError_t best_ms(hipStream_t s, int reps, F &&launch, float *out) {
  hipEvent_t a, b;
  hipError_t e = hipEventCreate(&a);
  if (e != hipSuccess) return e;
  e = hipEventCreate(&b);
  if (e != hipSuccess) {
    (void)hipEventDestroy(a);
    return e;
  }
  float best = 1e30f;
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    e = hipEventRecord(a, s);
    if (e == hipSuccess) {
      launch();
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(b, s);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e == hipSuccess) best = std::min(best, ms);
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  *out = best;
  return e;
}

}  // namespace

extern "C" td_status td_measure_peaks(void *buf, int64_t bytes, void *stream, double *hbm_read_gbs, double *copy_gbs,
                                      double *mfma_bf16_tflops) {
  const int64_t sink_bytes = (int64_t)PEAK_GRID * PEAK_THREADS * 16;
  if (!buf || !hbm_read_gbs || !copy_gbs || !mfma_bf16_tflops) return TD_EINVAL;
  if (bytes < ((int64_t)64 << 20) + sink_bytes || (reinterpret_cast<uintptr_t>(buf) & 15)) return TD_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  char *base = static_cast<char *>(buf);
  u32x4_t *sink = reinterpret_cast<u32x4_t *>(base + bytes - sink_bytes);
  const size_t n16 = (size_t)((bytes - sink_bytes) / 16);
  const int reps = 5;
  float ms = 0.f;
  hipError_t e;

  e = best_ms(s, reps, [&] {
    hipLaunchKernelGGL(read_stream_kernel, dim3(PEAK_GRID), dim3(PEAK_THREADS), 0, s,
                       reinterpret_cast<const u32x4_t *>(base), n16, sink);
  }, &ms);
  if (e != hipSuccess) return TD_EDEVICE;
  *hbm_read_gbs = (double)n16 * 16.0 / (ms * 1e-3) / 1e9;

  const size_t half = n16 / 2;
  e = best_ms(s, reps, [&] {
    hipLaunchKernelGGL(copy_kernel, dim3(PEAK_GRID), dim3(PEAK_THREADS), 0, s, reinterpret_cast<const u32x4_t *>(base),
                       reinterpret_cast<u32x4_t *>(base) + half, half);
  }, &ms);
  if (e != hipSuccess) return TD_EDEVICE;
  *copy_gbs = (double)half * 16.0 * 2.0 / (ms * 1e-3) / 1e9;   // bytes read + bytes written

  // Four waves per SIMD (256 CUs x 4 SIMDs), each with independent accumulator chains.
  const int grid = 1024, iters = 4096;
  float *fsink = reinterpret_cast<float *>(sink);
  double best = 0.0;
  e = best_ms(s, reps, [&] {
    hipLaunchKernelGGL(mfma16_loop_kernel<2>, dim3(grid), dim3(PEAK_THREADS), 0, s, iters, fsink);
  }, &ms);
  if (e != hipSuccess) return TD_EDEVICE;
  best = std::max(best, (double)grid * (PEAK_THREADS / 64) * iters * 2 * (2.0 * 16 * 16 * 32) / (ms * 1e-3) / 1e12);
  e = best_ms(s, reps, [&] {
    hipLaunchKernelGGL(mfma32_loop_kernel<2>, dim3(grid), dim3(PEAK_THREADS), 0, s, iters, fsink);
  }, &ms);
  if (e != hipSuccess) return TD_EDEVICE;
  best = std::max(best, (double)grid * (PEAK_THREADS / 64) * iters * 2 * (2.0 * 32 * 32 * 16) / (ms * 1e-3) / 1e12);
  *mfma_bf16_tflops = best;
  return TD_OK;
}
