// gpu_clock.hip -- shader-clock sampling (include/gpu_clock.h): a measurement aid.
//
// One wave reads the shader core's cycle counter (s_memtime) and the constant-rate
// wall-clock counter (s_memrealtime); the ratio of their increments is the shader
// clock over that interval.  The sampler sleeps between pairs, so beside a running
// kernel it costs one wave slot and almost no issue cycles.

#include "../../include/attn.h"
#include "../../include/gpu_clock.h"
#include "common.hpp"

namespace {

// Agent-scope accesses: the phase word is written by one kernel and read by the sampler
// while both run, possibly on different XCDs, so neither may stop at a non-coherent cache.
__device__ __forceinline__ int load_phase(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(64) void clock_sampler_kernel(uint64_t* out, const int* phase,
                                                           int stop_value, int max_samples,
                                                           uint64_t interval, uint64_t duration) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  int n = 0;
  // every iteration either stops (stop value seen, max_samples or duration reached) or
  // waits for the next interval boundary, which the monotonic wall clock always reaches
  while (n < max_samples) {
    const uint64_t rt = __builtin_amdgcn_s_memrealtime();
    const uint64_t ct = __builtin_amdgcn_s_memtime();
    const int ph = load_phase(phase);
    if (threadIdx.x == 0) {
      out[1 + 3 * n] = rt;
      out[2 + 3 * n] = ct;
      out[3 + 3 * n] = (uint64_t)(int64_t)ph;
    }
    ++n;
    if (ph == stop_value || rt - t0 >= duration) break;
    const uint64_t next = t0 + (uint64_t)n * interval;
    while (__builtin_amdgcn_s_memrealtime() < next) __builtin_amdgcn_s_sleep(32);
  }
  if (threadIdx.x == 0) out[0] = (uint64_t)n;
}

__global__ __launch_bounds__(64) void clock_mark_kernel(int* phase, int value) {
  if (threadIdx.x == 0)
    __hip_atomic_store(phase, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

extern "C" {

int attn_clock_sampler(uint64_t* samples, const int* phase, int stop_value, int max_samples,
                       uint64_t interval_ticks, uint64_t duration_ticks, void* stream) {
  if (!samples || !phase) return ATTN_ERR_NULL;
  if ((uintptr_t)samples % 8 || (uintptr_t)phase % 4) return ATTN_ERR_ALIGN;
  if (max_samples < 1 || max_samples > (1 << 20) || interval_ticks == 0 || duration_ticks == 0)
    return ATTN_ERR_SHAPE;
  clock_sampler_kernel<<<1, 64, 0, (hipStream_t)stream>>>(samples, phase, stop_value,
                                                          max_samples, interval_ticks,
                                                          duration_ticks);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_clock_mark(int* phase, int value, void* stream) {
  if (!phase) return ATTN_ERR_NULL;
  if ((uintptr_t)phase % 4) return ATTN_ERR_ALIGN;
  clock_mark_kernel<<<1, 64, 0, (hipStream_t)stream>>>(phase, value);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int64_t attn_clock_wall_hz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return ATTN_ERR_HIP;
  return (int64_t)khz * 1000;
}

}  // extern "C"
