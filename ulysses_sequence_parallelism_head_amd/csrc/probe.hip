// probe.hip -- shader-clock sampler for measurements.
//
// The matrix-core peak a kernel is compared with scales with the engine
// clock, and under sustained matrix work the clock runs below its 2.4 GHz
// maximum.  This kernel, one wave on a second stream beside the kernel being
// measured, reads the shader cycle counter against the constant-rate
// real-time counter at fixed real-time intervals, so the clock the
// measured kernel ran at is the ratio of the two counters' increments.  It
// needs a handful of registers and no LDS, so it fits beside the attention
// kernels' waves on a CU.
//
// Every wait ends: the spin stops at its real-time target or after a fixed
// number of polls, whichever comes first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace ulysses {

namespace {

constexpr uint32_t kMaxPolls = 1u << 24;   // per sample; far beyond any interval asked for

__global__ __launch_bounds__(64, 1) void clock_probe_kernel(uint64_t* out, int32_t samples, uint64_t interval) {
  const int lane = threadIdx.x;
  const uint64_t start = __builtin_amdgcn_s_memrealtime();
  uint64_t c_prev = __builtin_amdgcn_s_memtime();
  for (int32_t s = 0; s < samples; ++s) {
    const uint64_t target = start + uint64_t(s + 1) * interval;
    uint32_t polls = 0;
    while (__builtin_amdgcn_s_memrealtime() < target && ++polls < kMaxPolls) __builtin_amdgcn_s_sleep(2);
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    const uint64_t c = __builtin_amdgcn_s_memtime();
    // lanes 0 and 1 write the pair (real-time stamp, shader cycles since the
    // previous sample) at different addresses: plain vector stores
    if (lane < 2) out[2 * int64_t(s) + lane] = lane == 0 ? r : c - c_prev;
    c_prev = c;
  }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t* out, int32_t samples, uint32_t interval_us, int32_t* wall_khz,
                              hipStream_t stream) {
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  if (khz <= 0) return hipErrorInvalidValue;
  *wall_khz = khz;
  const uint64_t interval = uint64_t(interval_us) * uint64_t(khz) / 1000u;   // real-time ticks
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, samples, interval > 0 ? interval : 1);
  return hipGetLastError();
}

}  // namespace ulysses
