// Shader-clock probe for the benchmark (not part of the attention library):
// one wave reads the shader cycle counter (s_memtime) and the constant-rate
// wall clock (s_memrealtime) at the start and the end of a busy interval of
// a given wall-clock length, so that cycles / seconds is the clock of the CU
// it ran on while whatever else was on the GPU ran beside it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out,
                                                         unsigned long long wall_ticks) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long w = w0;
  // bounded: the wall clock advances on its own, and the iteration cap
  // ends the loop even if it did not
  for (int i = 0; i < (1 << 26) && w - w0 < wall_ticks; ++i) {
    __builtin_amdgcn_s_sleep(1);
    w = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = w - w0;
  }
}

}  // namespace

// out: 2 device uint64 (shader cycles, wall-clock ticks of the interval);
// wall_ticks: the interval in wall-clock ticks.  Returns a hipError_t.
extern "C" int ra_clock_probe(unsigned long long* out, unsigned long long wall_ticks, void* stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                     out, wall_ticks);
  return (int)hipGetLastError();
}

// Wall-clock rate in kHz of the current device (0 on failure).
extern "C" int ra_wall_clock_khz() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}
