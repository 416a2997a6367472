// Shader-clock probe for the measurements: one wave spins on the device's constant-rate wall clock
// and counts the shader-clock cycles that pass meanwhile. Run right after a timed region, it reads
// the clock the part settled at under that load (power management acts on millisecond scales).
#include "internal.h"

namespace fp8g {
namespace kernels {

__global__ void __launch_bounds__(64) clock_probe_kernel(unsigned long long* out, unsigned long long spin_ticks) {
  if (threadIdx.x != 0) return;
  const unsigned long long w0 = wall_clock64();
  const unsigned long long c0 = clock64();
  unsigned long long w = w0;
  // bounded: ends after spin_ticks of wall clock, or after 2^24 reads whatever the clock does
  for (int i = 0; i < (1 << 24) && w - w0 < spin_ticks; ++i) w = wall_clock64();
  const unsigned long long c1 = clock64();
  out[0] = c1 - c0;
  out[1] = w - w0;
}

}  // namespace kernels

hipError_t launch_clock_probe(unsigned long long* out, unsigned long long spin_ticks, hipStream_t stream) {
  hipLaunchKernelGGL(kernels::clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, spin_ticks);
  return hipGetLastError();
}

}  // namespace fp8g
