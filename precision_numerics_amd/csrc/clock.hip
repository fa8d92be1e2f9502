// Shader-clock sampler, a measurement aid for the kernels' timings.
//
// gfx950 counts shader clocks in a 64-bit counter (s_memtime) and real time
// in a 100 MHz counter (s_memrealtime).  The shader-clock counters of
// different compute units are not synchronised with each other (measured:
// they differ by up to ~10^8 cycles inside one XCD), so every sample
// records where it was taken (XCD id and the HW_ID register, which holds
// the shader engine, shader array and CU): two samples around a timed
// region, compared on the same CU, give the average shader clock there,
//     f = 100 MHz * (memtime_1 - memtime_0) / (realtime_1 - realtime_0).
// The power controller lowers the clock under sustained matrix work, which
// is what this measures.
#include "device.hpp"
#include "launch.hpp"

namespace pn {
namespace {

__global__ __launch_bounds__(64) void clock_sample_kernel(uint64_t* out) {
  uint32_t xcc, hwid;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hwid));
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    // location: XCD id, then HW_ID bits 8..15 (CU, shader array, engine)
    out[3 * blockIdx.x + 0] = (uint64_t)xcc << 8 | ((hwid >> 8) & 0xffu);
    out[3 * blockIdx.x + 1] = t;
    out[3 * blockIdx.x + 2] = r;
  }
}

}  // namespace

hipError_t launch_clock_sample(uint64_t* out, int slots, hipStream_t st) {
  hipLaunchKernelGGL(clock_sample_kernel, dim3(slots), dim3(64), 0, st, out);
  return hipGetLastError();
}

}  // namespace pn
