// Symmetric per-row int8 quantisation of fp32 rows (the int8 Q/K input of
// "INT-FlashAttention", abstract; the per-row absmax/127 scale is the
// library's reading, since that abstract stops before the scheme):
//   scale = fp32(absmax / 127) (IEEE division; 1 when that is 0)
//   code  = clamp(round_half_even(fp32(x / scale)), -127, 127)
// One wave64 per row; HBM-bound (4 bytes in, 1 byte out per element).
#include "device.hpp"
#include "launch.hpp"

namespace pn {
namespace {

__global__ __launch_bounds__(256) void quantize_kernel(const float* x, int64_t rows, int d,
                                                      int8_t* codes, float* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + r * d;
  float am = 0.f;
  for (int i = lane; i < d; i += 64) am = fmaxf(am, fabsf(xr[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  float sc = __fdiv_rn(am, 127.0f);
  if (sc == 0.f) sc = 1.0f;
  int8_t* cr = codes + r * d;
  for (int i = lane; i < d; i += 64) {
    const float q = fminf(fmaxf(rintf(__fdiv_rn(xr[i], sc)), -127.f), 127.f);
    cr[i] = (int8_t)(int)q;
  }
  if (lane == 0) scales[r] = sc;
}

// The same per-row scheme with the E4M3 fp8 format ("FP8 Formats for Deep
// Learning", in the reference list of "Why Low-Precision Transformer
// Training Fails"): scale = fp32(absmax / 448) (1 when that is 0),
// code = E4M3(fp32(x / scale)), nearest with ties to even.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const float* x, int64_t rows, int d,
                                                          uint8_t* codes, float* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* xr = x + r * d;
  float am = 0.f;
  for (int i = lane; i < d; i += 64) am = fmaxf(am, fabsf(xr[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  float sc = __fdiv_rn(am, 448.0f);
  if (sc == 0.f) sc = 1.0f;
  uint8_t* cr = codes + r * d;
  for (int i = lane; i < d; i += 64) cr[i] = f32_to_e4m3(__fdiv_rn(xr[i], sc));
  if (lane == 0) scales[r] = sc;
}

}  // namespace

hipError_t launch_quantize_fp8(const float* x, int64_t rows, int64_t d, uint8_t* codes,
                               float* scales, hipStream_t st) {
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, rows,
                     (int)d, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int64_t rows, int64_t d, int8_t* codes,
                           float* scales, hipStream_t st) {
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, (int)d,
                     codes, scales);
  return hipGetLastError();
}

}  // namespace pn
