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

// Per-tile int8 scales: the n rows of every group (a (batch, head)) are cut
// into tiles of tile_rows rows, the last one ragged; one workgroup per tile
// takes the tile's absmax (first pass), then writes the codes with the
// shared scale and that scale for each of its rows (second pass).
__global__ __launch_bounds__(256) void quantize_tiles_kernel(const float* x, int64_t n, int d,
                                                            int64_t tile_rows, int64_t tiles_per,
                                                            int8_t* codes, float* scales) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int64_t grp = t / tiles_per;
  const int64_t r0 = (t - grp * tiles_per) * tile_rows;
  const int64_t r1 = r0 + tile_rows < n ? r0 + tile_rows : n;
  const int64_t base = (grp * n + r0) * d;
  const int64_t cnt = (r1 - r0) * d;
  float am = 0.f;
  for (int64_t i = threadIdx.x; i < cnt; i += 256) am = fmaxf(am, fabsf(x[base + i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float sc = __fdiv_rn(am, 127.0f);
  if (sc == 0.f) sc = 1.0f;
  for (int64_t i = threadIdx.x; i < cnt; i += 256) {
    const float q = fminf(fmaxf(rintf(__fdiv_rn(x[base + i], sc)), -127.f), 127.f);
    codes[base + i] = (int8_t)(int)q;
  }
  for (int64_t r = r0 + threadIdx.x; r < r1; r += 256) scales[grp * n + r] = sc;
}

// The per-row int8 and E4M3 quantisers for rows of d = 4 * LPR elements:
// LPR lanes per row, one 16-byte load and one 4-byte store per lane, so a
// wave covers 64 / LPR rows.  Same arithmetic per element as the kernels
// above (bit-identical codes and scales).
template <int LPR, bool FP8>
__global__ __launch_bounds__(256) void quantize_vec_kernel(const float* x, int64_t rows,
                                                          void* codes, float* scales) {
  constexpr int d = 4 * LPR;
  const int lane = threadIdx.x & 63;
  const int64_t r = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;
  const int sub = lane % LPR;
  const bool ok = r < rows;
  float4 v = ok ? *(const float4*)(x + r * d + 4 * sub) : make_float4(0.f, 0.f, 0.f, 0.f);
  float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  float sc = __fdiv_rn(am, FP8 ? 448.0f : 127.0f);
  if (sc == 0.f) sc = 1.0f;
  if (!ok) return;
  uint32_t packed;
  if constexpr (FP8) {
    packed = (uint32_t)f32_to_e4m3(__fdiv_rn(v.x, sc)) |
             ((uint32_t)f32_to_e4m3(__fdiv_rn(v.y, sc)) << 8) |
             ((uint32_t)f32_to_e4m3(__fdiv_rn(v.z, sc)) << 16) |
             ((uint32_t)f32_to_e4m3(__fdiv_rn(v.w, sc)) << 24);
  } else {
    auto q = [&](float t) {
      return (uint32_t)(uint8_t)(int8_t)(int)fminf(fmaxf(rintf(__fdiv_rn(t, sc)), -127.f), 127.f);
    };
    packed = q(v.x) | (q(v.y) << 8) | (q(v.z) << 16) | (q(v.w) << 24);
  }
  ((uint32_t*)codes)[(r * d) / 4 + sub] = packed;
  if (sub == 0) scales[r] = sc;
}

template <bool FP8>
bool launch_vec(const float* x, int64_t rows, int64_t d, void* codes, float* scales,
                hipStream_t st) {
  // 16-byte loads and 4-byte stores need aligned rows
  if ((uintptr_t)x % 16 != 0 || (uintptr_t)codes % 4 != 0) return false;
  if (d != 64 && d != 128 && d != 256) return false;
  const int64_t per_block = 4 * (64 / (d / 4));
  const dim3 grid((unsigned)((rows + per_block - 1) / per_block));
  if (d == 64)
    hipLaunchKernelGGL((quantize_vec_kernel<16, FP8>), grid, dim3(256), 0, st, x, rows, codes, scales);
  else if (d == 128)
    hipLaunchKernelGGL((quantize_vec_kernel<32, FP8>), grid, dim3(256), 0, st, x, rows, codes, scales);
  else if (d == 256)
    hipLaunchKernelGGL((quantize_vec_kernel<64, FP8>), grid, dim3(256), 0, st, x, rows, codes, scales);
  else
    return false;
  return true;
}

}  // namespace

hipError_t launch_quantize_tiles(const float* x, int64_t groups, int64_t n, int64_t d,
                                 int64_t tile_rows, int8_t* codes, float* scales,
                                 hipStream_t st) {
  const int64_t tiles_per = (n + tile_rows - 1) / tile_rows;
  hipLaunchKernelGGL(quantize_tiles_kernel, dim3((unsigned)(groups * tiles_per)), dim3(256), 0,
                     st, x, n, (int)d, tile_rows, tiles_per, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const float* x, int64_t rows, int64_t d, uint8_t* codes,
                               float* scales, hipStream_t st) {
  if (launch_vec<true>(x, rows, d, codes, scales, st)) return hipGetLastError();
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, rows,
                     (int)d, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int64_t rows, int64_t d, int8_t* codes,
                           float* scales, hipStream_t st) {
  if (launch_vec<false>(x, rows, d, codes, scales, st)) return hipGetLastError();
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, (int)d,
                     codes, scales);
  return hipGetLastError();
}

}  // namespace pn
