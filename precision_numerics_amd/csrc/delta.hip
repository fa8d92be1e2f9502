// delta_i = sum_c dO[i,c] * O[i,c] for every row: the per-row term the
// attention backward pass derives from the forward output ("Why
// Low-Precision Transformer Training Fails": delta = rowsum(dO o O), the
// Figure 5 caption; that page traces the training failure to delta computed
// from the low-precision O).
//
// HBM-bound: each row is read once from O and once from dO.  A row of d
// elements is spread over d*sizeof(T)/16 lanes that each load one 16-byte
// chunk of O and of dO (coalesced: consecutive lanes read consecutive
// chunks), form their partial sum with one fused multiply-add per element,
// and combine the partial sums with a fixed xor butterfly, so the result is
// bitwise reproducible.  bf16 products are exact in fp32.
#include "device.hpp"
#include "launch.hpp"

namespace pn {
namespace {

constexpr int kDeltaThreads = 256;

template <typename T> __device__ __forceinline__ float elem(T x);
template <> __device__ __forceinline__ float elem<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <> __device__ __forceinline__ float elem<float>(float x) { return x; }

template <typename T, int D>
__global__ __launch_bounds__(kDeltaThreads) void delta_kernel(const T* __restrict__ o,
                                                              const T* __restrict__ g,
                                                              float* __restrict__ delta,
                                                              int64_t rows) {
  constexpr int kEPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int kLPR = D / kEPC;             // lanes per row
  constexpr int kRPW = 64 / kLPR;            // rows per wave and pass
  static_assert(kLPR >= 1 && kLPR <= 64 && 64 % kLPR == 0, "row must map onto whole lanes");
  const int lane = threadIdx.x & 63;
  const int sub = lane % kLPR;
  const int rw = lane / kLPR;
  const int64_t wave = ((int64_t)blockIdx.x * kDeltaThreads + threadIdx.x) >> 6;
  const int64_t nwave = ((int64_t)gridDim.x * kDeltaThreads) >> 6;
  for (int64_t r0 = wave * kRPW; r0 < rows; r0 += nwave * kRPW) {
    const int64_t row = r0 + rw;
    float acc = 0.f;
    if (row < rows) {
      const int64_t off = row * D + (int64_t)sub * kEPC;
      T ov[kEPC], gv[kEPC];
      *(i32x4*)ov = *(const i32x4*)(o + off);
      *(i32x4*)gv = *(const i32x4*)(g + off);
#pragma unroll
      for (int e = 0; e < kEPC; ++e) acc = __builtin_fmaf(elem<T>(gv[e]), elem<T>(ov[e]), acc);
    }
#pragma unroll
    for (int m = kLPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (sub == 0 && row < rows) delta[row] = acc;
  }
}

template <typename T, int D>
hipError_t launch_t(const void* o, const void* g, float* delta, int64_t rows, hipStream_t st) {
  constexpr int kRowsPerBlock = (kDeltaThreads / 64) * (64 / (D * (int)sizeof(T) / 16));
  const int64_t need = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const unsigned grid = (unsigned)(need < 8192 ? need : 8192);  // grid-stride beyond
  hipLaunchKernelGGL((delta_kernel<T, D>), dim3(grid), dim3(kDeltaThreads), 0, st,
                     (const T*)o, (const T*)g, delta, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_delta(const void* o, const void* d_o, int out_dtype, int head_dim,
                        int64_t rows, float* delta, hipStream_t stream) {
  if (out_dtype == kF32) {
    return head_dim == 64 ? launch_t<float, 64>(o, d_o, delta, rows, stream)
                          : launch_t<float, 128>(o, d_o, delta, rows, stream);
  }
  return head_dim == 64 ? launch_t<uint16_t, 64>(o, d_o, delta, rows, stream)
                        : launch_t<uint16_t, 128>(o, d_o, delta, rows, stream);
}

}  // namespace pn
