// Deviation summary of a low-precision attention output against a
// high-precision reference ("Is Flash Attention Stable?", abstract: numeric
// deviation of an isolated forward pass; O_lp and O_hp in "Why Low-Precision
// Transformer Training Fails", Figure 5).
//
// Two passes with a fixed element-to-thread map and fixed reduction trees, so
// the fp64 sums are bitwise reproducible run to run:
//   pass 1: G workgroups, each over one contiguous chunk, write a partial
//   pass 2: one workgroup folds the G partials in index order
// HBM-bound: reads n * (2 or 4) bytes of o_test and 8n bytes of o_ref once.
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace pn {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 1024;

struct Partial {
  double max_abs;  // -1 when no finite element was seen
  double sum_abs, sum_signed, sum_sq, max_ref;
  int64_t argmax, nonfinite;
};

__device__ __forceinline__ void fold(Partial& a, const Partial& b) {
  if (b.max_abs > a.max_abs || (b.max_abs == a.max_abs && b.argmax < a.argmax)) {
    a.max_abs = b.max_abs;
    a.argmax = b.argmax;
  }
  a.sum_abs += b.sum_abs;
  a.sum_signed += b.sum_signed;
  a.sum_sq += b.sum_sq;
  a.max_ref = fmax(a.max_ref, b.max_ref);
  a.nonfinite += b.nonfinite;
}

__device__ __forceinline__ Partial empty_partial() {
  Partial p;
  p.max_abs = -1.0;
  p.sum_abs = p.sum_signed = p.sum_sq = 0.0;
  p.max_ref = 0.0;
  p.argmax = INT64_MAX;
  p.nonfinite = 0;
  return p;
}

// Fixed-shape tree over the workgroup; result in lds[0].
__device__ void tree(Partial& mine, Partial* lds) {
  lds[threadIdx.x] = mine;
  __syncthreads();
  for (int s = kThreads / 2; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) fold(lds[threadIdx.x], lds[threadIdx.x + s]);
    __syncthreads();
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void deviation_pass1(const void* t, const double* ref,
                                                           int64_t n, int64_t chunk,
                                                           Partial* parts) {
  __shared__ Partial lds[kThreads];
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  Partial mine = empty_partial();
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
    const double x = BF16 ? (double)bf16_to_f32(((const uint16_t*)t)[i]) : (double)((const float*)t)[i];
    const double r = ref[i];
    const double e = x - r;
    if (isfinite(r)) mine.max_ref = fmax(mine.max_ref, fabs(r));
    if (!isfinite(e)) {
      mine.nonfinite += 1;
      continue;
    }
    const double ae = fabs(e);
    if (ae > mine.max_abs) {  // ascending i per thread: the first maximum wins
      mine.max_abs = ae;
      mine.argmax = i;
    }
    mine.sum_abs += ae;
    mine.sum_signed += e;
    mine.sum_sq += e * e;
  }
  tree(mine, lds);
  if (threadIdx.x == 0) parts[blockIdx.x] = lds[0];
}

// One element into a thread's partial (elements in ascending index order per
// thread: the first maximum wins).
__device__ __forceinline__ void visit(Partial& mine, double x, double r, int64_t i) {
  const double e = x - r;
  if (isfinite(r)) mine.max_ref = fmax(mine.max_ref, fabs(r));
  if (!isfinite(e)) {
    mine.nonfinite += 1;
    return;
  }
  const double ae = fabs(e);
  if (ae > mine.max_abs) {
    mine.max_abs = ae;
    mine.argmax = i;
  }
  mine.sum_abs += ae;
  mine.sum_signed += e;
  mine.sum_sq += e * e;
}

// The same pass with 16-byte loads (both operands 16-byte aligned, the chunk
// a multiple of 8 * kThreads): thread t takes the 8-element groups t,
// t + kThreads, .. of its workgroup's chunk, two at a time with all their
// loads issued before the arithmetic, then (thread 0) the chunk's last
// partial group.  Elements stay in ascending order within each thread.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void deviation_pass1_vec(const void* t, const double* ref,
                                                               int64_t n, int64_t chunk,
                                                               Partial* parts) {
  __shared__ Partial lds[kThreads];
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  const int64_t ngrp = hi > lo ? (hi - lo) / 8 : 0;  // whole 8-element groups
  Partial mine = empty_partial();
  auto load8 = [&](int64_t i0, double (&x)[8], double (&r)[8]) __attribute__((always_inline)) {
    if constexpr (BF16) {
      const uint4 v = *(const uint4*)((const uint16_t*)t + i0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = (double)bf16_to_f32((uint16_t)(w[k] & 0xffffu));
        x[2 * k + 1] = (double)bf16_to_f32((uint16_t)(w[k] >> 16));
      }
    } else {
      const float4 a = *(const float4*)((const float*)t + i0);
      const float4 b = *(const float4*)((const float*)t + i0 + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double2 d = *(const double2*)(ref + i0 + 2 * k);
      r[2 * k] = d.x;
      r[2 * k + 1] = d.y;
    }
  };
  int64_t gi = threadIdx.x;
  for (; gi + kThreads < ngrp; gi += 2 * kThreads) {
    double x0[8], r0[8], x1[8], r1[8];
    load8(lo + 8 * gi, x0, r0);
    load8(lo + 8 * (gi + kThreads), x1, r1);
#pragma unroll
    for (int k = 0; k < 8; ++k) visit(mine, x0[k], r0[k], lo + 8 * gi + k);
#pragma unroll
    for (int k = 0; k < 8; ++k) visit(mine, x1[k], r1[k], lo + 8 * (gi + kThreads) + k);
  }
  if (gi < ngrp) {
    double x0[8], r0[8];
    load8(lo + 8 * gi, x0, r0);
#pragma unroll
    for (int k = 0; k < 8; ++k) visit(mine, x0[k], r0[k], lo + 8 * gi + k);
  }
  if (threadIdx.x == 0) {
    for (int64_t i = lo + 8 * ngrp; i < hi; ++i) {
      const double x = BF16 ? (double)bf16_to_f32(((const uint16_t*)t)[i]) : (double)((const float*)t)[i];
      visit(mine, x, ref[i], i);
    }
  }
  tree(mine, lds);
  if (threadIdx.x == 0) parts[blockIdx.x] = lds[0];
}

__global__ __launch_bounds__(kThreads) void deviation_pass2(const Partial* parts, int nparts,
                                                           DeviationRecord* out, int64_t n) {
  __shared__ Partial lds[kThreads];
  Partial mine = empty_partial();
  for (int i = threadIdx.x; i < nparts; i += kThreads) fold(mine, parts[i]);
  tree(mine, lds);
  if (threadIdx.x == 0) {
    const Partial& p = lds[0];
    DeviationRecord r;
    r.max_abs = p.max_abs;
    r.sum_abs = p.sum_abs;
    r.sum_signed = p.sum_signed;
    r.sum_sq = p.sum_sq;
    r.max_ref_abs = p.max_ref;
    r.n_nonfinite = p.nonfinite;
    r.argmax = p.max_abs < 0 ? -1 : p.argmax;
    r.n = n;
    *out = r;
  }
}

int blocks_for(int64_t n) {
  int64_t b = (n + (int64_t)kThreads * 64 - 1) / ((int64_t)kThreads * 64);
  if (b < 1) b = 1;
  if (b > kMaxBlocks) b = kMaxBlocks;
  return (int)b;
}

// Scratch of the allocation-free entry point: one array per GPU, held until
// the process ends.  Its size covers the largest scratch any n needs (the
// partials are capped at kMaxBlocks).  In host code `scratch` names a
// host-side stand-in, not device memory: only the address returned by
// hipGetSymbolAddress for the current device may be passed to kernels.
constexpr size_t kNoAllocScratchBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t deviation_scratch_bytes(int64_t n) {
  return (size_t)blocks_for(n) * sizeof(Partial) + sizeof(DeviationRecord) + 256;
}

size_t deviation_noalloc_capacity() { return kNoAllocScratchBytes; }

hipError_t deviation_noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_deviation(const void* o_test, int o_dtype, const double* o_ref, int64_t n,
                            void* scratch, DeviationRecord* out_host, hipStream_t st) {
  const int nb = blocks_for(n);
  Partial* parts = (Partial*)scratch;
  DeviationRecord* rec =
      (DeviationRecord*)(((uintptr_t)(parts + nb) + 255) & ~(uintptr_t)255);
  const bool vec = ((uintptr_t)o_test % 16 == 0) && ((uintptr_t)o_ref % 16 == 0);
  if (vec) {
    // chunks of whole 8 * kThreads element groups (the last one ragged; any
    // workgroup past the end writes an empty partial)
    constexpr int64_t kGroup = 8 * kThreads;
    const int64_t chunk = ((n + nb - 1) / nb + kGroup - 1) / kGroup * kGroup;
    if (o_dtype == kBF16)
      hipLaunchKernelGGL((deviation_pass1_vec<true>), dim3(nb), dim3(kThreads), 0, st, o_test, o_ref, n, chunk, parts);
    else
      hipLaunchKernelGGL((deviation_pass1_vec<false>), dim3(nb), dim3(kThreads), 0, st, o_test, o_ref, n, chunk, parts);
  } else {
    const int64_t chunk = (n + nb - 1) / nb;
    if (o_dtype == kBF16)
      hipLaunchKernelGGL((deviation_pass1<true>), dim3(nb), dim3(kThreads), 0, st, o_test, o_ref, n, chunk, parts);
    else
      hipLaunchKernelGGL((deviation_pass1<false>), dim3(nb), dim3(kThreads), 0, st, o_test, o_ref, n, chunk, parts);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(deviation_pass2, dim3(1), dim3(kThreads), 0, st, parts, nb, rec, n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(out_host, rec, sizeof(DeviationRecord), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace pn
