// Host-side launchers behind the C ABI (internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pn {

enum DType : int { kF32 = 0, kBF16 = 1, kINT8 = 2, kF64 = 3, kFP8 = 4 };

struct AttnArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const float* q_scale = nullptr;
  const float* k_scale = nullptr;
  void* o = nullptr;
  float* lse = nullptr;
  int32_t* s_dbg = nullptr;
  int64_t batch = 0, heads = 0, seq_len = 0;
  int head_dim = 0;
  int causal = 0;
  int dtype = kBF16;
  int p_bf16 = 1;
  float scale = 0.f;  // resolved softmax scale (> 0)
  int stabilized = 0; // flash only: the repeated-max normaliser variant
  float beta = 0.f;   // its factor (> 1) for a repeated positive max
  int o_f32 = 0;      // O in fp32 (else in the V dtype)
};

// Flash forward; returns the launch status.
hipError_t launch_flash(const AttnArgs& a, hipStream_t stream);

// Baseline: workspace holds S [B,H,N,N] (4 B/elem) then P (2 or 4 B/elem).
size_t baseline_workspace_bytes(int64_t bh, int64_t n, int p_bf16);
hipError_t launch_baseline(const AttnArgs& a, void* workspace,
                           hipStream_t stream);

// Deviation summary; partials and the final record live in scratch.
size_t deviation_scratch_bytes(int64_t n);
struct DeviationRecord {
  double max_abs, sum_abs, sum_signed, sum_sq, max_ref_abs;
  int64_t n_nonfinite, argmax, n;
};
hipError_t launch_deviation(const void* o_test, int o_dtype,
                            const double* o_ref, int64_t n, void* scratch,
                            DeviationRecord* out_host, hipStream_t stream);
// The library's own deviation scratch on the current device (a file-scope
// device array, located once per device): its device address and size.
hipError_t deviation_noalloc_scratch(void** ptr);
size_t deviation_noalloc_capacity();

// FlashAttention backward (bf16): delta = rowsum(dO o O) into `delta`
// (B*H*N fp32, caller's workspace), then dK/dV and dQ.
struct AttnBwdArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const void* o = nullptr;
  const void* d_o = nullptr;
  const float* lse = nullptr;
  float* delta = nullptr;
  void* dq = nullptr;
  void* dk = nullptr;
  void* dv = nullptr;
  int64_t batch = 0, heads = 0, seq_len = 0;
  int head_dim = 0;
  int causal = 0;
  float scale = 0.f;
};
hipError_t launch_flash_bwd(const AttnBwdArgs& a, hipStream_t stream);

// Wasserstein distances of two n-element tensors (kF32, kBF16 or kF64):
// sorted keys and partials live in scratch; the record holds the sums.
struct WassersteinRecord {
  double sum_abs, sum_sq, max_abs;
  int64_t n_nonfinite;
};
size_t wasserstein_scratch_bytes(int64_t n, int a_dtype, int b_dtype);
hipError_t launch_wasserstein(const void* a, int a_dtype, const void* b, int b_dtype, int64_t n,
                              void* scratch, WassersteinRecord* out_host, hipStream_t stream);

// delta = rowsum(dO o O) over rows of head_dim elements of the output dtype
// (kF32, or bf16 for the others).
hipError_t launch_delta(const void* o, const void* d_o, int out_dtype, int head_dim,
                        int64_t rows, float* delta, hipStream_t stream);

hipError_t launch_quantize(const float* x, int64_t rows, int64_t d,
                           int8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_quantize_tiles(const float* x, int64_t groups, int64_t n, int64_t d,
                                 int64_t tile_rows, int8_t* codes, float* scales,
                                 hipStream_t stream);
hipError_t launch_quantize_fp8(const float* x, int64_t rows, int64_t d,
                               uint8_t* codes, float* scales, hipStream_t stream);

// One workgroup per slot records (XCD id, shader-clock counter, 100 MHz
// counter) into out[3 * slot + 0..2].
hipError_t launch_clock_sample(uint64_t* out, int slots, hipStream_t stream);

}  // namespace pn
