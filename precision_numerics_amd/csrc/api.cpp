// C ABI of libpnattn: argument validation (pure host code, before any HIP
// call), dispatch to the kernel launchers, and error reporting.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.hpp"
#include "pnattn.h"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxSeq = int64_t(1) << 22;
constexpr int64_t kMaxGridYZ = 65535;

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

attn_status_t ok() {
  g_last_error.clear();
  return ATTN_OK;
}

attn_status_t from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks shared by every attention entry point.  On success fills `a` (with
// the resolved softmax scale) and sets *empty when some size is zero.
attn_status_t check_problem(const attn_problem_t* prob, const void* q, const void* k,
                            const void* v, const float* q_scale, const float* k_scale,
                            const void* o, pn::AttnArgs* a, bool* empty) {
  if (prob == nullptr) return fail(ATTN_ERR_INVALID_ARG, "prob is NULL");
  if (prob->batch < 0 || prob->heads < 0 || prob->seq_len < 0)
    return fail(ATTN_ERR_INVALID_ARG, "negative size (batch=%lld heads=%lld seq_len=%lld)",
                (long long)prob->batch, (long long)prob->heads, (long long)prob->seq_len);
  if (prob->head_dim <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "head_dim must be positive (got %lld)",
                (long long)prob->head_dim);
  if (prob->head_dim != 64 && prob->head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim %lld not built (64 or 128)",
                (long long)prob->head_dim);
  if (prob->seq_len > kMaxSeq)
    return fail(ATTN_ERR_UNSUPPORTED, "seq_len %lld above the limit %lld",
                (long long)prob->seq_len, (long long)kMaxSeq);
  if (prob->batch > 0 && prob->heads > INT32_MAX / prob->batch)
    return fail(ATTN_ERR_UNSUPPORTED, "batch*heads too large");
  // the flash schedule numbers the 256-row query tiles of all heads in
  // 32-bit arithmetic
  if (prob->batch * prob->heads * ((prob->seq_len + 255) / 256) > (int64_t(1) << 30))
    return fail(ATTN_ERR_UNSUPPORTED, "more than 2^30 query tiles of 256 rows");
  if (prob->causal != 0 && prob->causal != 1)
    return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", prob->causal);
  if (prob->p_bf16 != 0 && prob->p_bf16 != 1)
    return fail(ATTN_ERR_INVALID_ARG, "p_bf16 must be 0 or 1 (got %d)", prob->p_bf16);
  if (prob->dtype != ATTN_F32 && prob->dtype != ATTN_BF16 && prob->dtype != ATTN_INT8 &&
      prob->dtype != ATTN_FP8)
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", prob->dtype);
  if (!std::isfinite(prob->softmax_scale))
    return fail(ATTN_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (prob->o_f32 != 0 && prob->o_f32 != 1)
    return fail(ATTN_ERR_INVALID_ARG, "o_f32 must be 0 or 1 (got %d)", prob->o_f32);
  if (prob->stabilized != 0 && prob->stabilized != 1)
    return fail(ATTN_ERR_INVALID_ARG, "stabilized must be 0 or 1 (got %d)", prob->stabilized);
  if (prob->stabilized == 0 && prob->beta != 0.f)
    return fail(ATTN_ERR_INVALID_ARG, "beta must be 0 unless stabilized is 1");
  if (prob->stabilized == 1) {
    if (!(std::isfinite(prob->beta) && prob->beta > 1.f))
      return fail(ATTN_ERR_INVALID_ARG, "stabilized needs a finite beta > 1 (got %g)",
                  (double)prob->beta);
    if (prob->dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, "the stabilized variant is built for ATTN_BF16 only");
  }
  const bool scaled = prob->dtype == ATTN_INT8 || prob->dtype == ATTN_FP8;
  if (scaled && (q_scale == nullptr || k_scale == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "ATTN_INT8 and ATTN_FP8 need q_scale and k_scale");
  if (!scaled && (q_scale != nullptr || k_scale != nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "q_scale/k_scale are only for ATTN_INT8 and ATTN_FP8");
  *empty = prob->batch == 0 || prob->heads == 0 || prob->seq_len == 0;
  if (!*empty && (q == nullptr || k == nullptr || v == nullptr || o == nullptr))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  a->q = q;
  a->k = k;
  a->v = v;
  a->q_scale = q_scale;
  a->k_scale = k_scale;
  a->o = const_cast<void*>(o);
  a->batch = prob->batch;
  a->heads = prob->heads;
  a->seq_len = prob->seq_len;
  a->head_dim = (int)prob->head_dim;
  a->causal = prob->causal;
  a->dtype = prob->dtype;
  a->p_bf16 = prob->p_bf16;
  a->stabilized = prob->stabilized;
  a->beta = prob->beta;
  a->o_f32 = prob->o_f32;
  a->scale = prob->softmax_scale > 0.f
                 ? prob->softmax_scale
                 : (float)(1.0 / std::sqrt((double)prob->head_dim));
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

const char* attn_version(void) { return "pnattn 0.3.0 (gfx950)"; }

attn_status_t attn_bwd_delta(const attn_problem_t* prob, const void* o, const void* d_o,
                             float* delta, void* stream) {
  if (prob == nullptr) return fail(ATTN_ERR_INVALID_ARG, "prob is NULL");
  if (prob->batch < 0 || prob->heads < 0 || prob->seq_len < 0)
    return fail(ATTN_ERR_INVALID_ARG, "negative size");
  if (prob->head_dim <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "head_dim must be positive (got %lld)",
                (long long)prob->head_dim);
  if (prob->head_dim != 64 && prob->head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim %lld not built (64 or 128)",
                (long long)prob->head_dim);
  if (prob->dtype != ATTN_F32 && prob->dtype != ATTN_BF16 && prob->dtype != ATTN_INT8 &&
      prob->dtype != ATTN_FP8)
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", prob->dtype);
  if (prob->batch > 0 && prob->heads > INT64_MAX / prob->batch)
    return fail(ATTN_ERR_UNSUPPORTED, "batch*heads too large");
  const int64_t bh = prob->batch * prob->heads;
  if (bh > 0 && prob->seq_len > INT64_MAX / 128 / bh)
    return fail(ATTN_ERR_UNSUPPORTED, "problem too large");
  const int64_t rows = bh * prob->seq_len;
  if (rows == 0) return ok();
  if (o == nullptr || d_o == nullptr || delta == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "o, d_o and delta must be non-NULL");
  if (prob->o_f32 != 0 && prob->o_f32 != 1)
    return fail(ATTN_ERR_INVALID_ARG, "o_f32 must be 0 or 1 (got %d)", prob->o_f32);
  const int out = (prob->dtype == ATTN_F32 || prob->o_f32) ? pn::kF32 : pn::kBF16;
  return from_hip(pn::launch_delta(o, d_o, out, (int)prob->head_dim, rows, delta,
                                   (hipStream_t)stream),
                  "attn_bwd_delta launch");
}

attn_status_t attn_bwd_workspace_size(const attn_problem_t* prob, size_t* bytes) {
  if (bytes == nullptr) return fail(ATTN_ERR_INVALID_ARG, "bytes is NULL");
  pn::AttnArgs a;
  bool empty = false;
  const void* fake = (const void*)prob;  // sizes only: pointers are not checked here
  attn_status_t st = check_problem(prob, fake, fake, fake, nullptr, nullptr, fake, &a, &empty);
  if (st != ATTN_OK) return st;
  *bytes = empty ? 0 : (size_t)(prob->batch * prob->heads * prob->seq_len) * sizeof(float);
  return ok();
}

attn_status_t attn_bwd_flash(const attn_problem_t* prob, const void* q, const void* k,
                             const void* v, const void* o, const void* d_o, const float* lse,
                             void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* stream) {
  pn::AttnArgs a;
  bool empty = false;
  attn_status_t st = check_problem(prob, q, k, v, nullptr, nullptr, o, &a, &empty);
  if (st != ATTN_OK) return st;
  if (prob->dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd_flash is built for ATTN_BF16 only");
  if (prob->stabilized != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd_flash is the standard variant's backward");
  if (prob->o_f32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd_flash takes the bf16 forward output");
  if (empty) return ok();
  if (d_o == nullptr || lse == nullptr || dq == nullptr || dk == nullptr || dv == nullptr ||
      workspace == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "d_o, lse, dq, dk, dv and workspace must be non-NULL");
  const size_t need = (size_t)(prob->batch * prob->heads * prob->seq_len) * sizeof(float);
  if (workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  pn::AttnBwdArgs b;
  b.q = q;
  b.k = k;
  b.v = v;
  b.o = o;
  b.d_o = d_o;
  b.lse = lse;
  b.delta = (float*)workspace;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.batch = prob->batch;
  b.heads = prob->heads;
  b.seq_len = prob->seq_len;
  b.head_dim = (int)prob->head_dim;
  b.causal = prob->causal;
  b.scale = a.scale;
  return from_hip(pn::launch_flash_bwd(b, (hipStream_t)stream), "attn_bwd_flash launch");
}

attn_status_t attn_fwd_flash(const attn_problem_t* prob, const void* q, const void* k,
                             const void* v, const float* q_scale, const float* k_scale,
                             void* o, float* lse, void* stream) {
  pn::AttnArgs a;
  bool empty = false;
  attn_status_t st = check_problem(prob, q, k, v, q_scale, k_scale, o, &a, &empty);
  if (st != ATTN_OK) return st;
  if (empty) return ok();
  a.lse = lse;
  return from_hip(pn::launch_flash(a, (hipStream_t)stream), "attn_fwd_flash launch");
}

attn_status_t attn_fwd_flash_debug_s(const attn_problem_t* prob, const void* q, const void* k,
                                     const void* v, const float* q_scale, const float* k_scale,
                                     void* o, int32_t* s_out, void* stream) {
  pn::AttnArgs a;
  bool empty = false;
  attn_status_t st = check_problem(prob, q, k, v, q_scale, k_scale, o, &a, &empty);
  if (st != ATTN_OK) return st;
  if (prob->dtype != ATTN_INT8)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_flash_debug_s is for ATTN_INT8 only");
  if (prob->o_f32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_flash_debug_s writes a bf16 output");
  if (empty) return ok();
  if (s_out == nullptr) return fail(ATTN_ERR_INVALID_ARG, "s_out is NULL");
  a.s_dbg = s_out;
  return from_hip(pn::launch_flash(a, (hipStream_t)stream), "attn_fwd_flash_debug_s launch");
}

attn_status_t attn_baseline_workspace_size(const attn_problem_t* prob, size_t* bytes) {
  if (prob == nullptr || bytes == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "prob and bytes must be non-NULL");
  if (prob->batch < 0 || prob->heads < 0 || prob->seq_len < 0)
    return fail(ATTN_ERR_INVALID_ARG, "negative size");
  if (prob->seq_len > kMaxSeq) return fail(ATTN_ERR_UNSUPPORTED, "seq_len above the limit");
  if (prob->p_bf16 != 0 && prob->p_bf16 != 1)
    return fail(ATTN_ERR_INVALID_ARG, "p_bf16 must be 0 or 1");
  *bytes = pn::baseline_workspace_bytes(prob->batch * prob->heads, prob->seq_len, prob->p_bf16);
  return ok();
}

attn_status_t attn_fwd_baseline(const attn_problem_t* prob, const void* q, const void* k,
                                const void* v, const float* q_scale, const float* k_scale,
                                void* workspace, size_t workspace_bytes, void* o,
                                void* stream) {
  pn::AttnArgs a;
  bool empty = false;
  attn_status_t st = check_problem(prob, q, k, v, q_scale, k_scale, o, &a, &empty);
  if (st != ATTN_OK) return st;
  if (prob->stabilized != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "the stabilized variant is a flash-kernel option");
  if (empty) return ok();
  const int64_t bh = prob->batch * prob->heads;
  if (bh > kMaxGridYZ)
    return fail(ATTN_ERR_UNSUPPORTED, "baseline supports batch*heads <= %lld", (long long)kMaxGridYZ);
  if ((prob->seq_len + 127) / 128 > kMaxGridYZ)
    return fail(ATTN_ERR_UNSUPPORTED, "baseline seq_len too large");
  const size_t need = pn::baseline_workspace_bytes(bh, prob->seq_len, prob->p_bf16);
  if (workspace == nullptr) return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return from_hip(pn::launch_baseline(a, workspace, (hipStream_t)stream),
                  "attn_fwd_baseline launch");
}

attn_status_t attn_deviation_scratch_size(int64_t n, size_t* bytes) {
  if (bytes == nullptr) return fail(ATTN_ERR_INVALID_ARG, "bytes is NULL");
  if (n < 0) return fail(ATTN_ERR_INVALID_ARG, "n must be >= 0");
  *bytes = n == 0 ? 0 : pn::deviation_scratch_bytes(n);
  return ok();
}

attn_status_t attn_deviation(const void* o_test, int32_t o_dtype, const double* o_ref, int64_t n,
                             void* scratch, size_t scratch_bytes, attn_deviation_t* out_host,
                             void* stream) {
  if (out_host == nullptr) return fail(ATTN_ERR_INVALID_ARG, "out_host is NULL");
  if (n < 0) return fail(ATTN_ERR_INVALID_ARG, "n must be >= 0");
  if (o_dtype != ATTN_F32 && o_dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_F32 or ATTN_BF16");
  if (n == 0) {
    *out_host = attn_deviation_t{0, 0, 0, 0, 0, 0, 0, 0, -1};
    return ok();
  }
  if (o_test == nullptr || o_ref == nullptr || scratch == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "o_test, o_ref and scratch must be non-NULL");
  const size_t need = pn::deviation_scratch_bytes(n);
  if (scratch_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "scratch has %zu bytes, needs %zu", scratch_bytes, need);
  pn::DeviationRecord r;
  hipError_t e = pn::launch_deviation(o_test, o_dtype, o_ref, n, scratch, &r, (hipStream_t)stream);
  if (e != hipSuccess) return from_hip(e, "attn_deviation");
  attn_deviation_t out;
  const int64_t fin = r.n - r.n_nonfinite;
  const double nan = std::nan("");
  out.n = r.n;
  out.n_nonfinite = r.n_nonfinite;
  out.argmax = r.argmax;
  out.max_ref_abs = r.max_ref_abs;
  if (fin == 0) {
    out.max_abs = out.mean_abs = out.mean_signed = out.rms = out.rel_normwise = nan;
  } else {
    out.max_abs = r.max_abs;
    out.mean_abs = r.sum_abs / (double)fin;
    out.mean_signed = r.sum_signed / (double)fin;
    out.rms = std::sqrt(r.sum_sq / (double)fin);
    out.rel_normwise = r.max_ref_abs > 0 ? r.max_abs / r.max_ref_abs
                                         : (r.max_abs == 0 ? 0.0 : INFINITY);
  }
  *out_host = out;
  return ok();
}

attn_status_t attn_deviation_noalloc(const void* o_test, int32_t o_dtype, const double* o_ref,
                                     int64_t n, attn_deviation_t* out_host, void* stream) {
  if (out_host == nullptr) return fail(ATTN_ERR_INVALID_ARG, "out_host is NULL");
  if (n < 0) return fail(ATTN_ERR_INVALID_ARG, "n must be >= 0");
  if (o_dtype != ATTN_F32 && o_dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_F32 or ATTN_BF16");
  if (n == 0) {
    *out_host = attn_deviation_t{0, 0, 0, 0, 0, 0, 0, 0, -1};
    return ok();
  }
  if (o_test == nullptr || o_ref == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "o_test and o_ref must be non-NULL");
  const size_t need = pn::deviation_scratch_bytes(n);
  const size_t have = pn::deviation_noalloc_capacity();
  if (need > have)
    return fail(ATTN_ERR_WORKSPACE, "n = %lld needs %zu bytes of scratch; the library's own "
                "array holds %zu", (long long)n, need, have);
  void* scratch = nullptr;
  hipError_t e = pn::deviation_noalloc_scratch(&scratch);
  if (e != hipSuccess) return from_hip(e, "attn_deviation_noalloc: locating the scratch array");
  return attn_deviation(o_test, o_dtype, o_ref, n, scratch, have, out_host, stream);
}

attn_status_t attn_clock_sample(uint64_t* out, int32_t slots, void* stream) {
  if (slots < 1 || slots > 4096) return fail(ATTN_ERR_INVALID_ARG, "slots must be in [1, 4096]");
  if (out == nullptr) return fail(ATTN_ERR_INVALID_ARG, "out is NULL");
  return from_hip(pn::launch_clock_sample(out, slots, (hipStream_t)stream),
                  "attn_clock_sample launch");
}

static bool w_dtype_ok(int32_t t) { return t == ATTN_F32 || t == ATTN_BF16 || t == ATTN_F64; }

attn_status_t attn_wasserstein_scratch_size(int64_t n, int32_t a_dtype, int32_t b_dtype,
                                            size_t* bytes) {
  if (bytes == nullptr) return fail(ATTN_ERR_INVALID_ARG, "bytes is NULL");
  if (n < 0 || n > INT32_MAX) return fail(ATTN_ERR_INVALID_ARG, "n must be in [0, 2^31 - 1]");
  if (!w_dtype_ok(a_dtype) || !w_dtype_ok(b_dtype))
    return fail(ATTN_ERR_INVALID_ARG, "dtypes must be ATTN_F32, ATTN_BF16 or ATTN_F64");
  *bytes = n == 0 ? 0 : pn::wasserstein_scratch_bytes(n, a_dtype, b_dtype);
  return ok();
}

attn_status_t attn_wasserstein(const void* a, int32_t a_dtype, const void* b, int32_t b_dtype,
                               int64_t n, void* scratch, size_t scratch_bytes,
                               attn_wasserstein_t* out_host, void* stream) {
  if (out_host == nullptr) return fail(ATTN_ERR_INVALID_ARG, "out_host is NULL");
  if (n < 0 || n > INT32_MAX) return fail(ATTN_ERR_INVALID_ARG, "n must be in [0, 2^31 - 1]");
  if (!w_dtype_ok(a_dtype) || !w_dtype_ok(b_dtype))
    return fail(ATTN_ERR_INVALID_ARG, "dtypes must be ATTN_F32, ATTN_BF16 or ATTN_F64");
  const double nan = std::nan("");
  if (n == 0) {
    *out_host = attn_wasserstein_t{nan, nan, nan, 0, 0};
    return ok();
  }
  if (a == nullptr || b == nullptr || scratch == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "a, b and scratch must be non-NULL");
  const size_t need = pn::wasserstein_scratch_bytes(n, a_dtype, b_dtype);
  if (scratch_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "scratch has %zu bytes, needs %zu", scratch_bytes, need);
  pn::WassersteinRecord r;
  hipError_t e = pn::launch_wasserstein(a, a_dtype, b, b_dtype, n, scratch, &r,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return from_hip(e, "attn_wasserstein");
  attn_wasserstein_t out;
  out.n = n;
  out.n_nonfinite = r.n_nonfinite;
  if (r.n_nonfinite > 0) {
    out.w1 = out.w2 = out.winf = nan;
  } else {
    out.w1 = r.sum_abs / (double)n;
    out.w2 = std::sqrt(r.sum_sq / (double)n);
    out.winf = r.max_abs;
  }
  *out_host = out;
  return ok();
}

attn_status_t attn_quantize_int8_tiles(const float* x, int64_t groups, int64_t n, int64_t d,
                                       int64_t tile_rows, int8_t* codes, float* scales,
                                       void* stream) {
  if (groups < 0 || n < 0) return fail(ATTN_ERR_INVALID_ARG, "groups and n must be >= 0");
  if (d < 1 || d > 1024) return fail(ATTN_ERR_INVALID_ARG, "d must be in [1, 1024] (got %lld)", (long long)d);
  if (tile_rows < 1) return fail(ATTN_ERR_INVALID_ARG, "tile_rows must be >= 1");
  if (groups == 0 || n == 0) return ok();
  if (x == nullptr || codes == nullptr || scales == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  const int64_t tile = tile_rows < n ? tile_rows : n;
  if (groups > INT32_MAX / ((n + tile - 1) / tile))
    return fail(ATTN_ERR_UNSUPPORTED, "too many tiles");
  return from_hip(pn::launch_quantize_tiles(x, groups, n, d, tile, codes, scales,
                                            (hipStream_t)stream),
                  "attn_quantize_int8_tiles launch");
}

attn_status_t attn_quantize_fp8(const float* x, int64_t rows, int64_t d, uint8_t* codes,
                                float* scales, void* stream) {
  if (rows < 0) return fail(ATTN_ERR_INVALID_ARG, "rows must be >= 0");
  if (d < 1 || d > 1024) return fail(ATTN_ERR_INVALID_ARG, "d must be in [1, 1024] (got %lld)", (long long)d);
  if (rows == 0) return ok();
  if (x == nullptr || codes == nullptr || scales == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if ((rows + 3) / 4 > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED, "too many rows");
  return from_hip(pn::launch_quantize_fp8(x, rows, d, codes, scales, (hipStream_t)stream),
                  "attn_quantize_fp8 launch");
}

attn_status_t attn_quantize_int8(const float* x, int64_t rows, int64_t d, int8_t* codes,
                                 float* scales, void* stream) {
  if (rows < 0) return fail(ATTN_ERR_INVALID_ARG, "rows must be >= 0");
  if (d < 1 || d > 1024) return fail(ATTN_ERR_INVALID_ARG, "d must be in [1, 1024] (got %lld)", (long long)d);
  if (rows == 0) return ok();
  if (x == nullptr || codes == nullptr || scales == nullptr)
    return fail(ATTN_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if ((rows + 3) / 4 > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED, "too many rows");
  return from_hip(pn::launch_quantize(x, rows, d, codes, scales, (hipStream_t)stream),
                  "attn_quantize_int8 launch");
}

}  // extern "C"
