/*
 * pnattn — exact softmax attention forward on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain C types only; every tensor is a pointer plus the sizes in an
 * attn_problem_t.  No exception or C++ type crosses this boundary.
 *
 * The operation ("Why Low-Precision Transformer Training Fails", Algorithm 1,
 * problem statement: Q, K, V in R^{N x d} split into row blocks of B_r and
 * B_c rows; "Is Flash Attention Stable?", abstract: Flash versus Baseline
 * Attention in an isolated forward pass at BF16):
 *
 *     S = scale * Q K^T   (causal: key j visible to query i iff j <= i)
 *     O = softmax_rows(S) V
 *
 * for every (batch, head).  attn_fwd_flash never stores S (online softmax
 * over key blocks); attn_fwd_baseline stores S and P in a workspace.
 *
 * Conventions shared by all entry points
 *  - Layout: contiguous [batch][heads][seq_len][head_dim] ("BHSD"), head_dim
 *    fastest; int8 and fp8 scales are [batch][heads][seq_len].
 *  - Pointers are device pointers (hipMalloc'd or torch CUDA tensors) unless
 *    named *_host.  The caller owns every buffer; the library allocates no
 *    device memory and keeps no state besides a thread-local error string.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls enqueue work and return; kernel faults surface at the caller's
 *    next synchronisation.  attn_deviation and attn_wasserstein are the
 *    exceptions: they synchronise their stream before they return.
 *  - Validation is pure host code and runs before any HIP call: on an error
 *    nothing is launched and no output is touched.  attn_last_error() then
 *    describes the failure.
 */
#ifndef PNATTN_H
#define PNATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad flag     */
  ATTN_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, dtype combo    */
  ATTN_ERR_WORKSPACE = 3,   /* workspace / scratch smaller than required     */
  ATTN_ERR_HIP = 4          /* a HIP call failed; attn_last_error() has text */
} attn_status_t;

typedef enum {
  ATTN_F32 = 0,  /* Q, K, V and O are fp32                                 */
  ATTN_BF16 = 1, /* Q, K, V and O are bf16                                 */
  ATTN_INT8 = 2, /* Q, K are int8 codes with fp32 per-row scales;
                    V and O are bf16                                        */
  ATTN_F64 = 3,  /* fp64 values: only as an input of attn_wasserstein      */
  ATTN_FP8 = 4   /* Q, K are E4M3 fp8 codes ("FP8 Formats for Deep
                    Learning": sign, 4 exponent bits of bias 7, 3 mantissa
                    bits, max 448) with fp32 per-row scales; V and O are
                    bf16.  S = scale * sq_i * sk_j * (Qd Kd^T)_ij of the
                    decoded codes; the fp8 matrix products sum their terms
                    with less than fp32 precision (about 7e-5 of the
                    largest partial sum)                                   */
} attn_dtype_t;

typedef struct {
  int64_t batch;     /* >= 0 (0, like any zero size, is an empty problem:
                        the call validates and returns ATTN_OK, launching
                        nothing)                                            */
  int64_t heads;     /* >= 0; batch*heads < 2^31                           */
  int64_t seq_len;   /* N >= 0, at most 2^22; queries and keys have the
                        same length; batch*heads*ceil(N/256) at most 2^30
                        (ATTN_ERR_UNSUPPORTED beyond these limits)          */
  int64_t head_dim;  /* d: 64 or 128                                       */
  int32_t causal;    /* 0 or 1 (key j visible to query i iff j <= i)       */
  int32_t dtype;     /* attn_dtype_t                                       */
  int32_t p_bf16;    /* 1: round the unnormalised probabilities P to bf16
                        (round-to-nearest-even) before the P*V product,
                        which then runs on bf16 MFMA; 0: keep P in fp32 and
                        run P*V on fp32 MFMA (V widened exactly)            */
  float softmax_scale; /* > 0; <= 0 selects 1/sqrt(head_dim)               */
  int32_t stabilized;  /* 0: FlashAttention as published.  1: the stabilised
                          variant ("Why Low-Precision Transformer Training
                          Fails", Figure 7 and Algorithm 1): when the running
                          row maximum r_m of the scaled scores has occurred
                          more than once, the normaliser of the
                          probabilities becomes beta*r_m if r_m > 0 and 0 if
                          r_m < 0 (r_m = 0 keeps 0), so that no unnormalised
                          probability is exactly 1.  Occurrences are counted
                          online over the key blocks processed so far.
                          Range guard: the normaliser is capped at
                          r_m + 64 ln 2 (64 in log2 units), so the largest
                          probability stays >= 2^-64 where the rule alone
                          would underflow every exp in fp32 (r_m >~ 44/(beta-1)
                          or r_m <~ -44) and give 0/0.
                          attn_fwd_flash with ATTN_BF16 only (ATTN_ERR_
                          UNSUPPORTED otherwise; attn_fwd_baseline rejects
                          it).  The output equals softmax(S)V in exact
                          arithmetic either way; only rounding differs.     */
  float beta;          /* stabilized = 1: the factor beta > 1 (finite); the
                          page's own value is lost, so there is no default.
                          stabilized = 0: must be 0.                        */
  int32_t o_f32;       /* 0: O in the V dtype (bf16 for ATTN_BF16, ATTN_INT8,
                          ATTN_FP8).  1: O in fp32 whatever the inputs: the
                          fp32 O = acc / l the kernels form, before any
                          rounding to bf16 (so rounding it to bf16 gives the
                          o_f32 = 0 output bit for bit).  This separates the
                          rounding of O itself from the rounding upstream of
                          it (the bf16 P of "Why Low-Precision Transformer
                          Training Fails", Figures 5 and 7).  Both forward
                          calls; the backward calls take bf16 O (o_f32 = 1 is
                          ATTN_ERR_UNSUPPORTED there).                       */
} attn_problem_t;

/* FlashAttention forward ("Why Low-Precision Transformer Training Fails",
 * Algorithm 1, and the online-softmax accumulation that page's referee
 * report places at its Eq. (2)):
 * per query block, a running row max m, a running row sum l of the fp32
 * unnormalised probabilities P = exp(S - m) (P is 1 at the running row max,
 * as that page's Figure 5 caption notes: to within an ulp in fp32, exactly
 * once rounded to bf16), and an exp-rescaled fp32 output accumulator;
 * O = acc / l at the end.  S is never stored.
 *   q, k   : [B,H,N,d] of dtype (int8 codes for ATTN_INT8, E4M3 bytes
 *            for ATTN_FP8)
 *   v      : [B,H,N,d] fp32 for ATTN_F32, bf16 otherwise
 *   o      : [B,H,N,d], fp32 for ATTN_F32 or o_f32 = 1, bf16 otherwise
 *   q_scale, k_scale : [B,H,N] fp32, required for ATTN_INT8 and ATTN_FP8,
 *            else NULL
 *   lse    : optional [B,H,N] fp32 log-sum-exp of each score row (natural
 *            log, scaled scores), or NULL.                                 */
attn_status_t attn_fwd_flash(const attn_problem_t* prob, const void* q,
                             const void* k, const void* v,
                             const float* q_scale, const float* k_scale,
                             void* o, float* lse, void* stream);

/* Debug form of the int8 flash kernel: a separate instance of the same
 * kernel template (same tiles, schedule and arithmetic, compiled with one
 * extra store) that also writes each int32 score tile Qc Kc^T it computes
 * (before scaling) to s_out [B,H,N,N] int32 (entries the kernel never
 * computes, e.g. masked causal blocks, are left untouched); its o is
 * bitwise the production instance's.  ATTN_INT8 only; for checking that
 * the integer products are exact ("INT-FlashAttention", abstract).       */
attn_status_t attn_fwd_flash_debug_s(const attn_problem_t* prob, const void* q,
                                     const void* k, const void* v,
                                     const float* q_scale,
                                     const float* k_scale, void* o,
                                     int32_t* s_out, void* stream);

/* Bytes of workspace attn_fwd_baseline needs: S [B,H,N,N] (fp32, or int32
 * for ATTN_INT8) followed by P [B,H,N,N] (bf16 if p_bf16, else fp32) and
 * 256 bytes of tail padding.  For ATTN_INT8 and ATTN_FP8, S holds the
 * unscaled code products.                                                 */
attn_status_t attn_baseline_workspace_size(const attn_problem_t* prob,
                                           size_t* bytes);

/* Baseline attention ("Is Flash Attention Stable?", abstract: the
 * non-fused attention that Flash is compared with): three kernels on one
 * stream.  K1 writes S = scale*QK^T (int32 Qc Kc^T for ATTN_INT8) for all
 * N x N pairs; K2 applies the mask and a row softmax in fp32 and writes the
 * normalised P (bf16 if p_bf16, else fp32); K3 computes O = P V with fp32
 * accumulation.  workspace must hold attn_baseline_workspace_size bytes;
 * S sits at offset 0 and can be read back after the call.                 */
attn_status_t attn_fwd_baseline(const attn_problem_t* prob, const void* q,
                                const void* k, const void* v,
                                const float* q_scale, const float* k_scale,
                                void* workspace, size_t workspace_bytes,
                                void* o, void* stream);

/* Summary of e = o_test - o_ref over n elements, the deviation of a
 * low-precision forward output from a high-precision one ("Is Flash
 * Attention Stable?", abstract; O_lp and O_hp in "Why Low-Precision
 * Transformer Training Fails", Figure 5).  Elements with a non-finite e are
 * counted in n_nonfinite and excluded from the other statistics; argmax is
 * the first flat index of the largest |e| (-1 if none is finite).  Two-pass
 * fixed-order reduction: the result is bitwise reproducible.             */
typedef struct {
  double max_abs, mean_abs, mean_signed, rms, max_ref_abs, rel_normwise;
  int64_t n, n_nonfinite, argmax;
} attn_deviation_t;

/* Bytes of device scratch attn_deviation needs for n elements (n >= 0).  */
attn_status_t attn_deviation_scratch_size(int64_t n, size_t* bytes);

/*   o_test  : n elements of o_dtype (ATTN_F32 or ATTN_BF16)
 *   o_ref   : n fp64 elements
 *   n == 0 gives n = 0, argmax = -1 and zero statistics without a launch.
 *   out_host: host pointer, filled after the stream has synchronised.     */
attn_status_t attn_deviation(const void* o_test, int32_t o_dtype,
                             const double* o_ref, int64_t n, void* scratch,
                             size_t scratch_bytes, attn_deviation_t* out_host,
                             void* stream);

/* attn_deviation without a caller-provided scratch buffer, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving or training loops, harnesses that forbid allocation).  The
 * partial sums live in a 64 KiB device array of the library, one per GPU,
 * located on the first call on each device and held until the process
 * ends; the call itself allocates nothing (no hipMalloc, no library
 * allocation).  The array holds the scratch of every n >= 0 (the partials
 * are capped at 1024 records); a size whose scratch would not fit is
 * rejected with ATTN_ERR_WORKSPACE.  Every call on one GPU uses that GPU's
 * array: calls that overlap on one GPU (other host threads, other streams)
 * race and must not be issued.  Same arguments, statistics and bitwise
 * results as attn_deviation; synchronises its stream before it returns. */
attn_status_t attn_deviation_noalloc(const void* o_test, int32_t o_dtype,
                                     const double* o_ref, int64_t n,
                                     attn_deviation_t* out_host, void* stream);

/* Wasserstein distances between the empirical distributions of two tensors
 * of n values each ("Is Flash Attention Stable?", abstract: the impact of
 * numeric deviation measured with the Wasserstein distance, after
 * "Statistical Aspects of Wasserstein Distances" in its reference list).
 * Each tensor is the uniform distribution on its n values; on the real line
 * the optimal coupling pairs equal order statistics a_(i), b_(i), so
 *   w1   = sum_i |a_(i) - b_(i)| / n
 *   w2   = sqrt(sum_i (a_(i) - b_(i))^2 / n)
 *   winf = max_i |a_(i) - b_(i)|
 * computed in fp64 from the exact values, in a fixed order (bitwise
 * reproducible).  If either tensor holds a NaN or an infinity the three
 * distances are NaN and n_nonfinite counts those elements.               */
typedef struct {
  double w1, w2, winf;
  int64_t n, n_nonfinite;
} attn_wasserstein_t;

/* Bytes of device scratch attn_wasserstein needs (n >= 0; dtypes as below;
 * about 2n times the two element sizes).                                 */
attn_status_t attn_wasserstein_scratch_size(int64_t n, int32_t a_dtype, int32_t b_dtype,
                                            size_t* bytes);

/*   a, b    : n device elements each, of a_dtype / b_dtype, any of
 *             ATTN_F32, ATTN_BF16, ATTN_F64 (a and b may differ);
 *             read only.  0 <= n <= 2^31 - 1.
 *   scratch : device memory of at least the size above (the sorted keys
 *             of both inputs and the partial sums; caller-owned).
 *   out_host: host pointer, filled after the stream has synchronised (this
 *             call synchronises its stream).  n == 0 gives NaN distances
 *             without a launch.                                          */
attn_status_t attn_wasserstein(const void* a, int32_t a_dtype, const void* b, int32_t b_dtype,
                               int64_t n, void* scratch, size_t scratch_bytes,
                               attn_wasserstein_t* out_host, void* stream);

/* delta = rowsum(dO o O): for every row i of every (batch, head),
 * delta_i = sum_c dO[i,c] * O[i,c] -- the per-row term the attention backward
 * pass derives from the forward output ("Why Low-Precision Transformer
 * Training Fails", Figure 5 caption; that page traces the training failure
 * to delta computed from the low-precision O).
 *   prob  : sizes and dtype as for the forward call (causal, p_bf16,
 *           softmax_scale, stabilized and beta are not used)
 *   o, d_o: [B,H,N,d] in the forward output dtype (fp32 for ATTN_F32,
 *           bf16 otherwise)
 *   delta : [B,H,N] fp32
 * One fused multiply-add per element in fp32 (bf16 products are exact),
 * then a fixed-order combination of the partial sums: bitwise
 * reproducible.  A zero size validates and returns ATTN_OK.              */
attn_status_t attn_bwd_delta(const attn_problem_t* prob, const void* o,
                             const void* d_o, float* delta, void* stream);

/* Bytes of workspace attn_bwd_flash needs: delta, B*H*N fp32.           */
attn_status_t attn_bwd_workspace_size(const attn_problem_t* prob, size_t* bytes);

/* FlashAttention backward: the gradients of O = softmax_rows(S) V with
 * S = scale Q K^T (causal mask as in the forward) for the upstream gradient
 * dO, from the stored forward output O and its lse:
 *   delta = rowsum(dO o O), dV = P^T dO, dP = dO V^T,
 *   dS = P o (dP - delta), dQ = scale dS K, dK = scale dS^T Q
 * ("Why Low-Precision Transformer Training Fails": delta = rowsum(dO o O),
 * Figure 5 caption; delta is formed from the stored, low-precision O, as
 * that page's analysis of the error in O has it).  P is recomputed from
 * q, k and lse block by block (nothing N x N is stored).
 *   prob   : as for the forward; ATTN_BF16 only (UNSUPPORTED otherwise),
 *            standard variant (stabilized = 0); p_bf16 is not used (the
 *            backward rounds P and dS to bf16 for its bf16 products)
 *   q,k,v,o,d_o : [B,H,N,d] bf16 (o and lse from attn_fwd_flash)
 *   lse    : [B,H,N] fp32, natural log, as attn_fwd_flash writes it
 *   dq,dk,dv : [B,H,N,d] bf16 outputs (RNE of the fp32 accumulations)
 *   workspace: attn_bwd_workspace_size bytes; holds delta afterwards.
 * Deterministic: every output element is accumulated by one lane in a
 * fixed order.                                                            */
attn_status_t attn_bwd_flash(const attn_problem_t* prob, const void* q, const void* k,
                             const void* v, const void* o, const void* d_o, const float* lse,
                             void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Symmetric per-row int8 quantisation of fp32 rows x [rows][d] (the int8
 * Q/K input of "INT-FlashAttention", abstract; the per-row absmax/127
 * granularity is this library's reading):
 *   scale_r = fp32(absmax_r / 127)  (IEEE division), 1 if that is 0;
 *   code    = clamp(round_half_even(fp32(x / scale_r)), -127, 127).
 * codes: [rows][d] int8, scales: [rows] fp32.  1 <= d <= 1024.            */
attn_status_t attn_quantize_int8(const float* x, int64_t rows, int64_t d,
                                 int8_t* codes, float* scales, void* stream);

/* Per-tile int8 scales (the per-block scale granularity among the
 * low-precision variants): x [groups][n][d] fp32, e.g. groups = batch*heads;
 * the n rows of each group form tiles of tile_rows consecutive rows (the
 * last one ragged, tiles never span two groups), and each tile shares
 *   scale_t = fp32(absmax over the tile / 127)  (IEEE division), 1 if 0;
 *   code    = clamp(round_half_even(fp32(x / scale_t)), -127, 127).
 * codes: [groups][n][d] int8; scales: [groups][n] fp32, every row holding
 * its tile's scale, so attn_fwd_flash/attn_fwd_baseline take them as the
 * per-row scales of ATTN_INT8.  tile_rows = 1 is attn_quantize_int8.
 * 1 <= d <= 1024, tile_rows >= 1; zero sizes validate and return ATTN_OK. */
attn_status_t attn_quantize_int8_tiles(const float* x, int64_t groups, int64_t n,
                                       int64_t d, int64_t tile_rows, int8_t* codes,
                                       float* scales, void* stream);

/* The same per-row scheme with E4M3 fp8 codes (ATTN_FP8; the per-row
 * absmax/448 scale is this library's reading, as for int8):
 *   scale_r = fp32(absmax_r / 448)  (IEEE division), 1 if that is 0;
 *   code    = E4M3(fp32(x / scale_r)): nearest, ties to the even code,
 *             magnitudes at or above 448 give 448, the sign bit is x's
 *             (a NaN input gives 0x7f).
 * codes: [rows][d] uint8, scales: [rows] fp32.  1 <= d <= 1024.           */
attn_status_t attn_quantize_fp8(const float* x, int64_t rows, int64_t d,
                                uint8_t* codes, float* scales, void* stream);

/* Measurement aid: samples of the shader clock, for reading a timed region
 * against the clock it ran at (the power controller lowers the shader clock
 * under sustained matrix work).  Launches `slots` workgroups on stream;
 * each writes (location, 64-bit shader-clock counter s_memtime, 100 MHz
 * real-time counter s_memrealtime) to out[3*i .. 3*i+2], where location =
 * XCD id << 8 | HW_ID bits 8..15 (CU, shader array, shader engine).  The
 * counters of different CUs are not synchronised, so two calls are
 * compared on the same location: clock = 100 MHz * d(memtime) /
 * d(realtime).  A few hundred slots cover every CU.
 *   out  : device buffer of 3*slots uint64_t;  1 <= slots <= 4096.       */
attn_status_t attn_clock_sample(uint64_t* out, int32_t slots, void* stream);

const char* attn_status_string(attn_status_t status);
/* Detail of the last failing call on this thread ("" if none).           */
const char* attn_last_error(void);
/* Library version string.                                                 */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PNATTN_H */
