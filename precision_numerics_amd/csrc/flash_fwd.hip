// FlashAttention forward for gfx950: tiled exact attention with an online
// softmax; the score matrix S is never stored.
//
// Method ("Why Low-Precision Transformer Training Fails", Algorithm 1: Q is
// split into T_r = ceil(N/B_r) row blocks and K, V into T_c = ceil(N/B_c)
// row blocks; the online-softmax accumulation its referee report places at
// Eq. (2)).  For each query block and each key block j in ascending order:
//     m'  = max(m, rowmax(S_j))
//     P_j = exp(S_j - m')              (unnormalised; exactly 1 at the max)
//     l'  = exp(m - m') l + rowsum(P_j)
//     O'  = exp(m - m') O + P_j V_j
// and finally O = O' / l'.  In exact arithmetic this is softmax(S) V for any
// B_r, B_c; only rounding depends on them.
//
// Mapping onto CDNA4:
//  * One workgroup = 4 wave64s = B_r = 128 query rows; each wave owns 32 rows.
//    B_c = 64 keys per step, staged in LDS (K and V row-major, padded rows).
//  * The wave computes S^T = K_j Q^T (32 keys x 32 queries per MFMA tile), so
//    lane l owns query l%32 and half of the block's keys: the row max and row
//    sum are in-lane reductions plus one permlane32_swap, and exp(m - m') is
//    a per-lane scalar.  The K rows are fed to the MFMA in a permuted order
//    so that accumulator register r of lane group g holds key
//    16*(r/8) + 8*g + r%8, which is exactly the order in which the P^T
//    operand of the next product must present keys.
//  * O^T = V_j^T P_j^T accumulates in fp32 registers (32 x d per wave).  The
//    V^T operand comes straight from the row-major V tile through the
//    transposing LDS read ds_read_b64_tr_b16.
//  * Scores are kept in log2 units (scale * log2 e folded into one multiply)
//    so every exponential is one v_exp_f32.
//  * Grid = (batch*heads, query tiles).  Causal launches hand out the longest
//    query tiles first; when batch*heads is a multiple of 8 all tiles of one
//    head land on the same XCD (round-robin dispatch), sharing its L2.
#include "device.hpp"
#include "launch.hpp"

namespace pn {
namespace {

enum QKKind { QK_BF16 = 0, QK_I8 = 1, QK_F32 = 2 };
// P*V engines: bf16 P and bf16 V on bf16 MFMA; otherwise fp32 MFMA with V
// widened exactly (V stored as bf16 or as fp32).
enum PVKind { PV_BF16 = 0, PV_F32_VBF16 = 1, PV_F32_VF32 = 2 };

constexpr int kWaves = 4;            // waves per workgroup (one per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;     // query rows per workgroup
constexpr int kBC = 64;              // keys per step

template <int QK> struct QKTraits;
template <> struct QKTraits<QK_BF16> { using T = uint16_t; };
template <> struct QKTraits<QK_I8> { using T = int8_t; };
template <> struct QKTraits<QK_F32> { using T = float; };
template <int PV> struct VTraits { using T = uint16_t; };
template <> struct VTraits<PV_F32_VF32> { using T = float; };

// LDS tile geometry.  Rows are padded so that the two read patterns of the
// kernel are free of bank conflicts: +16 bytes per K row (16 consecutive K
// rows read the same 16-byte column), +64 bytes per V row (the transposing
// reads touch 4 rows x 64 bytes at a time).  Tiles are whole multiples of
// 1 KiB, the footprint of one wave-wide 16-byte buffer load into LDS.
template <int D, int QK, int PV> struct Tile {
  static constexpr int kRowK = D * (int)sizeof(typename QKTraits<QK>::T);
  static constexpr int kRowV = D * (int)sizeof(typename VTraits<PV>::T);
  static constexpr int kStrK = kRowK + 16;
  static constexpr int kStrV = kRowV + 64;
  static constexpr int kBytesK = kBC * kStrK;
  static constexpr int kBytesV = kBC * kStrV;
  static constexpr int kSegK = kBytesK / 1024;
  static constexpr int kSegV = kBytesV / 1024;
  static constexpr int kSegKPerWave = (kSegK + kWaves - 1) / kWaves;
  static constexpr int kSegVPerWave = (kSegV + kWaves - 1) / kWaves;
  static constexpr int kBytesSk = (QK == QK_I8) ? kBC * 4 : 0;
  // [K buf0][K buf1][V buf0][V buf1][sk buf0][sk buf1]
  static constexpr int kOffV = 2 * kBytesK;
  static constexpr int kOffSk = kOffV + 2 * kBytesV;
  static constexpr int kLds = kOffSk + 2 * kBytesSk;
  static_assert(kBytesK % 1024 == 0 && kBytesV % 1024 == 0, "tiles must be whole segments");
};

struct FlashParams {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;
  const float* k_scale;
  void* o;
  float* lse;
  int32_t* s_dbg;
  int n;             // sequence length
  float scale_log2;  // softmax scale * log2(e)
  int p_round;       // fp32 P*V engines: round P to bf16 values first
};

// Key (0..31 inside a 32-key subtile) that row m of the K operand carries.
__device__ __forceinline__ int key_of_row(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}
// Key (0..31 inside a 32-key subtile) in accumulator register r of group g.
__device__ __forceinline__ int key_of_reg(int r, int g) {
  return 16 * (r >> 3) + 8 * g + (r & 7);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }

typedef __attribute__((address_space(3))) char lds_char;

// Byte offset, inside one tile, that lane `lane` of segment `seg` fills, as
// a source offset relative to the tile's first key row (or ~0 for padding
// slots, which the bounds-checked load turns into a harmless zero fill).
__device__ __forceinline__ uint32_t seg_src_offset(int seg, int lane, int row_bytes, int stride) {
  const int pos = (seg * 64 + lane) * 16;
  const int row = pos / stride, col = pos % stride;
  return col < row_bytes ? (uint32_t)(row * row_bytes + col) : 0x7ffffff0u;
}

// Issue this wave's share of the bounds-checked 16-byte buffer loads that
// fill K/V tile buffer `buf` with key rows kb..kb+63 (and, for int8, the 64
// key scales).  Asynchronous: completion is awaited with vmcnt before the
// workgroup barrier that publishes the tile.
template <int D, int QK, int PV>
__device__ __forceinline__ void issue_block(char* smem, int wave, int lane, int kb, int buf,
                                            const void* kbase, const void* vbase,
                                            const void* sbase, int n, const uint32_t* voffK,
                                            const uint32_t* voffV) {
  using TL = Tile<D, QK, PV>;
  // buffer resources spanning exactly this head: key rows >= n read as zeros
  const int nbK = n * TL::kRowK, nbV = n * TL::kRowV;
  const __amdgpu_buffer_rsrc_t rsK =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nbK, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsV =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nbV, 0x00020000);
  lds_char* lds = (lds_char*)smem;
#pragma unroll
  for (int i = 0; i < TL::kSegKPerWave; ++i) {
    const int seg = wave + i * kWaves;
    // (arguments go through locals: a template-dependent expression written
    // straight into this builtin makes clang's host pass drop the kernel)
    const int soff = kb * TL::kRowK;
    lds_char* dst = lds + (buf * TL::kBytesK + seg * 1024);
    if (TL::kSegK % kWaves == 0 || seg < TL::kSegK)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, dst, 16, voffK[i], soff, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < TL::kSegVPerWave; ++i) {
    const int seg = wave + i * kWaves;
    const int soff = kb * TL::kRowV;
    lds_char* dst = lds + (TL::kOffV + buf * TL::kBytesV + seg * 1024);
    if (TL::kSegV % kWaves == 0 || seg < TL::kSegV)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, dst, 16, voffV[i], soff, 0, 0);
  }
  if constexpr (QK == QK_I8) {
    const int nbS = n * 4;
    const __amdgpu_buffer_rsrc_t rsS =
        __builtin_amdgcn_make_buffer_rsrc((void*)sbase, (short)0, nbS, 0x00020000);
    const int soff = kb * 4;
    const uint32_t voff = lane * 4;
    lds_char* dst = lds + (TL::kOffSk + buf * TL::kBytesSk);
    if (wave == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsS, dst, 4, voff, soff, 0, 0);
  }
}

// Two waves per SIMD (two workgroups per CU) where the LDS tiles allow it.
template <int D, int QK, int PV>
constexpr int min_waves_per_simd() { return Tile<D, QK, PV>::kLds * 2 <= 160 * 1024 ? 2 : 1; }

template <int D, int QK, int PV, bool CAUSAL, bool DEBUG_S>
__global__ __launch_bounds__(kThreads, (min_waves_per_simd<D, QK, PV>()))
void flash_fwd_kernel(FlashParams p) {
  using QT = typename QKTraits<QK>::T;
  using VT = typename VTraits<PV>::T;
  using TL = Tile<D, QK, PV>;
  constexpr int DT = D / 32;  // 32-row d subtiles of O^T

  __shared__ __attribute__((aligned(1024))) char smem[TL::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int n = lane & 31;
  const int N = p.n;
  const int64_t bh = blockIdx.x;
  const int tile = CAUSAL ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int q0 = tile * kBR;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + n;
  const bool qvalid = qrow < N;
  const int64_t hoff = bh * (int64_t)N * D;
  const QT* Qg = (const QT*)p.q + hoff;

  // ---- this lane's query row as the B operand of S^T = K Q^T (registers)
  constexpr int QST = (QK == QK_BF16) ? D / 16 : (QK == QK_I8 ? D / 32 : D / 2);
  i32x4 qv[QK == QK_F32 ? 1 : QST];
  float qf[QK == QK_F32 ? QST : 1];
  float sq_log2 = 0.f;
  if constexpr (QK == QK_F32) {
#pragma unroll
    for (int t = 0; t < QST; ++t)
      qf[t] = qvalid ? Qg[(int64_t)qrow * D + 2 * t + g] : 0.f;
  } else {
    constexpr int EPC = 16 / (int)sizeof(QT);  // elements per 16-byte chunk
#pragma unroll
    for (int t = 0; t < QST; ++t) {
      const QT* src = Qg + (int64_t)qrow * D + 2 * EPC * t + EPC * g;
      qv[t] = qvalid ? *(const i32x4*)src : i32x4{0, 0, 0, 0};
    }
    if constexpr (QK == QK_I8)
      sq_log2 = qvalid ? p.q_scale[bh * N + qrow] * p.scale_log2 : 0.f;
  }

  // ---- K/V block streaming: bounds-checked buffer loads straight into LDS
  const void* kbase = (const char*)p.k + hoff * (int64_t)sizeof(QT);
  const void* vbase = (const char*)p.v + hoff * (int64_t)sizeof(VT);
  const void* sbase = (QK == QK_I8) ? (const void*)(p.k_scale + bh * N) : nullptr;
  uint32_t voffK[TL::kSegKPerWave], voffV[TL::kSegVPerWave];
#pragma unroll
  for (int i = 0; i < TL::kSegKPerWave; ++i)
    voffK[i] = seg_src_offset(wave + i * kWaves, lane, TL::kRowK, TL::kStrK);
#pragma unroll
  for (int i = 0; i < TL::kSegVPerWave; ++i)
    voffV[i] = seg_src_offset(wave + i * kWaves, lane, TL::kRowV, TL::kStrV);
  const int kend = CAUSAL ? min(N, q0 + kBR) : N;
  const int nblk = (kend + kBC - 1) / kBC;
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};

  // per-lane LDS byte offsets of the operand reads (block-independent)
  const int k_lane = key_of_row(n) * TL::kStrK;
  const int v_lane = (8 * g + ((lane & 15) >> 2)) * TL::kStrV +
                     (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * (int)sizeof(VT);

  issue_block<D, QK, PV>(smem, wave, lane, 0, 0, kbase, vbase, sbase, N, voffK, voffV);
  for (int j = 0; j < nblk; ++j) {
    const int kb = j * kBC;
    const int buf = j & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of block j landed
    __syncthreads();  // every wave's loads landed; every wave is done with block j-1
    if (j + 1 < nblk)
      issue_block<D, QK, PV>(smem, wave, lane, kb + kBC, buf ^ 1, kbase, vbase, sbase, N,
                             voffK, voffV);
    if (CAUSAL && kb > q0w + 31) continue;  // block entirely above this wave's diagonal

    const char* kt = (const char*)smem + buf * TL::kBytesK;
    const char* vt = (const char*)smem + TL::kOffV + buf * TL::kBytesV;

    // ---- S^T = K_j Q^T for two 32-key subtiles, in log2 units
    float s[2][16];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const char* krow = kt + ks * 32 * TL::kStrK + k_lane;
      if constexpr (QK == QK_BF16) {
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < QST; ++t) {
          const i32x4 a = *(const i32x4*)(krow + 32 * t + 16 * g);
          acc = mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qv[t]), acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[ks][r] = acc[r] * p.scale_log2;
      } else if constexpr (QK == QK_I8) {
        i32x16 acc = {};
#pragma unroll
        for (int t = 0; t < QST; ++t) {
          const i32x4 a = *(const i32x4*)(krow + 32 * t + 16 * g);
          acc = mfma_i8(a, qv[t], acc);
        }
        if constexpr (DEBUG_S) {
          if (qvalid) {
            int32_t* dst = p.s_dbg + (bh * N + qrow) * (int64_t)N;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb + 32 * ks + key_of_reg(r, g);
              if (key < N) dst[key] = acc[r];
            }
          }
        }
        const float* skt = (const float*)(smem + TL::kOffSk + buf * TL::kBytesSk);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[ks][r] = (float)acc[r] * (skt[32 * ks + key_of_reg(r, g)] * sq_log2);
      } else {
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < QST; ++t)
          acc = mfma_f32(*(const float*)(krow + 4 * (2 * t + g)), qf[t], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[ks][r] = acc[r] * p.scale_log2;
      }
    }

    // ---- causal diagonal and ragged tail: invisible keys score -inf
    const bool need_mask = (kb + kBC > N) || (CAUSAL && kb + kBC - 1 > q0w);
    if (need_mask) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * ks + key_of_reg(r, g);
          if (key >= N || (CAUSAL && key > qrow)) s[ks][r] = -INFINITY;
        }
    }

    // ---- online softmax: running max, rescale factor, P, running sum
    float mx = s[0][0];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[ks][r]);
    mx = pair32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_approx(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[ks][r] = exp2_approx(s[ks][r] - m_use);
        rs += s[ks][r];
      }
    l_run = l_run * alpha + rs;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }

    // ---- O^T += V_j^T P_j^T
    if constexpr (PV == PV_BF16) {
      bf16x8 pb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[u][e] = (__bf16)s[u >> 1][8 * (u & 1) + e];
      const char* vl = vt + v_lane;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const char* src = vl + 16 * u * TL::kStrV + 64 * dt;
          const i16x4 lo = lds_read_tr16(src);
          const i16x4 hi = lds_read_tr16(src + 4 * TL::kStrV);
          oacc[dt] = mfma_bf16(join_bf16x8(lo, hi), pb[u], oacc[dt]);
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = p.p_round ? round_to_bf16(s[ks][r]) : s[ks][r];
          const VT* vr = (const VT*)(vt + (32 * ks + key_of_reg(r, g)) * TL::kStrV) + n;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            oacc[dt] = mfma_f32(to_f32<VT>(vr[32 * dt]), pv, oacc[dt]);
        }
    }
  }

  // ---- epilogue: O = O^T / l, stored row-major; optional log-sum-exp
  const float l_tot = pair32_sum(l_run);
  const float inv = 1.f / l_tot;
  if (qvalid) {
    VT* dst = (VT*)p.o + hoff + (int64_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int d0 = 32 * dt + 8 * b4 + 4 * g;
        const float x0 = oacc[dt][4 * b4 + 0] * inv, x1 = oacc[dt][4 * b4 + 1] * inv;
        const float x2 = oacc[dt][4 * b4 + 2] * inv, x3 = oacc[dt][4 * b4 + 3] * inv;
        if constexpr (sizeof(VT) == 2) {
          uint2 w;
          w.x = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
          w.y = (uint32_t)f32_to_bf16(x2) | ((uint32_t)f32_to_bf16(x3) << 16);
          *(uint2*)(dst + d0) = w;
        } else {
          *(float4*)(dst + d0) = make_float4(x0, x1, x2, x3);
        }
      }
    if (p.lse != nullptr && g == 0)
      p.lse[bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, int QK, int PV, bool CAUSAL, bool DEBUG_S>
hipError_t launch_t(const FlashParams& fp, int64_t bh, int ntiles, hipStream_t st) {
  dim3 grid((unsigned)bh, (unsigned)ntiles, 1);
  hipLaunchKernelGGL((flash_fwd_kernel<D, QK, PV, CAUSAL, DEBUG_S>), grid, dim3(kThreads), 0,
                     st, fp);
  return hipGetLastError();
}

template <int D, int QK, int PV, bool DEBUG_S>
hipError_t launch_c(const FlashParams& fp, bool causal, int64_t bh, int nt, hipStream_t st) {
  return causal ? launch_t<D, QK, PV, true, DEBUG_S>(fp, bh, nt, st)
                : launch_t<D, QK, PV, false, DEBUG_S>(fp, bh, nt, st);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const FlashParams& fp, int64_t bh, int nt,
                    hipStream_t st) {
  const bool c = a.causal != 0;
  switch (a.dtype) {
    case kF32:
      return launch_c<D, QK_F32, PV_F32_VF32, false>(fp, c, bh, nt, st);
    case kBF16:
      return a.p_bf16 ? launch_c<D, QK_BF16, PV_BF16, false>(fp, c, bh, nt, st)
                      : launch_c<D, QK_BF16, PV_F32_VBF16, false>(fp, c, bh, nt, st);
    case kINT8:
      if (a.s_dbg != nullptr)
        return a.p_bf16 ? launch_c<D, QK_I8, PV_BF16, true>(fp, c, bh, nt, st)
                        : launch_c<D, QK_I8, PV_F32_VBF16, true>(fp, c, bh, nt, st);
      return a.p_bf16 ? launch_c<D, QK_I8, PV_BF16, false>(fp, c, bh, nt, st)
                      : launch_c<D, QK_I8, PV_F32_VBF16, false>(fp, c, bh, nt, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_flash(const AttnArgs& a, hipStream_t stream) {
  FlashParams fp;
  fp.q = a.q;
  fp.k = a.k;
  fp.v = a.v;
  fp.q_scale = a.q_scale;
  fp.k_scale = a.k_scale;
  fp.o = a.o;
  fp.lse = a.lse;
  fp.s_dbg = a.s_dbg;
  fp.n = (int)a.seq_len;
  fp.scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  fp.p_round = (a.dtype == kF32) ? a.p_bf16 : 0;
  const int64_t bh = a.batch * a.heads;
  const int ntiles = (int)((a.seq_len + kBR - 1) / kBR);
  if (a.head_dim == 64) return launch_d<64>(a, fp, bh, ntiles, stream);
  if (a.head_dim == 128) return launch_d<128>(a, fp, bh, ntiles, stream);
  return hipErrorInvalidValue;
}

}  // namespace pn
