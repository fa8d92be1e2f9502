// Baseline attention for gfx950: the score matrix is materialised in HBM.
//
// "Is Flash Attention Stable?" (abstract) compares FlashAttention with the
// plain, non-fused attention ("Baseline Attention") in an isolated forward
// pass.  Three kernels on one stream, each a separate pass over HBM:
//   K1 scores : S = scale * Q K^T for all N x N (query, key) pairs, fp32
//               (int8 Q/K: the exact int32 products Qc Kc^T, unscaled;
//               E4M3 fp8 Q/K: the fp32 products of the codes, unscaled)
//   K2 softmax: per row, the causal mask, the row max, exp, the row sum and
//               the normalised P = e / sum in fp32, stored as bf16 (RNE) or
//               fp32
//   K3 pv     : O = P V with fp32 accumulation (bf16 MFMA when P and V are
//               both bf16, fp32 MFMA otherwise)
// The kernels are HBM-bound by design (about 12 bytes of traffic per score
// element with bf16 P); the naive path computes and stores every one of the
// N^2 entries, masked or not.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace pn {
namespace {

constexpr int kThreads = 256;
// bytes after P in the workspace: the P.V kernel's 16-byte loads may run up
// to 15 bytes past the last row
constexpr size_t kWorkspaceTail = 256;

// ---------------------------------------------------------------------------
// K1: S tile of 128 queries x 128 keys per workgroup; wave w owns 32 query
// rows and all 128 keys (4 MFMA tiles).  The wave's Q rows come straight
// from global memory into registers (16-byte loads along d); the K tile is
// loaded once per workgroup into LDS (buffer loads straight into LDS, rows
// padded by 16 bytes so that the 32 lanes reading one 16-byte column of 32
// rows hit distinct banks) and read from there by all four waves -- read
// from global memory by every wave, the K rows were 2.5 bytes of L2 traffic
// per byte of S written and the kernel's bound.  The output leaves in
// 128-byte row segments.
// ---------------------------------------------------------------------------
// Workgroup -> (head, tile of the head).  Workgroups go to the eight XCDs in
// turn (linear dispatch index mod 8); when the head count is a multiple of
// eight, head 8c + x takes the slots c*T .. (c+1)*T - 1 of XCD x, so every
// tile of a head runs on one XCD and the K and V rows its tiles share are
// fetched from HBM into that XCD's L2 once (in dispatch order the tiles of
// a head would go to all eight).  Any other head count: head-major order.
__device__ __forceinline__ void head_tile(int64_t tiles_per_head, int64_t heads, int64_t& head,
                                          int64_t& tile) {
  const int64_t L = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  if (heads % 8 == 0) {
    const int64_t i = L >> 3;
    head = (i / tiles_per_head) * 8 + (L & 7);
    tile = i % tiles_per_head;
  } else {
    head = L / tiles_per_head;
    tile = L % tiles_per_head;
  }
}

template <int D, int QK> struct ScoresLds {
  static constexpr int kRow = QK == 0 ? 2 * D : D;  // bytes per K row (8/16-bit codes)
  static constexpr int kStr = kRow + 16;            // padded LDS row
  static constexpr int kBytes = QK == 2 ? 16 : 128 * kStr;
  static constexpr int kSeg = kBytes / 1024;
};

template <int D, int QK>  // QK: 0 bf16, 1 int8, 2 fp32, 3 E4M3 fp8
__global__ __launch_bounds__(kThreads) void scores_kernel(const void* qp, const void* kp,
                                                         void* sp, int N, float scale) {
  using SL = ScoresLds<D, QK>;
  __shared__ __attribute__((aligned(1024))) char kt[SL::kBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, n = lane & 31;
  int64_t bh, tile;
  head_tile((int64_t)gridDim.x * gridDim.y, gridDim.z, bh, tile);
  const int i0 = (int)(tile / gridDim.x) * 128 + wave * 32;
  const int j0 = (int)(tile % gridDim.x) * 128;
  const int64_t hoff = bh * (int64_t)N * D;
  const int qi = i0 + n;  // A-operand row of this lane
  if constexpr (QK == 0 || QK == 1 || QK == 3) {
    using T = typename std::conditional<QK == 0, uint16_t, int8_t>::type;
    constexpr int EPC = 16 / (int)sizeof(T);
    constexpr int ST = D / (2 * EPC);
    static_assert(SL::kBytes % 1024 == 0, "the K tile is whole load segments");
    const T* Q = (const T*)qp + hoff;
    const T* K = (const T*)kp + hoff;
    i32x4 a[ST];
#pragma unroll
    for (int t = 0; t < ST; ++t)
      a[t] = qi < N ? *(const i32x4*)(Q + (int64_t)qi * D + 2 * EPC * t + EPC * g)
                    : i32x4{0, 0, 0, 0};
    // K rows j0 .. j0 + 127 into LDS (rows past N arrive as zeros through
    // the buffer range check; their scores are not stored)
    {
      const i32x4 rs = buffer_rsrc(K, (uint32_t)N * SL::kRow);
      for (int sg = wave; sg < SL::kSeg; sg += kThreads / 64)
        lds_load16<0>(rs, seg_src_offset(sg, lane, SL::kRow, SL::kStr), (uint32_t)j0 * SL::kRow,
                      lds_address(kt) + sg * 1024);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int kj = j0 + 32 * jt + n;  // B-operand column of this lane
      using Acc = typename std::conditional<QK == 1, i32x16, f32x16>::type;
      Acc acc = {};
      const char* krow = kt + (32 * jt + n) * SL::kStr + 16 * g;
#pragma unroll
      for (int t = 0; t < ST; ++t) {
        const i32x4 b = *(const i32x4*)(krow + 32 * t);
        if constexpr (QK == 0)
          acc = mfma_bf16(__builtin_bit_cast(bf16x8, a[t]), __builtin_bit_cast(bf16x8, b), acc);
        else if constexpr (QK == 1)
          acc = mfma_i8(a[t], b, acc);
        else
          acc = mfma_fp8x2(a[t], b, acc);
      }
      if (kj < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (i < N) {
            const int64_t off = (bh * N + i) * (int64_t)N + kj;
            // S is written once and read once, far beyond any cache:
            // non-temporal stores
            if constexpr (QK == 0)
              __builtin_nontemporal_store(acc[r] * scale, (float*)sp + off);
            else if constexpr (QK == 1)
              __builtin_nontemporal_store((int32_t)acc[r], (int32_t*)sp + off);
            else
              __builtin_nontemporal_store((float)acc[r], (float*)sp + off);  // unscaled; K2 applies the row scales
          }
        }
      }
    }
  } else {
    const float* Q = (const float*)qp + hoff;
    const float* K = (const float*)kp + hoff;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int kj = j0 + 32 * jt + n;
      f32x16 acc = {};
      for (int t = 0; t < D / 2; ++t) {
        const float a = qi < N ? Q[(int64_t)qi * D + 2 * t + g] : 0.f;
        const float b = kj < N ? K[(int64_t)kj * D + 2 * t + g] : 0.f;
        acc = mfma_f32(a, b, acc);
      }
      if (kj < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (i < N) ((float*)sp)[(bh * N + i) * (int64_t)N + kj] = acc[r] * scale;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K2: one workgroup per score row: mask, max, exp, sum, normalise, store P.
// Fixed thread-to-element map and reduction tree: deterministic.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// SMODE: 0 scores already scaled (fp32), 1 int32 products of int8 codes,
// 2 fp32 products of E4M3 codes; 1 and 2 apply scale * sq_i * sk_j here.
// CACHE > 0 (rows of at most CACHE * kThreads entries): each thread keeps
// its scores in registers, so the row is read from HBM once instead of
// three times; the order of every operation is the same either way, so
// both forms give the same bits.
template <int SMODE, bool PBF16, int CACHE>
__global__ __launch_bounds__(kThreads) void softmax_kernel(const void* sp, void* pp,
                                                          const float* q_scale,
                                                          const float* k_scale, int N,
                                                          int causal, float scale) {
  __shared__ float red[kThreads / 64];
  const int i = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t row = (bh * N + i) * (int64_t)N;
  const int jend = causal ? i + 1 : N;  // visible keys: j < jend
  const float sqc = SMODE != 0 ? q_scale[bh * N + i] * scale : 0.f;
  // S: read once (non-temporal)
  auto score = [&](int j) -> float {
    if constexpr (SMODE == 1)
      return (float)__builtin_nontemporal_load((const int32_t*)sp + row + j) *
             (k_scale[bh * N + j] * sqc);
    else if constexpr (SMODE == 2)
      return __builtin_nontemporal_load((const float*)sp + row + j) * (k_scale[bh * N + j] * sqc);
    else
      return __builtin_nontemporal_load((const float*)sp + row + j);
  };
  auto store = [&](int j, float pv) {
    // P: written once, read once by K3 (non-temporal)
    if constexpr (PBF16)
      __builtin_nontemporal_store(f32_to_bf16(pv), (uint16_t*)pp + row + j);
    else
      __builtin_nontemporal_store(pv, (float*)pp + row + j);
  };
  float m = -INFINITY;
  if constexpr (CACHE > 0) {
    float x[CACHE];
#pragma unroll
    for (int c = 0; c < CACHE; ++c) {
      const int j = (int)threadIdx.x + c * kThreads;
      x[c] = j < jend ? score(j) : -INFINITY;
      m = fmaxf(m, x[c]);
    }
    m = block_reduce(m, true, red);
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < CACHE; ++c) {
      x[c] = exp2_approx((x[c] - m) * kLog2e);  // 0 past jend
      if ((int)threadIdx.x + c * kThreads < jend) sum += x[c];
    }
    sum = block_reduce(sum, false, red);
    const float inv = 1.f / sum;
#pragma unroll
    for (int c = 0; c < CACHE; ++c) {
      const int j = (int)threadIdx.x + c * kThreads;
      if (j < N) store(j, j < jend ? x[c] * inv : 0.f);
    }
  } else {
    for (int j = threadIdx.x; j < jend; j += kThreads) m = fmaxf(m, score(j));
    m = block_reduce(m, true, red);
    float sum = 0.f;
    for (int j = threadIdx.x; j < jend; j += kThreads)
      sum += exp2_approx((score(j) - m) * kLog2e);
    sum = block_reduce(sum, false, red);
    const float inv = 1.f / sum;
    for (int j = threadIdx.x; j < N; j += kThreads)
      store(j, j < jend ? exp2_approx((score(j) - m) * kLog2e) * inv : 0.f);
  }
}

// ---------------------------------------------------------------------------
// K3: O = P V.  Workgroup = 128 query rows (4 waves x 32); keys in blocks of
// 64 staged in LDS (P tile and V tile, both row-major).  Each wave forms
// O^T = V^T P^T: V^T through the transposing LDS read, P^T straight from its
// row-major tile.
// ---------------------------------------------------------------------------
template <int D, typename PT, typename VT, typename OT>
__global__ __launch_bounds__(kThreads) void pv_kernel(const void* pp, const void* vp, void* op,
                                                     int N) {
  constexpr bool BF16MMA = sizeof(PT) == 2 && sizeof(VT) == 2;
  constexpr int PS = 64 + 16 / (int)sizeof(PT);                 // P tile row stride
  constexpr int VS = D + (sizeof(VT) == 2 ? 32 : 4);            // V tile row stride
  constexpr int PCPR = 64 * (int)sizeof(PT) / 16, PCH = 128 * PCPR / kThreads;
  constexpr int VCPR = D * (int)sizeof(VT) / 16, VCH = 64 * VCPR / kThreads;
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(16))) PT p_lds[128 * PS];
  __shared__ __attribute__((aligned(16))) VT v_lds[64 * VS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  int64_t bh, tile;
  head_tile(gridDim.x, gridDim.y, bh, tile);
  const int q0 = (int)tile * 128;
  const PT* P = (const PT*)pp + bh * (int64_t)N * N;
  const VT* V = (const VT*)vp + bh * (int64_t)N * D;
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  constexpr int EPC_P = 16 / (int)sizeof(PT);
  for (int kb = 0; kb < N; kb += 64) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PCH; ++i) {
      const int c = tid + i * kThreads, row = c / PCPR, col = c % PCPR;
      const int q = q0 + row, key = kb + EPC_P * col;
      i32x4 val = {0, 0, 0, 0};
      if (q < N) {
        const PT* src = P + (int64_t)q * N + key;
        if (key + EPC_P <= N && (((uintptr_t)src) & 15) == 0) {
          val = *(const i32x4*)src;
        } else {
          PT tmp[EPC_P];
#pragma unroll
          for (int e = 0; e < EPC_P; ++e) tmp[e] = key + e < N ? src[e] : PT(0);
          __builtin_memcpy(&val, tmp, 16);
        }
      }
      *(i32x4*)((char*)(p_lds + row * PS) + 16 * col) = val;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + i * kThreads, row = c / VCPR, col = c % VCPR;
      const int key = kb + row;
      *(i32x4*)((char*)(v_lds + row * VS) + 16 * col) =
          key < N ? *(const i32x4*)((const char*)(V + (int64_t)key * D) + 16 * col)
                  : i32x4{0, 0, 0, 0};
    }
    __syncthreads();
    const PT* prow = p_lds + (32 * wave + n) * PS;
    if constexpr (BF16MMA) {
      const int vrow = 8 * g + ((lane & 15) >> 2);
      const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, *(const i32x4*)(prow + 16 * u + 8 * g));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const VT* src = v_lds + (16 * u + vrow) * VS + 32 * dt + vcol;
          oacc[dt] = mfma_bf16(join_bf16x8(lds_read_tr16(src), lds_read_tr16(src + 4 * VS)), pb,
                               oacc[dt]);
        }
      }
    } else {
      for (int t = 0; t < 32; ++t) {
        const int key = 2 * t + g;
        float pv;
        if constexpr (sizeof(PT) == 2) pv = bf16_to_f32(prow[key]);
        else pv = prow[key];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          float vv;
          if constexpr (sizeof(VT) == 2) vv = bf16_to_f32(v_lds[key * VS + 32 * dt + n]);
          else vv = v_lds[key * VS + 32 * dt + n];
          oacc[dt] = mfma_f32(vv, pv, oacc[dt]);
        }
      }
    }
  }
  const int q = q0 + 32 * wave + n;
  if (q < N) {
    OT* dst = (OT*)op + (bh * N + q) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int d0 = 32 * dt + 8 * b4 + 4 * g;
        const float x0 = oacc[dt][4 * b4], x1 = oacc[dt][4 * b4 + 1];
        const float x2 = oacc[dt][4 * b4 + 2], x3 = oacc[dt][4 * b4 + 3];
        if constexpr (sizeof(OT) == 2) {
          uint2 w;
          w.x = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
          w.y = (uint32_t)f32_to_bf16(x2) | ((uint32_t)f32_to_bf16(x3) << 16);
          *(uint2*)(dst + d0) = w;
        } else {
          *(float4*)(dst + d0) = make_float4(x0, x1, x2, x3);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// K3 for bf16 P and bf16 V: the same product O^T = V^T P^T, with the P and V
// blocks of 64 keys streamed through two LDS buffers by buffer loads straight
// into LDS -- block k + 1 loads while block k's products run, one barrier
// per step.  P rows are gathered from their stride-N rows in HBM (padded by
// 16 bytes in LDS: conflict-free 16-byte column reads of 32 rows); V rows
// are padded by 64 bytes for the transposing reads.
// ---------------------------------------------------------------------------
template <int D> struct PvLds {
  static constexpr int kBK = 64;                // keys per step
  static constexpr int kPRow = 2 * kBK;         // bytes of a P row per step
  static constexpr int kPStr = kPRow + 16;
  static constexpr int kPBytes = 128 * kPStr;   // 128 query rows
  static constexpr int kVRow = 2 * D;
  static constexpr int kVStr = kVRow + 64;
  static constexpr int kVBytes = kBK * kVStr;
  static constexpr int kPSeg = kPBytes / 1024, kVSeg = kVBytes / 1024;
  static constexpr int kPPer = (kPSeg + 3) / 4, kVPer = (kVSeg + 3) / 4;
  static constexpr int kBuf = kPBytes + kVBytes;
  static_assert(kPBytes % 1024 == 0 && kVBytes % 1024 == 0, "whole load segments");
};

template <int D, typename OT>
__global__ __launch_bounds__(kThreads) void pv_bf16_kernel(const void* pp, const void* vp, void* op,
                                                          int N) {
  using L = PvLds<D>;
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[2 * L::kBuf];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  int64_t bh, tile;
  head_tile(gridDim.x, gridDim.y, bh, tile);
  const int q0 = (int)tile * 128;
  const int rows = min(128, N - q0);
  // P rows q0 .. q0 + rows - 1 of this head (2N bytes each); V rows of the head
  const char* Pg = (const char*)pp + ((bh * N + q0) * (int64_t)N) * 2;
  const char* Vg = (const char*)vp + bh * (int64_t)N * D * 2;
  // Buffer loads check their range a dword at a time, so a 16-byte chunk
  // crossing the end of the tile's rows would come back partly zero: the
  // range runs to the next 16-byte boundary (the next row's first values, or
  // the workspace's tail padding after the last row; columns past N are
  // masked below, rows past N never stored).
  const i32x4 rsP = buffer_rsrc(Pg, ((uint32_t)rows * (uint32_t)N * 2 + 15u) & ~15u);
  const i32x4 rsV = buffer_rsrc(Vg, (uint32_t)N * L::kVRow);
  // per-lane source offsets of this wave's segments (block-independent)
  uint32_t offP[L::kPPer], offV[L::kVPer];
#pragma unroll
  for (int i = 0; i < L::kPPer; ++i) {
    const int pos = ((wave + 4 * i) * 64 + lane) * 16;
    const int r = pos / L::kPStr, c = pos % L::kPStr;
    offP[i] = c < L::kPRow ? (uint32_t)r * (uint32_t)N * 2 + c : 0x7ffffff0u;
  }
#pragma unroll
  for (int i = 0; i < L::kVPer; ++i) offV[i] = seg_src_offset(wave + 4 * i, lane, L::kVRow, L::kVStr);
  auto issue = [&](int kb, int buf) __attribute__((always_inline)) {
    const uint32_t base = lds_address(smem) + buf * L::kBuf + wave * 1024;
#pragma unroll
    for (int i = 0; i < L::kPPer; ++i)
      if (wave + 4 * i < L::kPSeg) lds_load16<0>(rsP, offP[i], (uint32_t)kb * 2, base + i * 4096);
#pragma unroll
    for (int i = 0; i < L::kVPer; ++i)
      if (wave + 4 * i < L::kVSeg)
        lds_load16<0>(rsV, offV[i], (uint32_t)kb * L::kVRow, base + L::kPBytes + i * 4096);
  };
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  const int vrow = 8 * g + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int steps = (N + L::kBK - 1) / L::kBK;
  issue(0, 0);
  for (int st = 0; st < steps; ++st) {
    const int kb = st * L::kBK;
    // block st landed for every wave; every wave is done with block st - 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (st + 1 < steps) issue(kb + L::kBK, (st + 1) & 1);
    const char* pl = smem + (st & 1) * L::kBuf + (32 * wave + n) * L::kPStr + 16 * g;
    const char* vl = smem + (st & 1) * L::kBuf + L::kPBytes;
    const bool tail = kb + L::kBK > N;  // P columns past N hold the next row's values
#pragma unroll
    for (int u = 0; u < L::kBK / 16; ++u) {
      i32x4 pw = *(const i32x4*)(pl + 32 * u);
      if (tail) {
        // keys kb + 16u + 8g + e: zero past N (V rows there are zeros, but
        // 0 * a non-finite P would not be)
        const int k0 = kb + 16 * u + 8 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t w = (uint32_t)pw[e];
          if (k0 + 2 * e >= N) w &= 0xffff0000u;
          if (k0 + 2 * e + 1 >= N) w &= 0x0000ffffu;
          pw[e] = (int)w;
        }
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const char* src = vl + (16 * u + vrow) * L::kVStr + (32 * dt + vcol) * 2;
        oacc[dt] = mfma_bf16(join_bf16x8(lds_read_tr16(src), lds_read_tr16(src + 4 * L::kVStr)), pb,
                             oacc[dt]);
      }
    }
  }
  const int q = q0 + 32 * wave + n;
  if (q < N) {
    OT* dst = (OT*)op + (bh * N + q) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        const int d0 = 32 * dt + 8 * b4 + 4 * g;
        const float x0 = oacc[dt][4 * b4], x1 = oacc[dt][4 * b4 + 1];
        const float x2 = oacc[dt][4 * b4 + 2], x3 = oacc[dt][4 * b4 + 3];
        if constexpr (sizeof(OT) == 2) {
          uint2 w;
          w.x = (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
          w.y = (uint32_t)f32_to_bf16(x2) | ((uint32_t)f32_to_bf16(x3) << 16);
          *(uint2*)(dst + d0) = w;
        } else {
          *(float4*)(dst + d0) = make_float4(x0, x1, x2, x3);
        }
      }
  }
}

template <int D>
hipError_t launch_scores(const AttnArgs& a, void* s, hipStream_t st) {
  const int N = (int)a.seq_len;
  const int t = (N + 127) / 128;
  dim3 grid(t, t, (unsigned)(a.batch * a.heads));
  if (a.dtype == kBF16)
    hipLaunchKernelGGL((scores_kernel<D, 0>), grid, dim3(kThreads), 0, st, a.q, a.k, s, N, a.scale);
  else if (a.dtype == kINT8)
    hipLaunchKernelGGL((scores_kernel<D, 1>), grid, dim3(kThreads), 0, st, a.q, a.k, s, N, a.scale);
  else if (a.dtype == kFP8)
    hipLaunchKernelGGL((scores_kernel<D, 3>), grid, dim3(kThreads), 0, st, a.q, a.k, s, N, a.scale);
  else
    hipLaunchKernelGGL((scores_kernel<D, 2>), grid, dim3(kThreads), 0, st, a.q, a.k, s, N, a.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pv(const AttnArgs& a, const void* p, hipStream_t st) {
  const int N = (int)a.seq_len;
  dim3 grid((N + 127) / 128, (unsigned)(a.batch * a.heads));
  const bool vf32 = a.dtype == kF32;
  const bool of32 = vf32 || a.o_f32;  // fp32 V always gives fp32 O
  // The streamed kernel needs 16-byte aligned P rows (N a multiple of 8);
  // other lengths take the register-staged one, which loads unaligned rows
  // element by element.
  const bool aligned = N % 8 == 0;
  if (a.p_bf16 && !vf32 && !of32 && aligned)
    hipLaunchKernelGGL((pv_bf16_kernel<D, uint16_t>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  else if (a.p_bf16 && !vf32 && aligned)
    hipLaunchKernelGGL((pv_bf16_kernel<D, float>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  else if (a.p_bf16 && !vf32 && !of32)
    hipLaunchKernelGGL((pv_kernel<D, uint16_t, uint16_t, uint16_t>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  else if (a.p_bf16 && !vf32)
    hipLaunchKernelGGL((pv_kernel<D, uint16_t, uint16_t, float>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  else if (a.p_bf16)
    hipLaunchKernelGGL((pv_kernel<D, uint16_t, float, float>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  else if (!vf32 && !of32)
    hipLaunchKernelGGL((pv_kernel<D, float, uint16_t, uint16_t>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  else if (!vf32)
    hipLaunchKernelGGL((pv_kernel<D, float, uint16_t, float>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  else
    hipLaunchKernelGGL((pv_kernel<D, float, float, float>), grid, dim3(kThreads), 0, st, p, a.v, a.o, N);
  return hipGetLastError();
}

template <int CACHE>
hipError_t launch_softmax(int mode, const AttnArgs& a, const void* s, void* p, dim3 grid,
                          hipStream_t st) {
  const int N = (int)a.seq_len;
  if (mode == 1 && a.p_bf16)
    hipLaunchKernelGGL((softmax_kernel<1, true, CACHE>), grid, dim3(kThreads), 0, st, s, p, a.q_scale, a.k_scale, N, a.causal, a.scale);
  else if (mode == 1)
    hipLaunchKernelGGL((softmax_kernel<1, false, CACHE>), grid, dim3(kThreads), 0, st, s, p, a.q_scale, a.k_scale, N, a.causal, a.scale);
  else if (mode == 2 && a.p_bf16)
    hipLaunchKernelGGL((softmax_kernel<2, true, CACHE>), grid, dim3(kThreads), 0, st, s, p, a.q_scale, a.k_scale, N, a.causal, a.scale);
  else if (mode == 2)
    hipLaunchKernelGGL((softmax_kernel<2, false, CACHE>), grid, dim3(kThreads), 0, st, s, p, a.q_scale, a.k_scale, N, a.causal, a.scale);
  else if (a.p_bf16)
    hipLaunchKernelGGL((softmax_kernel<0, true, CACHE>), grid, dim3(kThreads), 0, st, s, p, a.q_scale, a.k_scale, N, a.causal, a.scale);
  else
    hipLaunchKernelGGL((softmax_kernel<0, false, CACHE>), grid, dim3(kThreads), 0, st, s, p, a.q_scale, a.k_scale, N, a.causal, a.scale);
  return hipGetLastError();
}

}  // namespace

size_t baseline_workspace_bytes(int64_t bh, int64_t n, int p_bf16) {
  const size_t elems = (size_t)bh * (size_t)n * (size_t)n;
  return elems * 4 + elems * (p_bf16 ? 2 : 4) + kWorkspaceTail;
}

hipError_t launch_baseline(const AttnArgs& a, void* workspace, hipStream_t st) {
  const int64_t bh = a.batch * a.heads;
  const int N = (int)a.seq_len;
  void* s = workspace;
  void* p = (char*)workspace + (size_t)bh * N * (size_t)N * 4;
  hipError_t e = a.head_dim == 64 ? launch_scores<64>(a, s, st) : launch_scores<128>(a, s, st);
  if (e != hipSuccess) return e;
  dim3 grid2((unsigned)N, (unsigned)bh);
  const int mode = a.dtype == kINT8 ? 1 : (a.dtype == kFP8 ? 2 : 0);
  if (N <= 8 * kThreads)
    e = launch_softmax<8>(mode, a, s, p, grid2, st);
  else if (N <= 32 * kThreads)
    e = launch_softmax<32>(mode, a, s, p, grid2, st);
  else
    e = launch_softmax<0>(mode, a, s, p, grid2, st);
  if (e != hipSuccess) return e;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.head_dim == 64 ? launch_pv<64>(a, p, st) : launch_pv<128>(a, p, st);
}

}  // namespace pn
