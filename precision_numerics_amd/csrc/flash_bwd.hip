// FlashAttention backward for bf16 on gfx950: dQ, dK, dV from Q, K, V, the
// stored output O, its upstream gradient dO and the forward's log-sum-exp.
//
// Chain rule through O = P V, P = row-softmax(S), S = scale Q K^T:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),  delta = rowsum(dO o O)
//   dQ = scale dS K,  dK = scale dS^T Q
// ("Why Low-Precision Transformer Training Fails": delta = rowsum(dO o O) in
// the Figure 5 caption; the section isolating the error in O forms delta
// from the stored low-precision O, as here).  P is recomputed block by
// block as exp2(scale log2(e) q.k - lse log2(e)) from the forward's lse, so
// no N x N matrix is stored.
//
// Precision (the usual bf16 FlashAttention backward): the products run on
// bf16 MFMA with fp32 accumulation; P is rounded to bf16 for dV and dS for
// dQ and dK; P, dP, dS themselves are fp32; dQ, dK, dV leave as bf16 (RNE).
//
// Two deterministic kernels (no atomics: every output element is summed by
// one lane in a fixed order):
//   dq kernel : a workgroup owns 128 query rows (32 per wave, a lane per
//               query) and walks the key blocks: S^T = K Q^T and
//               dP^T = V dO^T (K and V rows fed in a permuted order so that
//               accumulator register r of lane group g holds key
//               16(r/8) + 8g + r%8, the order the dS^T operand of the next
//               product needs), then dQ^T += K^T dS^T with K^T read
//               through the transposing LDS read.
//   dkv kernel: a workgroup owns 128 key rows (a lane per key) and walks the
//               query blocks: S = Q K^T and dP = dO V^T with permuted query
//               rows, then dV^T += dO^T P and dK^T += Q^T dS.
// The blocks of the other operand stream through two LDS buffers by
// buffer-to-LDS loads: the loads of block j + 1 run while block j's
// products do (zeros past N); the per-row lse and delta of a query block
// sit in LDS beside it.
#include "device.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace pn {
namespace {

constexpr int kThreads = 256;   // four waves
constexpr int kTile = 128;      // rows a workgroup owns (32 per wave)
// Rows of the other operand per step: 32 for the dq kernel, whose registers
// then fit two workgroups per compute unit (two waves per SIMD, one
// covering the other's latencies), 64 for the dkv kernel, whose two output
// accumulators keep it at one wave per SIMD anyway.
constexpr int kStepDq = 32;
constexpr int kStepDkv = 64;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* d_o;
  const float* lse;
  const float* delta;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int n;
  int tiles;          // 128-row tiles per head
  int bh_count;       // batch * heads
  float scale;
  float scale_log2;   // scale * log2(e)
};

// Row m of a 32-row A operand carries element perm_row(m) of its subtile;
// then accumulator register r of lane group g holds element elem_of_reg(r, g).
__device__ __forceinline__ int perm_row(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}
__device__ __forceinline__ int elem_of_reg(int r, int g) { return 16 * (r >> 3) + 8 * g + (r & 7); }

// Workgroup -> (head, tile).  Causal tiles differ in length (the dkv
// kernel's tile t walks N - 128 t queries, the dq kernel's 128 (t + 1)
// keys), so they go out longest first, every head's tile of one length
// together: the short ones then fill the machine at the end instead of a
// few long ones running alone.  Without the mask all tiles are equal and
// a head's tiles go out together.
template <bool CAUSAL, bool LONG_FIRST_LOW>
__device__ __forceinline__ void tile_of(const BwdParams& p, int64_t& bh, int& tile) {
  const int64_t b = blockIdx.x;
  if constexpr (CAUSAL) {
    const int t = (int)(b / p.bh_count);
    bh = b - (int64_t)t * p.bh_count;
    tile = LONG_FIRST_LOW ? t : p.tiles - 1 - t;
  } else {
    bh = b / p.tiles;
    tile = (int)(b - bh * p.tiles);
  }
}

template <int D, int STEP> struct Geo {
  static constexpr int kRow = D * 2;         // bf16 row bytes
  // Each block sits in LDS twice, with two row paddings: 16 bytes for the
  // row reads of the A operands (16 lanes read one 16-byte column of 16
  // rows: the rows then fall on distinct banks) and 64 bytes for the
  // transposing reads (lanes read 8-byte pieces of four rows, 64 bytes
  // apart within each row).
  static constexpr int kStrA = kRow + 16;
  static constexpr int kStrB = kRow + 64;
  // 1 KB load segments per copy, and the copy's LDS bytes (whole segments)
  static constexpr int kSegA = (STEP * kStrA + 1023) / 1024;
  static constexpr int kSegB = (STEP * kStrB + 1023) / 1024;
  static constexpr int kBytesA = kSegA * 1024;
  static constexpr int kBytesB = kSegB * 1024;
  static constexpr int QST = D / 16;         // 16-element chunks of a row
  static constexpr int DT = D / 32;          // 32-row subtiles of a transposed output
};

template <int I> struct Slot { static constexpr int value = I; };
template <bool B> struct Flag { static constexpr bool value = B; };

// f(Slot<0>{}), ..., f(Slot<N-1>{}): a loop whose index is a constant
template <int N, int I = 0, typename F>
__device__ __forceinline__ void for_slots(F&& f) {
  if constexpr (I < N) {
    f(Slot<I>{});
    for_slots<N, I + 1>(f);
  }
}

// This wave's share of the buffer-to-LDS loads that fill the two LDS copies
// of a STEP-row block of a [N][D] bf16 matrix: segments w, w + 4, .. of each
// copy, with each lane's source offset inside the block (rows past N read
// zeros through the buffer range check).  Asynchronous: the loads are
// awaited by an explicit s_waitcnt vmcnt(0) before the barrier that
// publishes the block.
template <int D, int STEP> struct BlockDma {
  using G = Geo<D, STEP>;
  static constexpr int kPerA = (G::kSegA + 3) / 4;
  static constexpr int kPerB = (G::kSegB + 3) / 4;
  uint32_t offA[kPerA], offB[kPerB];
  int wave;
  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < kPerA; ++i) offA[i] = seg_src_offset(w + 4 * i, lane, G::kRow, G::kStrA);
#pragma unroll
    for (int i = 0; i < kPerB; ++i) offB[i] = seg_src_offset(w + 4 * i, lane, G::kRow, G::kStrB);
  }
  // rows r0.. into the row-read copy at LDS address lds_a and, if B_COPY,
  // the transposing-read copy at lds_b
  template <bool B_COPY>
  __device__ __forceinline__ void issue(i32x4 rs, int r0, uint32_t lds_a, uint32_t lds_b) const {
    const uint32_t soff = (uint32_t)r0 * G::kRow;
    for_slots<kPerA>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if (4 * i + 3 < G::kSegA || wave + 4 * i < G::kSegA)
        lds_load16<i * 4096>(rs, offA[i], soff, lds_a + wave * 1024);
    });
    if constexpr (B_COPY) {
      for_slots<kPerB>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if (4 * i + 3 < G::kSegB || wave + 4 * i < G::kSegB)
          lds_load16<i * 4096>(rs, offB[i], soff, lds_b + wave * 1024);
      });
    }
  }
};

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Make the row registers' values needed here (the compiler then waits for
// their loads at this point).
template <int N>
__device__ __forceinline__ void settle(i32x4 (&x)[N]) {
#pragma unroll
  for (int t = 0; t < N; ++t) asm volatile("" : "+v"(x[t]));
}

// a row of the B operand (16 bytes per 16-element chunk, lane group g holds
// elements 8g..8g+7 of each chunk)
template <int D> using RowRegs = i32x4[D / 16];
template <int D> using TileAcc = f32x16[D / 32];

template <int D>
__device__ __forceinline__ void load_row(RowRegs<D>& dst, const uint16_t* row, bool ok, int g) {
#pragma unroll
  for (int t = 0; t < Geo<D, 64>::QST; ++t)
    dst[t] = ok ? *(const i32x4*)(row + 16 * t + 8 * g) : i32x4{0, 0, 0, 0};
}

// store 32 lanes' transposed accumulators (register r of tile dt: element
// 32 dt + 8(r/4) + 4g + r%4 of this lane's row), times `mul`, as bf16
template <int D>
__device__ __forceinline__ void store_row(uint16_t* dst, const TileAcc<D>& acc, float mul,
                                          int g) {
#pragma unroll
  for (int dt = 0; dt < Geo<D, 64>::DT; ++dt)
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      const int d0 = 32 * dt + 8 * b4 + 4 * g;
      uint2 w;
      w.x = (uint32_t)f32_to_bf16(acc[dt][4 * b4 + 0] * mul) |
            ((uint32_t)f32_to_bf16(acc[dt][4 * b4 + 1] * mul) << 16);
      w.y = (uint32_t)f32_to_bf16(acc[dt][4 * b4 + 2] * mul) |
            ((uint32_t)f32_to_bf16(acc[dt][4 * b4 + 3] * mul) << 16);
      *(uint2*)(dst + d0) = w;
    }
}

// lanes' LDS byte offsets: permuted A-operand rows, and the transposing read
template <int D>
__device__ __forceinline__ int row_lane(int n) { return perm_row(n) * Geo<D, 64>::kStrA; }
template <int D>
__device__ __forceinline__ int tr_lane(int lane) {
  const int g = lane >> 5;
  return (8 * g + ((lane & 15) >> 2)) * Geo<D, 64>::kStrB +
         (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int kStep = kStepDq;
  using G = Geo<D, kStep>;
  // two buffers, each: K and V blocks for the row reads, K again for the
  // transposing reads
  constexpr int kBuf = 2 * G::kBytesA + G::kBytesB;
  __shared__ __attribute__((aligned(16))) char smem[2 * kBuf];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int N = p.n;
  int64_t bh;
  int tile;
  tile_of<CAUSAL, false>(p, bh, tile);
  const int q0 = tile * kTile;
  const int qrow = q0 + wave * 32 + n;
  const bool qok = qrow < N;
  const int64_t hoff = bh * (int64_t)N * D;
  i32x4 qv[G::QST], gv[G::QST];
  load_row<D>(qv, p.q + hoff + (int64_t)qrow * D, qok, g);
  load_row<D>(gv, p.d_o + hoff + (int64_t)qrow * D, qok, g);
  float lse2 = qok ? p.lse[bh * N + qrow] * kLog2e : 0.f;
  float dlt = qok ? p.delta[bh * N + qrow] : 0.f;
  // The loop's loads are not visible to the compiler's wait counting: its
  // wait for these values must fall here, not inside the loop, where it
  // would also wait for the next block's loads.
  settle(qv);
  settle(gv);
  asm volatile("" : "+v"(lse2), "+v"(dlt));
  f32x16 dq[G::DT];
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) dq[dt] = f32x16{};
  const int kend = CAUSAL ? min(N, q0 + kTile) : N;
  const int a_off = row_lane<D>(n) + 16 * g;
  const int t_off = tr_lane<D>(lane);
  BlockDma<D, kStep> dma;
  dma.init(__builtin_amdgcn_readfirstlane(wave), lane);
  const i32x4 rsK = buffer_rsrc(p.k + hoff, (uint32_t)N * G::kRow);
  const i32x4 rsV = buffer_rsrc(p.v + hoff, (uint32_t)N * G::kRow);
  auto issue = [&](int kb, int buf) __attribute__((always_inline)) {
    const uint32_t b = lds_address(smem) + buf * kBuf;
    dma.template issue<true>(rsK, kb, b, b + 2 * G::kBytesA);
    dma.template issue<false>(rsV, kb, b + G::kBytesA, 0);
  };
  // block kb (in buffer buf) complete and visible; then the next block's
  // loads into the other buffer, whose last reader was the previous step
  auto stage = [&](int kb, int buf) __attribute__((always_inline)) {
    wait_loads();
    __syncthreads();
    if (kb + kStep < kend) issue(kb + kStep, buf ^ 1);
  };
  auto step = [&](int kb, int buf, auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    const char* smem_b = smem + buf * kBuf;
    f32x16 s[kStep / 32], dp[kStep / 32];
#pragma unroll
    for (int ks = 0; ks < kStep / 32; ++ks) {
      s[ks] = f32x16{};
      dp[ks] = f32x16{};
      const char* kr = smem_b + ks * 32 * G::kStrA + a_off;
      const char* vr = smem_b + G::kBytesA + ks * 32 * G::kStrA + a_off;
#pragma unroll
      for (int t = 0; t < G::QST; ++t) {
        s[ks] = mfma_bf16(__builtin_bit_cast(bf16x8, *(const i32x4*)(kr + 32 * t)),
                          __builtin_bit_cast(bf16x8, qv[t]), s[ks]);
        dp[ks] = mfma_bf16(__builtin_bit_cast(bf16x8, *(const i32x4*)(vr + 32 * t)),
                           __builtin_bit_cast(bf16x8, gv[t]), dp[ks]);
      }
    }
    // dS^T as the B operand of the next product: keys 16u + 8g + e
    bf16x8 dsb[kStep / 16];
#pragma unroll
    for (int ks = 0; ks < kStep / 32; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_approx(__builtin_fmaf(s[ks][r], p.scale_log2, -lse2));
        if constexpr (MASK) {
          const int key = kb + 32 * ks + elem_of_reg(r, g);
          pv = key < N && (!CAUSAL || key <= qrow) ? pv : 0.f;
        }
        dsb[2 * ks + (r >> 3)][r & 7] = (__bf16)(pv * (dp[ks][r] - dlt));
      }
#pragma unroll
    for (int u = 0; u < kStep / 16; ++u)
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        const char* src = smem_b + 2 * G::kBytesA + t_off + 16 * u * G::kStrB + 64 * dt;
        const i16x4 lo = lds_read_tr16(src);
        const i16x4 hi = lds_read_tr16(src + 4 * G::kStrB);
        dq[dt] = mfma_bf16(join_bf16x8(lo, hi), dsb[u], dq[dt]);
      }
  };
  // Key blocks wholly visible to every query of the tile (causal: below
  // its first query; all: inside N) run without the mask, the rest (the
  // tile's diagonal blocks, the ragged last block) with it.
  const int kfull = min(CAUSAL ? q0 : N, N / kStep * kStep);
  issue(0, 0);
  int kb = 0, buf = 0;
  for (; kb < kfull; kb += kStep, buf ^= 1) {
    stage(kb, buf);
    step(kb, buf, Flag<false>{});
  }
  for (; kb < kend; kb += kStep, buf ^= 1) {
    stage(kb, buf);
    step(kb, buf, Flag<true>{});
  }
  if (qok) store_row<D>(p.dq + hoff + (int64_t)qrow * D, dq, p.scale, g);
}

// One query block (kStep = 64 queries, two 32-query subtiles) of the dkv
// kernel: S = Q K^T and dP = dO V^T for the block's queries against this
// lane's key, P = exp2(S scale log2(e) - lse log2(e)), dS = P o (dP - delta),
// then dV^T += dO^T P and dK^T += Q^T dS.  MASK zeroes P of queries past N
// and (causal) of queries before the key.
//
// The block's products form one sequence of slots (S and dP of subtile 0,
// of subtile 1, then dV and dK of queries 0..15, .., 48..63), placed in
// program order and fenced against the scheduler.  Each slot issues the LDS
// reads of the product kAhead slots later, and the softmax arithmetic of a
// subtile fills the slots that follow its last S and dP product, so that a
// single wave per SIMD keeps its matrix unit fed.
template <int D, int kStep, bool CAUSAL, bool MASK>
__device__ __forceinline__ void dkv_step(const char* smem, const float* lse_t, const float* dlt_t,
                                         int a_off, int t_off, int g, int qb, int krow, int N,
                                         float scale_log2, const RowRegs<D>& kv,
                                         const RowRegs<D>& vv, TileAcc<D>& dk, TileAcc<D>& dv) {
  static_assert(kStep == 64, "two 32-query subtiles per step");
  using G = Geo<D, kStep>;
  constexpr int QST = G::QST, DT = G::DT;
  constexpr int NM = 2 * QST;           // S and dP products per subtile
  constexpr int NU = 2 * DT;            // dV and dK products per 16 queries
  constexpr int NSLOT = 2 * NM + 4 * NU;
  constexpr int kAhead = 4;
  constexpr int kSoftRead = 4;          // slots between the lse/delta reads and their use
  i32x4 qa[2][QST], ga[2][QST];
  float lv[2][16], dl[2][16];
  i16x4 tr[4][DT][4];   // per 16 queries and d tile: dO^T lo, hi, Q^T lo, hi
  f32x16 s[2], dp[2];
  bf16x8 pb[4], dsb[4];

  auto reads_of = [&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
    if constexpr (m < 2 * NM) {
      constexpr int qs = m / NM, i = m % NM, t = i >> 1;
      const char* base = smem + a_off + qs * 32 * G::kStrA + 32 * t;
      if constexpr (i & 1)
        ga[qs][t] = *(const i32x4*)(base + G::kBytesA);
      else
        qa[qs][t] = *(const i32x4*)base;
    } else {
      constexpr int u = (m - 2 * NM) / NU, i = (m - 2 * NM) % NU, dt = i >> 1;
      const char* src = smem + 2 * G::kBytesA + ((i & 1) ? 0 : G::kBytesB) + t_off +
                        16 * u * G::kStrB + 64 * dt;
      tr[u][dt][2 * (i & 1)] = lds_read_tr16(src);
      tr[u][dt][2 * (i & 1) + 1] = lds_read_tr16(src + 4 * G::kStrB);
    }
  };
  auto product = [&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
    if constexpr (m < 2 * NM) {
      constexpr int qs = m / NM, i = m % NM, t = i >> 1;
      if constexpr (i & 1)
        dp[qs] = mfma_bf16(__builtin_bit_cast(bf16x8, ga[qs][t]),
                           __builtin_bit_cast(bf16x8, vv[t]), dp[qs]);
      else
        s[qs] = mfma_bf16(__builtin_bit_cast(bf16x8, qa[qs][t]),
                          __builtin_bit_cast(bf16x8, kv[t]), s[qs]);
    } else {
      constexpr int u = (m - 2 * NM) / NU, i = (m - 2 * NM) % NU, dt = i >> 1;
      if constexpr (i & 1)
        dk[dt] = mfma_bf16(join_bf16x8(tr[u][dt][2], tr[u][dt][3]), dsb[u], dk[dt]);
      else
        dv[dt] = mfma_bf16(join_bf16x8(tr[u][dt][0], tr[u][dt][1]), pb[u], dv[dt]);
    }
  };
  auto read_soft = [&](auto qc) __attribute__((always_inline)) {
    constexpr int qs = decltype(qc)::value;
    // -lse log2(e) and delta of queries 32 qs + elem_of_reg(r, g)
    const float4* l4 = (const float4*)(lse_t + 32 * qs + 8 * g);
    const float4* d4 = (const float4*)(dlt_t + 32 * qs + 8 * g);
    for_slots<4>([&](auto hc) __attribute__((always_inline)) {
      constexpr int h = decltype(hc)::value;
      const float4 l = l4[(h & 1) + 4 * (h >> 1)], d = d4[(h & 1) + 4 * (h >> 1)];
      lv[qs][4 * h] = -kLog2e * l.x;
      lv[qs][4 * h + 1] = -kLog2e * l.y;
      lv[qs][4 * h + 2] = -kLog2e * l.z;
      lv[qs][4 * h + 3] = -kLog2e * l.w;
      dl[qs][4 * h] = d.x; dl[qs][4 * h + 1] = d.y; dl[qs][4 * h + 2] = d.z; dl[qs][4 * h + 3] = d.w;
    });
  };
  auto soft = [&](auto qc, auto rc) __attribute__((always_inline)) {
    constexpr int qs = decltype(qc)::value, r = decltype(rc)::value;
    float pv = exp2_approx(__builtin_fmaf(s[qs][r], scale_log2, lv[qs][r]));
    if constexpr (MASK) {
      const int qi = qb + 32 * qs + elem_of_reg(r, g);
      pv = qi < N && (!CAUSAL || krow <= qi) ? pv : 0.f;
    }
    pb[2 * qs + (r >> 3)][r & 7] = (__bf16)pv;
    dsb[2 * qs + (r >> 3)][r & 7] = (__bf16)(pv * (dp[qs][r] - dl[qs][r]));
  };

  s[0] = s[1] = dp[0] = dp[1] = f32x16{};
  for_slots<kAhead>([&](auto mc) __attribute__((always_inline)) { reads_of(mc); });
  __builtin_amdgcn_sched_barrier(0);
  for_slots<NSLOT>([&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
    product(mc);
    if constexpr (m + kAhead < NSLOT) reads_of(Slot<m + kAhead>{});
    if constexpr (m == NM - kSoftRead) read_soft(Slot<0>{});
    if constexpr (m == 2 * NM - kSoftRead) read_soft(Slot<1>{});
    if constexpr (m >= NM && m < 2 * NM) {
      // subtile 0's softmax over subtile 1's products
      constexpr int E = 16 / NM;
      for_slots<E>([&](auto ec) __attribute__((always_inline)) {
        soft(Slot<0>{}, Slot<E * (m - NM) + decltype(ec)::value>{});
      });
    } else if constexpr (m >= 2 * NM && m < 2 * NM + 2 * NU) {
      // subtile 1's softmax over the dV, dK products of queries 0..31
      constexpr int E = 16 / (2 * NU);
      for_slots<E>([&](auto ec) __attribute__((always_inline)) {
        soft(Slot<1>{}, Slot<E * (m - 2 * NM) + decltype(ec)::value>{});
      });
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dkv_kernel(BwdParams p) {
  constexpr int kStep = kStepDkv;
  using G = Geo<D, kStep>;
  // two buffers, each: Q and dO blocks for the row reads, again for the
  // transposing reads, then the block's lse and delta
  constexpr int kOffL = 2 * G::kBytesA + 2 * G::kBytesB;
  constexpr int kBuf = kOffL + 2 * kStep * 4;
  __shared__ __attribute__((aligned(16))) char smem[2 * kBuf];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int N = p.n;
  int64_t bh;
  int tile;
  tile_of<CAUSAL, true>(p, bh, tile);
  const int k0 = tile * kTile;
  const int krow = k0 + wave * 32 + n;
  const bool kok = krow < N;
  const int64_t hoff = bh * (int64_t)N * D;
  i32x4 kv[G::QST], vv[G::QST];
  load_row<D>(kv, p.k + hoff + (int64_t)krow * D, kok, g);
  load_row<D>(vv, p.v + hoff + (int64_t)krow * D, kok, g);
  // The loop's loads are not visible to the compiler's wait counting: its
  // wait for these rows must fall here, not inside the loop, where it would
  // also wait for the next block's loads.
  settle(kv);
  settle(vv);
  f32x16 dk[G::DT], dv[G::DT];
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  const int a_off = row_lane<D>(n) + 16 * g;
  const int t_off = tr_lane<D>(lane);
  // causal: queries below this tile's first key see none of its keys
  const int qstart = CAUSAL ? k0 : 0;
  BlockDma<D, kStep> dma;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  dma.init(wv, lane);
  const i32x4 rsQ = buffer_rsrc(p.q + hoff, (uint32_t)N * G::kRow);
  const i32x4 rsG = buffer_rsrc(p.d_o + hoff, (uint32_t)N * G::kRow);
  const i32x4 rsL = buffer_rsrc(p.lse + bh * N, (uint32_t)N * 4);
  const i32x4 rsD = buffer_rsrc(p.delta + bh * N, (uint32_t)N * 4);
  static_assert(kStep == 64, "one 4-byte load per lane fills a block's lse or delta");
  auto issue = [&](int qb, int buf) __attribute__((always_inline)) {
    const uint32_t b = lds_address(smem) + buf * kBuf;
    dma.template issue<true>(rsQ, qb, b, b + 2 * G::kBytesA);
    dma.template issue<true>(rsG, qb, b + G::kBytesA, b + 2 * G::kBytesA + G::kBytesB);
    if (wv == 0) lds_load4(rsL, (uint32_t)lane * 4, (uint32_t)qb * 4, b + kOffL);
    if (wv == 1) lds_load4(rsD, (uint32_t)lane * 4, (uint32_t)qb * 4, b + kOffL + kStep * 4);
  };
  // block qb (in buffer buf) complete and visible; then the next block's
  // loads into the other buffer, whose last reader was the previous step
  auto stage = [&](int qb, int buf) __attribute__((always_inline)) {
    wait_loads();
    __syncthreads();
    if (qb + kStep < N) issue(qb + kStep, buf ^ 1);
  };
  auto run = [&](int qb, int buf, auto maskc) __attribute__((always_inline)) {
    const char* b = smem + buf * kBuf;
    dkv_step<D, kStep, CAUSAL, decltype(maskc)::value>(
        b, (const float*)(b + kOffL), (const float*)(b + kOffL + kStep * 4), a_off, t_off, g, qb,
        krow, N, p.scale_log2, kv, vv, dk, dv);
  };
  // Blocks that need the mask (causal: the two holding this tile's own
  // queries; the ragged last block) and the rest run in separate loops, so
  // that the common one carries no compares and the accumulators keep one
  // register assignment per loop.
  const int qfull = CAUSAL ? k0 + kTile : 0;
  const int nfull = N / kStep * kStep;
  issue(qstart, 0);
  int qb = qstart, buf = 0;
  for (; qb < min(qfull, N); qb += kStep, buf ^= 1) {
    stage(qb, buf);
    run(qb, buf, Flag<true>{});
  }
  for (; qb < nfull; qb += kStep, buf ^= 1) {
    stage(qb, buf);
    run(qb, buf, Flag<false>{});
  }
  for (; qb < N; qb += kStep, buf ^= 1) {
    stage(qb, buf);
    run(qb, buf, Flag<true>{});
  }
  if (kok) {
    store_row<D>(p.dk + hoff + (int64_t)krow * D, dk, p.scale, g);
    store_row<D>(p.dv + hoff + (int64_t)krow * D, dv, 1.0f, g);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_dc(const BwdParams& bp, int64_t bh, hipStream_t st) {
  const dim3 grid((unsigned)(bh * bp.tiles));
  hipLaunchKernelGGL((bwd_dkv_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, st, bp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, st, bp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_flash_bwd(const AttnBwdArgs& a, hipStream_t st) {
  const int64_t bh = a.batch * a.heads;
  const int64_t rows = bh * a.seq_len;
  hipError_t e = launch_delta(a.o, a.d_o, kBF16, a.head_dim, rows, a.delta, st);
  if (e != hipSuccess) return e;
  BwdParams bp;
  bp.q = (const uint16_t*)a.q;
  bp.k = (const uint16_t*)a.k;
  bp.v = (const uint16_t*)a.v;
  bp.d_o = (const uint16_t*)a.d_o;
  bp.lse = a.lse;
  bp.delta = a.delta;
  bp.dq = (uint16_t*)a.dq;
  bp.dk = (uint16_t*)a.dk;
  bp.dv = (uint16_t*)a.dv;
  bp.n = (int)a.seq_len;
  bp.tiles = (int)((a.seq_len + kTile - 1) / kTile);
  bp.bh_count = (int)bh;
  bp.scale = a.scale;
  bp.scale_log2 = (float)((double)a.scale * 1.4426950408889634);
  if (a.head_dim == 64)
    return a.causal ? launch_bwd_dc<64, true>(bp, bh, st) : launch_bwd_dc<64, false>(bp, bh, st);
  if (a.head_dim == 128)
    return a.causal ? launch_bwd_dc<128, true>(bp, bh, st) : launch_bwd_dc<128, false>(bp, bh, st);
  return hipErrorInvalidValue;
}

}  // namespace pn
