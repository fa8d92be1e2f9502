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
//               rows, then dV^T += dO^T P and dK^T += Q^T dS, split between
//               the two waves of a pair (S, P, dV / dP, dS, dK).
// The blocks of the other operand stream through LDS buffers by
// buffer-to-LDS loads: the loads of block j + 1 run while block j's
// products do (zeros past N); the per-row lse and delta of a query block
// sit in LDS beside it.
#include "device.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace pn {
namespace {

constexpr int kThreads = 256;   // four waves (dq kernel)
constexpr int kTile = 128;      // rows a workgroup owns (32 per wave)
// Rows of the other operand per step (both kernels run two waves per SIMD,
// one covering the other's latencies).
constexpr int kStepDq = 32;
constexpr int kStepDkv = 32;

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
  int tiles;          // 128-query tiles per head (dq kernel)
  int tiles_kv;       // key tiles per head (dkv kernel)
  int bh_count;       // batch * heads
  float scale;
  float scale_log2;   // scale * log2(e)
};

// Workgroup -> (head, tile).  Workgroups go to the eight XCDs in turn, so
// heads are taken in groups of eight, head 8c + x on XCD x: each XCD then
// works through its heads one at a time, all tiles of a head together, and
// the head's K, V, Q, dO rows stay in that XCD's L2.  Within a head,
// causal tiles differ in length (the dkv kernel's tile t walks N - 64 t
// queries, the dq kernel's 128 (t + 1) keys) and go out longest first, so
// short ones fill the machine at the end.  Heads past the last whole group
// of eight follow one after another.
template <bool CAUSAL, bool LONG_FIRST_LOW>
__device__ __forceinline__ void tile_of(const BwdParams& p, int T, int64_t& bh, int& tile) {
  const int64_t b = blockIdx.x;
  const int64_t grouped = (int64_t)(p.bh_count / 8) * 8 * T;
  int t;
  if (b < grouped) {
    const int64_t m = b >> 3;
    bh = (m / T) * 8 + (b & 7);
    t = (int)(m % T);
  } else {
    const int64_t r = b - grouped;
    bh = (int64_t)(p.bh_count / 8) * 8 + r / T;
    t = (int)(r % T);
  }
  tile = !CAUSAL || LONG_FIRST_LOW ? t : T - 1 - t;
}

template <int D, int STEP> struct Geo {
  static constexpr int kRow = D * 2;           // bf16 row bytes
  static constexpr int kBytes = STEP * kRow;   // one block in LDS, unpadded
  static constexpr int kSeg = kBytes / 1024;   // 1 KB load segments
  static_assert(kBytes % 1024 == 0, "a block is whole load segments");
  static constexpr int QST = D / 16;           // 16-element chunks of a row
  static constexpr int DT = D / 32;            // 32-row subtiles of a transposed output
};

// LDS layout of a block: row R at R * 2D bytes, its 16-byte chunk c at chunk
// position c ^ swz(R).  Both read patterns then miss bank conflicts:
// 16 lanes reading one chunk of 16 different rows (the A-operand row reads)
// land on 16 distinct chunk positions (swz is one-to-one on the low four
// row bits for d = 128, and on rows of one parity for d = 64, where two
// rows share a 256-byte bank sweep), and 32 lanes reading 8-byte pieces of
// chunks 4dt .. 4dt + 3 of four consecutive rows (the transposing read)
// land on 32 distinct 8-byte slots (swz moves consecutive rows to different
// groups of four chunks).
template <int D> __device__ __forceinline__ int swz(int R) {
  if constexpr (D == 128) return ((R & 3) << 2) | ((R >> 2) & 3);
  else return (((R >> 1) & 1) << 2) | ((R >> 2) & 3);
}

// Source offset, inside a block's rows, of the 16 bytes that lane `lane` of
// load segment `seg` writes at LDS position (seg * 64 + lane) * 16.
template <int D> __device__ __forceinline__ uint32_t swz_src_offset(int seg, int lane) {
  constexpr int kRow = 2 * D;
  const int pos = (seg * 64 + lane) * 16;
  const int R = pos / kRow, cpos = (pos % kRow) / 16;
  return (uint32_t)(R * kRow + 16 * (cpos ^ swz<D>(R)));
}

// This wave's share of the buffer-to-LDS loads that fill the LDS image of a
// STEP-row block of a [N][D] bf16 matrix, among W issuing waves: segments
// w, w + W, .., with each lane's source offset inside the block (rows past N
// read zeros through the buffer range check).  Asynchronous: the loads are
// awaited by an explicit s_waitcnt vmcnt(0) before the barrier that
// publishes the block.
template <int D, int STEP, int W> struct BlockDma {
  using G = Geo<D, STEP>;
  static constexpr int kPer = (G::kSeg + W - 1) / W;
  uint32_t off[kPer];
  int wave;
  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int i = 0; i < kPer; ++i) off[i] = swz_src_offset<D>(w + W * i, lane);
  }
  // rows r0.. into the block image at LDS address lds
  __device__ __forceinline__ void issue(i32x4 rs, int r0, uint32_t lds) const {
    const uint32_t soff = (uint32_t)r0 * G::kRow;
    static_for<kPer>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if (W * i + W - 1 < G::kSeg || wave + W * i < G::kSeg)
        lds_load16<i * W * 1024>(rs, off[i], soff, lds + wave * 1024);
    });
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

// This lane's LDS byte offsets inside a block image: the A-operand row
// reads (row perm_row(n), chunk 2t + g, t = 0 .. D/16 - 1) and the
// transposing reads (8 bytes of rows 8g + (lane%16)/4 + 4hi, at byte column
// 64dt + 32((lane/16)%2) + 8(lane%4)); 16 more rows add 16 * 2D bytes.
template <int D> struct LaneAddr {
  int row[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, n = lane & 31;
    const int R = perm_row(n);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) row[t] = R * 2 * D + 16 * ((2 * t + g) ^ swz<D>(R));
    const int k = (lane & 15) >> 2, h = (lane >> 4) & 1, c = lane & 3;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 8 * g + k + 4 * hi;
        tr[dt][hi] = r * 2 * D + 16 * ((4 * dt + 2 * h + (c >> 1)) ^ swz<D>(r)) + 8 * (c & 1);
      }
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int kStep = kStepDq;
  using G = Geo<D, kStep>;
  // two buffers, each: the K and V blocks
  constexpr int kBuf = 2 * G::kBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * kBuf];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int N = p.n;
  int64_t bh;
  int tile;
  tile_of<CAUSAL, false>(p, p.tiles, bh, tile);
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
  LaneAddr<D> la;
  la.init(lane);
  BlockDma<D, kStep, 4> dma;
  dma.init(__builtin_amdgcn_readfirstlane(wave), lane);
  // the descriptors are uniform: made scalar once here, not at every load
  const i32x4 rsK = uniform(buffer_rsrc(p.k + hoff, (uint32_t)N * G::kRow));
  const i32x4 rsV = uniform(buffer_rsrc(p.v + hoff, (uint32_t)N * G::kRow));
  auto issue = [&](int kb, int buf) __attribute__((always_inline)) {
    const uint32_t b = lds_address(smem) + buf * kBuf;
    dma.issue(rsK, kb, b);
    dma.issue(rsV, kb, b + G::kBytes);
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
      const char* kr = smem_b + ks * 32 * G::kRow;
      const char* vr = smem_b + G::kBytes + ks * 32 * G::kRow;
#pragma unroll
      for (int t = 0; t < G::QST; ++t) {
        s[ks] = mfma_bf16(__builtin_bit_cast(bf16x8, *(const i32x4*)(kr + la.row[t])),
                          __builtin_bit_cast(bf16x8, qv[t]), s[ks]);
        dp[ks] = mfma_bf16(__builtin_bit_cast(bf16x8, *(const i32x4*)(vr + la.row[t])),
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
        const char* src = smem_b + 16 * u * G::kRow;
        const i16x4 lo = lds_read_tr16(src + la.tr[dt][0]);
        const i16x4 hi = lds_read_tr16(src + la.tr[dt][1]);
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
    step(kb, buf, BoolC<false>{});
  }
  for (; kb < kend; kb += kStep, buf ^= 1) {
    stage(kb, buf);
    step(kb, buf, BoolC<true>{});
  }
  if (qok) store_row<D>(p.dq + hoff + (int64_t)qrow * D, dq, p.scale, g);
}

// dkv kernel: a workgroup owns 64 keys; four waves in two pairs that share
// 32 keys each (a lane per key), two workgroups per compute unit, so one
// workgroup's barrier waits are filled by the other's work.  The first wave
// of a pair forms S = Q K^T, P = exp2(S scale log2(e) - lse log2(e)) and
// dV^T += dO^T P; the second forms dP = dO V^T, dS = P o (dP - delta) with P
// taken from LDS (fp32, lane for lane), and dK^T += Q^T dS.  Each holds one
// output accumulator and one row operand, which is what lets two waves
// share a SIMD.  The second wave runs one query block behind the first, so at
// every step the pair works on different blocks with no wait between them:
// one wave's matrix products cover the other's softmax arithmetic.  Query
// blocks therefore live in three LDS buffers (loading, first wave's,
// second wave's) and P in two.  Query rows of S and dP are permuted so that
// P and dS land in the B-operand order of the dV and dK products; dO^T and
// Q^T come through the transposing LDS read.
constexpr int kDkvWaves = 4;                  // two pairs
constexpr int kDkvPairs = kDkvWaves / 2;
constexpr int kDkvTile = 32 * kDkvPairs;      // keys a workgroup owns

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kDkvWaves, 2) void bwd_dkv_kernel(BwdParams p) {
  constexpr int kStep = kStepDkv;
  static_assert(kStep == 32, "one 32-query subtile per step");
  using G = Geo<D, kStep>;
  constexpr int QST = G::QST, DT = G::DT;
  // three buffers, each: the Q and dO blocks, then 64 lse and 64 delta
  // values (one 4-byte load per lane; the block uses the first 32); then
  // two P exchange buffers, 16 floats per lane of each pair, stored as four
  // float4 planes
  constexpr int kOffL = 2 * G::kBytes;
  constexpr int kBuf = kOffL + 2 * 256;
  constexpr int kOffP = 3 * kBuf;
  constexpr int kXBuf = kDkvPairs * 4096;
  __shared__ __attribute__((aligned(16))) char smem[kOffP + 2 * kXBuf];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  // role 0: S, P, dV; role 1: dP, dS, dK; kg: the pair
  const int role = wave / kDkvPairs, kg = wave % kDkvPairs;
  const int g = lane >> 5, n = lane & 31;
  const int N = p.n;
  int64_t bh;
  int tile;
  tile_of<CAUSAL, true>(p, p.tiles_kv, bh, tile);
  const int k0 = tile * kDkvTile;
  const int krow = k0 + kg * 32 + n;
  const bool kok = krow < N;
  const int64_t hoff = bh * (int64_t)N * D;
  // K rows (role 0) or V rows (role 1) of this lane's key: the B operand
  RowRegs<D> kr;
  load_row<D>(kr, (role == 0 ? p.k : p.v) + hoff + (int64_t)krow * D, kok, g);
  settle(kr);
  TileAcc<D> acc;   // dV^T (role 0) or dK^T (role 1)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  LaneAddr<D> la;
  la.init(lane);
  char* xp = smem + kOffP + kg * 4096 + lane * 16;   // this lane's P exchange slot
  // causal: queries below this tile's first key see none of its keys
  const int qstart = CAUSAL ? k0 : 0;
  BlockDma<D, kStep, kDkvWaves> dma;
  dma.init(wave, lane);
  // the descriptors are uniform: made scalar once here, not at every load
  const i32x4 rsQ = uniform(buffer_rsrc(p.q + hoff, (uint32_t)N * G::kRow));
  const i32x4 rsG = uniform(buffer_rsrc(p.d_o + hoff, (uint32_t)N * G::kRow));
  const i32x4 rsL = uniform(buffer_rsrc(p.lse + bh * N, (uint32_t)N * 4));
  const i32x4 rsD = uniform(buffer_rsrc(p.delta + bh * N, (uint32_t)N * 4));
  auto issue = [&](int qb, int buf) __attribute__((always_inline)) {
    const uint32_t b = lds_address(smem) + buf * kBuf;
    dma.issue(rsQ, qb, b);
    dma.issue(rsG, qb, b + G::kBytes);
    if (wave == 0) lds_load4(rsL, (uint32_t)lane * 4, (uint32_t)qb * 4, b + kOffL);
    if (wave == 1) lds_load4(rsD, (uint32_t)lane * 4, (uint32_t)qb * 4, b + kOffL + 256);
  };
  // per-lane values of queries elem_of_reg(r, g) of a block: lse or delta
  auto row_vals = [&](const char* b, int which, float (&v)[16]) __attribute__((always_inline)) {
    const float4* v4 = (const float4*)(b + kOffL + which * 256) + 2 * g;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 x = v4[(h & 1) + 4 * (h >> 1)];
      v[4 * h] = x.x;
      v[4 * h + 1] = x.y;
      v[4 * h + 2] = x.z;
      v[4 * h + 3] = x.w;
    }
  };
  // dV^T += dO^T P (role 0) or dK^T += Q^T dS (role 1): the A operands
  // (dO^T or Q^T of the block, through the transposing read) in tr
  using TrRegs = i16x4[2][DT][2];
  auto read_t = [&](const char* b, TrRegs& tr, auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value, u = i / DT, dt = i % DT;
    const char* src = b + (role == 0 ? G::kBytes : 0) + 16 * u * G::kRow;
    tr[u][dt][0] = lds_read_tr16(src + la.tr[dt][0]);
    tr[u][dt][1] = lds_read_tr16(src + la.tr[dt][1]);
  };
  auto outer = [&](const TrRegs& tr, const bf16x8 (&bop)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = mfma_bf16(join_bf16x8(tr[u][dt][0], tr[u][dt][1]), bop[u], acc[dt]);
  };
  // S (role 0) or dP (role 1) of the block in b, this lane's key against
  // queries elem_of_reg(r, g); all A-operand reads go out first, and the
  // transposing reads of the outer product ride between the products
  auto inner = [&](const char* b, TrRegs& tr) __attribute__((always_inline)) {
    const char* ar = b + role * G::kBytes;
    i32x4 a[QST];
#pragma unroll
    for (int t = 0; t < QST; ++t) a[t] = *(const i32x4*)(ar + la.row[t]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sd = f32x16{};
    static_for<QST>([&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      sd = mfma_bf16(__builtin_bit_cast(bf16x8, a[t]), __builtin_bit_cast(bf16x8, kr[t]), sd);
      // 2 DT transposing read pairs over QST = 2 DT products
      read_t(b, tr, tc);
      __builtin_amdgcn_sched_barrier(0);
    });
    return sd;
  };
  // Step j: the first wave takes block j, the second block j - 1; block
  // j + 1 loads meanwhile.  The barrier at the start of a step publishes
  // block j's loads and P of block j - 1, and retires every read of the
  // buffers that step j's loads and P writes reuse.  WHO: 0 both waves of
  // each pair work, 1 only the first (j = 0), 2 only the second (the last
  // step).  The matrix products sit outside any branch on the role, so the
  // accumulators keep one register assignment.
  const int nblk = (N - qstart + kStep - 1) / kStep;
  int j = 0, buf = 0, prev = 2;   // buf = j % 3, prev = (j - 1) % 3
  auto step = [&](auto maskc, auto whoc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    constexpr int WHO = decltype(whoc)::value;
    wait_loads();
    __syncthreads();
    const int nxt = buf == 2 ? 0 : buf + 1;
    if (j + 1 < nblk) issue(qstart + (j + 1) * kStep, nxt);
    if (WHO == 0 || (WHO == 1) == (role == 0)) {
      const int qb = qstart + (role == 0 ? j : j - 1) * kStep;
      const char* b = smem + (role == 0 ? buf : prev) * kBuf;
      TrRegs tr;
      const f32x16 sd = inner(b, tr);
      float rv[16];   // lse (role 0) or delta (role 1)
      row_vals(b, role, rv);
      bf16x8 bop[2];
      if (role == 0) {
        char* xw = xp + (j & 1) * kXBuf;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * h + e;
            float t = exp2_approx(__builtin_fmaf(sd[r], p.scale_log2, -kLog2e * rv[r]));
            if constexpr (MASK) {
              const int qi = qb + elem_of_reg(r, g);
              t = qi < N && (!CAUSAL || krow <= qi) ? t : 0.f;
            }
            pv[e] = t;
            bop[r >> 3][r & 7] = (__bf16)t;
          }
          *(float4*)(xw + h * 1024) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        }
      } else {
        const char* xr = xp + ((j - 1) & 1) * kXBuf;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float4 pv = *(const float4*)(xr + h * 1024);
          const float ps[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * h + e;
            bop[r >> 3][r & 7] = (__bf16)(ps[e] * (sd[r] - rv[r]));
          }
        }
      }
      outer(tr, bop);
    }
    prev = buf;
    buf = nxt;
    ++j;
  };
  // Blocks that need the mask (causal: the two holding this tile's own
  // queries; the ragged last block) and the rest run in separate loops, so
  // that the common one carries no compares.
  const int jmask = CAUSAL ? min(nblk, kDkvTile / kStep) : 0;
  const int jfull = min(nblk, max(jmask, (N - qstart) / kStep));
  issue(qstart, 0);
  step(BoolC<true>{}, IntC<1>{});
  while (j < jmask) step(BoolC<true>{}, IntC<0>{});
  while (j < jfull) step(BoolC<false>{}, IntC<0>{});
  while (j < nblk) step(BoolC<true>{}, IntC<0>{});
  step(BoolC<false>{}, IntC<2>{});
  if (kok) {
    if (role == 0)
      store_row<D>(p.dv + hoff + (int64_t)krow * D, acc, 1.0f, g);
    else
      store_row<D>(p.dk + hoff + (int64_t)krow * D, acc, p.scale, g);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_dc(const BwdParams& bp, int64_t bh, hipStream_t st) {
  const dim3 grid_kv((unsigned)(bh * bp.tiles_kv));
  hipLaunchKernelGGL((bwd_dkv_kernel<D, CAUSAL>), grid_kv, dim3(64 * kDkvWaves), 0, st, bp);
  const dim3 grid((unsigned)(bh * bp.tiles));
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
  bp.tiles_kv = (int)((a.seq_len + kDkvTile - 1) / kDkvTile);
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
