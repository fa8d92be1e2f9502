// FlashAttention forward for gfx950: tiled exact attention with an online
// softmax; the score matrix S is never stored.
//
// Method ("Why Low-Precision Transformer Training Fails", Algorithm 1: Q is
// split into T_r = ceil(N/B_r) row blocks and K, V into T_c = ceil(N/B_c)
// row blocks; the online-softmax accumulation its referee report places at
// Eq. (2)).  For each query block and each key block j in ascending order:
//     m'  = max(m, rowmax(S_j))
//     P_j = exp(S_j - m')              (unnormalised; 1 at the running max)
//     l'  = exp(m - m') l + rowsum(P_j)
//     O'  = exp(m - m') O + P_j V_j
// and finally O = O' / l'.  In exact arithmetic this is softmax(S) V for any
// B_r, B_c; only rounding depends on them.
//
// Mapping onto CDNA4:
//  * One workgroup = 8 wave64s = B_r = 256 query rows; each wave owns 32 rows.
//    B_c = 128 keys per step (64 for the fp32 P*V engines, whose fp32 P
//    operand needs twice the registers), staged in LDS (K and V row-major,
//    padded rows), double-buffered: the next block's K and V stream from HBM
//    straight into LDS (buffer loads with the lds modifier) while the current
//    one is used.  The long block halves the per-key cost of the rescale of O,
//    of the barriers and of the loop bookkeeping.
//  * The eight waves form two groups of four, one wave of each group per
//    SIMD.  The groups run half a step apart, so that while one wave of a
//    SIMD issues its matrix products (P_{j-1} V_{j-1}, then S_j) the other
//    does its softmax arithmetic (mask, max, exp, sums, the rescale of O by
//    exp(m - m'), P -> bf16) on VALU: the two instruction streams overlap
//    on each SIMD, and the matrix half-step holds no VALU instruction
//    (8-bit Q/K aside: their scores take their key scales at the end of it,
//    int8's after the exact conversion to fp32).
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
//  * The row max is taken on the raw dot products (the scale is positive);
//    each probability is then exp2(fma(s, scale*log2 e, -m)): one fma and one
//    v_exp_f32 per score.  At the row max the fma leaves only the rounding
//    residual of the scaled max, so P is 1 to within an ulp there and exactly
//    1 once rounded to bf16.
//  * Persistent grid: min(tiles, compute units) workgroups, each walking a
//    list of 256-row query tiles (see tile_of): every tile of a head runs on
//    one XCD, causal launches hand out the longest tiles first, and the
//    next tile's first K/V block and Q rows load while the current tile
//    finishes.
#include <atomic>

#include "device.hpp"
#include "launch.hpp"
#include "lds_dma.hpp"

namespace pn {
namespace {

enum QKKind { QK_BF16 = 0, QK_I8 = 1, QK_F32 = 2, QK_F8 = 3 };
// 8-bit Q/K codes with per-row fp32 scales (int8, or E4M3 fp8)
template <int QK> constexpr bool kScaledQK = QK == QK_I8 || QK == QK_F8;
// P*V engines: bf16 P and bf16 V on bf16 MFMA; otherwise fp32 MFMA with V
// widened exactly (V stored as bf16 or as fp32).
enum PVKind { PV_BF16 = 0, PV_F32_VBF16 = 1, PV_F32_VF32 = 2 };

constexpr int kWaves = 8;            // two groups of four: one wave of each per SIMD
// Stabilised variant: largest distance (log2 units) of the normaliser above
// the running row max (see the range guard in the softmax half-step).
constexpr float kStabMaxShift = 64.f;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;     // query rows per workgroup

// Keys per step: 128 when P enters P*V as bf16, 64 for the fp32 engines.
template <int PV> struct BlockKeys { static constexpr int value = 128; };
template <> struct BlockKeys<1> { static constexpr int value = 64; };
template <> struct BlockKeys<2> { static constexpr int value = 64; };

template <int QK> struct QKTraits;
template <> struct QKTraits<QK_BF16> { using T = uint16_t; };
template <> struct QKTraits<QK_I8> { using T = int8_t; };
template <> struct QKTraits<QK_F32> { using T = float; };
template <> struct QKTraits<QK_F8> { using T = uint8_t; };
template <int PV> struct VTraits { using T = uint16_t; };
template <> struct VTraits<PV_F32_VF32> { using T = float; };

// LDS tile geometry.  Rows are padded so that the two read patterns of the
// kernel are free of bank conflicts: +16 bytes per K row (16 consecutive K
// rows read the same 16-byte column), +64 bytes per V row (the transposing
// reads touch 4 rows x 64 bytes at a time).  Tiles are whole multiples of
// 1 KiB, the footprint of one wave-wide 16-byte buffer load into LDS.
template <int D, int QK, int PV> struct Tile {
  static constexpr int kBC = BlockKeys<PV>::value;
  static constexpr int kRowK = D * (int)sizeof(typename QKTraits<QK>::T);
  static constexpr int kRowV = D * (int)sizeof(typename VTraits<PV>::T);
  static constexpr int kStrK = kRowK + 16;
  static constexpr int kStrV = kRowV + 64;
  static constexpr int kBytesK = kBC * kStrK;
  static constexpr int kBytesV = kBC * kStrV;
  static constexpr int kSegK = kBytesK / 1024;
  static constexpr int kSegV = kBytesV / 1024;
  // the four waves of group 0 issue the K tiles, those of group 1 the V tiles
  static constexpr int kIssuers = kWaves / 2;
  static constexpr int kSegKPerWave = (kSegK + kIssuers - 1) / kIssuers;
  static constexpr int kSegVPerWave = (kSegV + kIssuers - 1) / kIssuers;
  static constexpr int kSegPerWave = kSegKPerWave > kSegVPerWave ? kSegKPerWave : kSegVPerWave;
  static constexpr int kBytesSk = kScaledQK<QK> ? kBC * 4 : 0;
  // [K buf0][K buf1][V buf0][V buf1][sk buf0][sk buf1].  The key scales of
  // block j are read at the end of each group's M_j; those of block j + 2
  // load in group 0's M_{j+1}, after group 1's M_j.
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
  float beta;        // stabilised variant: normaliser factor for a repeated positive max
  int64_t bh_count;  // batch * heads
  int q_tiles;       // query tiles per (batch, head)
  int64_t tiles;     // bh_count * q_tiles
  int grp4;          // tile order in groups of four heads per XCD (bh_count % 32 == 0)
  unsigned grid;     // workgroups: min(tiles, compute units)
};

// Tile schedule.  Logical tile L (0..tiles-1) is dispatched in an order
// that keeps each head on one XCD (L % 8) and, with grp4, works on four
// heads of an XCD at a time, longest causal query tiles first inside the
// group: the K/V rows that concurrently resident workgroups re-read then fit
// in the XCD's L2.  Workgroup w of a grid of P runs logical tiles
// r*P + 8*jj + w%8 for rounds r = 0, 1, ..., where jj walks the XCD's
// workgroups forward on even rounds and backward on odd ones: pairing long
// and short causal tiles balances the work.  With P = tiles every
// workgroup runs one tile.
struct TileId {
  int bh;      // batch * heads + head
  int q0;      // first query row
  int nblk;    // key blocks to visit
  bool valid;
};

template <bool CAUSAL, int BC>
__device__ __forceinline__ TileId tile_of(const FlashParams& p, int round) {
  const uint32_t P = gridDim.x, w = blockIdx.x;
  uint32_t L;
  if (P % 8 == 0) {
    const uint32_t J = P / 8, jw = w / 8;
    const uint32_t jj = (round & 1) ? J - 1 - jw : jw;
    L = (uint32_t)round * P + 8 * jj + w % 8;
  } else {
    L = (uint32_t)round * P + w;
  }
  TileId t;
  t.valid = L < (uint32_t)p.tiles;
  const uint32_t NT = (uint32_t)p.q_tiles;
  uint32_t rank;  // 0 = the longest causal tile
  if (p.grp4) {
    const uint32_t x = L % 8, r = L / 8;
    const uint32_t grp = r / (4 * NT), wi = r - grp * (4 * NT);
    t.bh = (int)((grp * 4 + wi % 4) * 8 + x);
    rank = wi / 4;
  } else {
    const uint32_t BHn = (uint32_t)p.bh_count;
    rank = L / BHn;
    t.bh = (int)(L - rank * BHn);
  }
  const int qt = CAUSAL ? (int)NT - 1 - (int)rank : (int)rank;
  t.q0 = qt * kBR;
  const int kend = CAUSAL ? min(p.n, t.q0 + kBR) : p.n;
  t.nblk = t.valid ? (kend + BC - 1) / BC : 0;
  return t;
}

// Max of the N scores of a lane as a tree of 3-input maxima (v_max3_f32).
template <int N>
__device__ __forceinline__ float tree_max(const float (&x)[N]) {
  if constexpr (N == 1) {
    return x[0];
  } else if constexpr (N == 2) {
    return fmaxf(x[0], x[1]);
  } else {
    constexpr int M = (N + 2) / 3;
    float y[M];
#pragma unroll
    for (int i = 0; i < N / 3; ++i) y[i] = fmaxf(fmaxf(x[3 * i], x[3 * i + 1]), x[3 * i + 2]);
    if constexpr (N % 3 == 1) y[M - 1] = x[N - 1];
    if constexpr (N % 3 == 2) y[M - 1] = fmaxf(x[N - 2], x[N - 1]);
    return tree_max<M>(y);
  }
}

// Ends the live range of a register value: the result is unspecified and
// costs no instruction.  Used where a path leaves a value the program never
// reads again, so that the register allocator does not keep it alive across
// the other paths that merge with it.
template <typename T> __device__ __forceinline__ void forget(T& x) {
  x = __builtin_nondeterministic_value(x);
}

// Pins a register value at this point of the program: the empty asm claims
// to read and rewrite it, so the code producing the value cannot sink below
// this point and its users cannot rise above it.  The workgroup barrier
// orders memory operations only; without pins the compiler moves a
// half-step's register arithmetic across it into the next slot, where the
// wave would run it serially with its matrix products.
template <typename T> __device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }


// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x0008;
constexpr int kSchedDsRead = 0x0100;

// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with expcnt and lgkmcnt
// left at their maxima: wait for this wave's outstanding vector-memory ops.
constexpr int kWaitVmcnt0 = 0x0F70;
// the same for vmcnt(n): all but this wave's n most recent vector-memory
// operations done (they complete in issue order)
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// dword 3 of a raw buffer resource (as buffer_rsrc builds it)
constexpr int kRsrcWord3 = 0x00020000;

// Wave priority (s_setprio) while a wave issues its matrix products.
constexpr int kPrioMfma = 2;

// Instruction-group orders for the matrix half-step (bf16 engines).  The
// P.V products and the S products are scheduled as two separate regions: a
// group mask names an instruction class, not an instruction, so in a shared
// region the scheduler would fill the groups from whichever stream is ready.
//
// P.V region: per product two LDS reads, kAhead products ahead.
template <int N, int I = 0>
__device__ __forceinline__ void pv_schedule_step() {
  constexpr int kAhead = 4;
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (I + kAhead < N) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    pv_schedule_step<N, I + 1>();
  }
}
template <int N>
__device__ __forceinline__ void pv_schedule() {
  constexpr int kAhead = 4;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * (N < kAhead ? N : kAhead), 0);
  pv_schedule_step<N>();
}
// S region: one LDS read per product, kAhead products ahead.
template <int N, int I = 0>
__device__ __forceinline__ void s_schedule_step() {
  constexpr int kAhead = 4;
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if constexpr (I + kAhead < N) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    s_schedule_step<N, I + 1>();
  }
}
template <int N>
__device__ __forceinline__ void s_schedule() {
  constexpr int kAhead = 4;
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, N < kAhead ? N : kAhead, 0);
  s_schedule_step<N>();
}


// The key scales of rows kb.. into key-scale buffer skbuf (one wave).
template <int D, int QK, int PV>
__device__ __forceinline__ void issue_sk(char* smem, int lane, int kb, int skbuf,
                                         const void* sbase, int n) {
  using TL = Tile<D, QK, PV>;
  const i32x4 rsS = buffer_rsrc(sbase, (uint32_t)n * 4);
#pragma unroll
  for (int h = 0; h < TL::kBC / 64; ++h)
    lds_load4(rsS, (uint32_t)lane * 4, (uint32_t)(kb + 64 * h) * 4,
              lds_address(smem) + TL::kOffSk + skbuf * TL::kBytesSk + 256 * h);
}

// Issue this wave's share (w = 0..3 inside the issuing group) of the loads
// that fill K tile buffer `buf` with key rows kb.. (and, for 8-bit Q/K, the
// key scales into key-scale buffer skbuf).  Asynchronous.
template <int D, int QK, int PV>
__device__ __forceinline__ void issue_k(char* smem, int w, int lane, int kb, int buf, int skbuf,
                                        const void* kbase, const void* sbase, int n,
                                        const uint32_t* voffK) {
  using TL = Tile<D, QK, PV>;
  const i32x4 rsK = buffer_rsrc(kbase, (uint32_t)n * TL::kRowK);
  const uint32_t base = lds_address(smem) + buf * TL::kBytesK + w * 1024;
  const uint32_t soff = (uint32_t)kb * TL::kRowK;
  static_for<TL::kSegKPerWave>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    if (TL::kSegK % TL::kIssuers == 0 || w + i * TL::kIssuers < TL::kSegK)
      lds_load16<i * TL::kIssuers * 1024>(rsK, voffK[i], soff, base);
  });
  if constexpr (kScaledQK<QK>) {
    if (w == 0) issue_sk<D, QK, PV>(smem, lane, kb, skbuf, sbase, n);
  }
}

// The same for V tile buffer `buf` (issued by group 1).
template <int D, int QK, int PV>
__device__ __forceinline__ void issue_v(char* smem, int w, int kb, int buf, const void* vbase,
                                        int n, const uint32_t* voffV) {
  using TL = Tile<D, QK, PV>;
  const i32x4 rsV = buffer_rsrc(vbase, (uint32_t)n * TL::kRowV);
  const uint32_t base = lds_address(smem) + TL::kOffV + buf * TL::kBytesV + w * 1024;
  const uint32_t soff = (uint32_t)kb * TL::kRowV;
  static_for<TL::kSegVPerWave>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    if (TL::kSegV % TL::kIssuers == 0 || w + i * TL::kIssuers < TL::kSegV)
      lds_load16<i * TL::kIssuers * 1024>(rsV, voffV[i], soff, base);
  });
}

// Workgroup barrier without the memory fence that __syncthreads() carries.
// The fence would make every wave wait at the barrier for its in-flight
// buffer->LDS loads, which are meant to overlap the following half-steps;
// those loads are awaited explicitly (vmcnt) where the schedule needs them.
// This wave's own LDS reads are drained first (lgkmcnt), and the asm's memory
// clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Schedule ("ping-pong").  Each key block j is split into two half-steps:
//   M_j : the MFMA half-step  -- O^T += V_{j-1}^T P_{j-1}^T, then S_j = K_j Q^T
//   X_j : the VALU half-step  -- mask, online max, exponentials, row sum,
//                                rescale of O, P_j -> bf16
// A wave runs M_0 X_0 M_1 X_1 ... M_n (the last M has only the P.V part).
// The eight waves form two groups of four; group 1 runs one half-step
// behind group 0, and every half-step ends at a workgroup barrier.  The two
// waves sharing a SIMD therefore always run opposite half-steps: one keeps
// the matrix cores busy while the other works the vector ALUs.  K and V
// blocks are double-buffered in LDS (the slot loop below gives the exact
// issue and wait points).  The kernel is persistent: a workgroup walks a
// list of query tiles, and one tile's last slots overlap the next one's
// first.
template <int D, int QK, int PV, bool CAUSAL, bool DEBUG_S, bool STAB, bool OF32>
__global__ __launch_bounds__(kThreads) void flash_fwd_kernel(FlashParams p) {
  using QT = typename QKTraits<QK>::T;
  using VT = typename VTraits<PV>::T;
  using TL = Tile<D, QK, PV>;
  constexpr int BC = TL::kBC;
  constexpr int NKS = BC / 32;  // 32-key subtiles of S^T per block
  constexpr int DT = D / 32;    // 32-row d subtiles of O^T

  __shared__ __attribute__((aligned(1024))) char smem[TL::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int g = lane >> 5;
  const int n = lane & 31;
  const int N = p.n;
  const int wg = wave & (TL::kIssuers - 1);  // wave index inside its group

  // ---- the tile this workgroup works on (its identity changes at the
  // switch to the next tile), and the next one
  int round = 0;
  int jg0 = 0;  // global number of the current tile's first key block
  TileId cur = tile_of<CAUSAL, BC>(p, 0);
  TileId nxt = tile_of<CAUSAL, BC>(p, 1);
  if (!cur.valid) return;  // never: the grid has at most `tiles` workgroups
  int q0w = cur.q0 + wave * 32;
  int qrow = q0w + n;
  bool qvalid = qrow < N;
  int bh = cur.bh;
  auto head_ptr = [&](const void* base, int b, int esize) __attribute__((always_inline)) {
    return (const void*)((const char*)base + (int64_t)b * N * D * esize);
  };

  // group 0 holds the source offsets of its K segments, group 1 those of
  // its V segments, in the same registers
  uint32_t voff[TL::kSegPerWave];
#pragma unroll
  for (int i = 0; i < TL::kSegPerWave; ++i)
    voff[i] = group == 0 ? seg_src_offset(wg + i * TL::kIssuers, lane, TL::kRowK, TL::kStrK)
                         : seg_src_offset(wg + i * TL::kIssuers, lane, TL::kRowV, TL::kStrV);

  // The first K tile streams in while this lane's Q row loads.
  if (group == 0)
    issue_k<D, QK, PV>(smem, wg, lane, 0, 0, 0, head_ptr(p.k, bh, sizeof(QT)),
                       kScaledQK<QK> ? (const void*)(p.k_scale + (int64_t)bh * N) : nullptr, N, voff);

  // ---- this lane's query row as the B operand of S^T = K Q^T (registers)
  constexpr int QST = (QK == QK_BF16) ? D / 16 : (kScaledQK<QK> ? D / 32 : D / 2);
  i32x4 qv[QK == QK_F32 ? 1 : QST];
  float qf[QK == QK_F32 ? QST : 1];
  float sq_log2 = 0.f;  // this tile's row scale times scale * log2(e) (8-bit Q/K)
  float sq_pend = 0.f;  // the row scale (unscaled) of the tile whose Q rows were loaded last
  // load the Q row of query `row` of head `b` (zeros past the sequence end)
  auto load_q = [&](int b, int row) __attribute__((always_inline)) {
    const bool ok = row < N;
    const QT* Qg = (const QT*)p.q + (int64_t)b * N * D;
    if constexpr (QK == QK_F32) {
#pragma unroll
      for (int t = 0; t < QST; ++t) qf[t] = ok ? Qg[(int64_t)row * D + 2 * t + g] : 0.f;
    } else {
      // Range-checked buffer loads, issued by every lane whatever its row
      // (a row past the sequence end starts at the end of the range and
      // reads zeros): each wave issues exactly kQLoads vector-memory
      // instructions here, which the counted wait at a tile switch relies on.
      constexpr int EPC = 16 / (int)sizeof(QT);  // elements per 16-byte chunk
      const uint32_t rowc = (uint32_t)(ok ? row : N);
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          (void*)Qg, (short)0, (int)((uint32_t)N * D * sizeof(QT)), kRsrcWord3);
#pragma unroll
      for (int t = 0; t < QST; ++t)
        qv[t] = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (int)((rowc * D + 2 * EPC * t + EPC * g) * sizeof(QT)), 0, 0);
      if constexpr (kScaledQK<QK>) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.q_scale + (int64_t)b * N), (short)0, (int)((uint32_t)N * 4), kRsrcWord3);
        // used only once the tile becomes current (a use here would wait
        // for the load at once)
        sq_pend = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(rowc * 4), 0, 0));
      }
    }
  };
  // vector-memory instructions of one load_q (none counted for fp32 Q, whose
  // loads are waited for in full)
  constexpr int kQLoads = QK == QK_F32 ? -1 : QST + (kScaledQK<QK> ? 1 : 0);
  load_q(bh, qrow);
  sq_log2 = sq_pend * p.scale_log2;

  // One wait for the Q row and the first K tile, with a wait the compiler
  // sees: otherwise its wait-count pass, unsure the Q loads finished before
  // the loop, waits for all vector-memory traffic at their first use in
  // every iteration, which would also drain the K/V prefetch.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // Near the causal diagonal a block can lie entirely above a wave's rows:
  // its scores are all masked, so m and l are unchanged (exp(m - m') = 1)
  // and P = 0 adds nothing to O.  Inside the main loop every wave still runs
  // such blocks, which keeps the loop free of per-wave conditions whose
  // merging paths would keep dead score registers alive; only the last
  // block of a tile is skipped, group-wide, after the loop (see the slots).

  float m_run = -INFINITY;     // normaliser of the accumulated block sums, log2 units
  float mraw_run = -INFINITY;  // running max of the unscaled scores
  float l_run = 0.f;
  int nmax_run = 0;            // stabilised variant: occurrences of the running max
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  f32x16 s[NKS];                                             // S_j, then P_j (fp32)
  bf16x8 pb[PV == PV_BF16 ? BC / 16 : 1];                    // P_j as the bf16 operand
  float pf[PV == PV_BF16 ? 1 : NKS][PV == PV_BF16 ? 1 : 16];  // P_j for the fp32 engines
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[ks][r] = 0.f;

  // per-lane LDS byte offsets of the operand reads (block-independent)
  const int k_lane = perm_row(n) * TL::kStrK;
  const int v_lane = (8 * g + ((lane & 15) >> 2)) * TL::kStrV +
                     (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * (int)sizeof(VT);

  block_barrier();

  // ================= M_j: O^T += V_{j-1}^T P_{j-1}^T, then S_j = K_j Q^T
  // (in this order the P_{j-1} registers die before the new scores are born).
  // DO_PV / DO_S select the parts at compile time, so that the steady-state
  // step is one straight-line region the scheduler can interleave: LDS reads
  // run a few matrix products ahead of their use.
  // Loads a matrix half-step issues for a following block (of this tile or
  // of the next one): rows kb.. of the K (group 0) or V (group 1) head at
  // base (and, for int8 K, its key scales at sbase) into buffer buf, if on.
  struct Prefetch {
    const void* base;
    const void* sbase;
    int kb, buf, skbuf;
    bool on;
  };
  // this wave's K segment q of a request (with the first, the key scales)
  auto issue_one = [&](auto qc, const Prefetch& rq) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    if (rq.on && (TL::kSegK % TL::kIssuers == 0 || wg + q * TL::kIssuers < TL::kSegK))
      lds_load16<q * TL::kIssuers * 1024>(
          buffer_rsrc(rq.base, (uint32_t)N * TL::kRowK), voff[q], (uint32_t)rq.kb * TL::kRowK,
          lds_address(smem) + rq.buf * TL::kBytesK + wg * 1024);
    if constexpr (q == 0 && kScaledQK<QK>) {
      if (rq.on && wg == 0) issue_sk<D, QK, PV>(smem, lane, rq.kb, rq.skbuf, rq.sbase, N);
    }
  };

  // The fenced matrix half-step (products and LDS reads only) serves bf16 P
  // with bf16, int8 or fp8 Q/K.
  constexpr bool kFenced = PV == PV_BF16 && (QK == QK_BF16 || kScaledQK<QK>);
  // 8-bit scores in the fenced half-step take their key scales at the end
  // of it (after the exact int32 -> fp32 conversion for int8) and their row
  // scale with the exp2 argument.  In the softmax half-step, whose vector
  // work bounds the 8-bit steps, the key scales measured 0.8 % (int8) and
  // 5.6 % (fp8) slower on c5.
  constexpr bool kScaleInX = kFenced && kScaledQK<QK>;

  auto m_body = [&](const int jl, const int jg, auto do_pv_c, auto do_s_c, auto issue_c,
                    const Prefetch& rq) __attribute__((always_inline)) {
    constexpr bool DO_PV = decltype(do_pv_c)::value;
    constexpr bool DO_S = decltype(do_s_c)::value;
    // loads to issue: 0 none, 1 K (spread over the products), 2 V (before
    // the first product, or spread over the first half of the products)
    constexpr int ISSUE = decltype(issue_c)::value;
    constexpr int NSEG = TL::kSegKPerWave;
    // At d = 128 group 1's V loads are spread over the first half of its
    // fenced products: issued back to back they delay the first product by
    // their issue time (about 240 cycles), while the last one still has half
    // the half-step to land before the wait at its end.  (At d = 64 the
    // half-step is too short for that: back to back measures faster.)
    constexpr bool kSpreadV = kFenced && D == 128;
    constexpr int NSEGV = TL::kSegVPerWave;
    i32x4 rsV = {0, 0, 0, 0};
    uint32_t vsoff = 0, vlds = 0;
    if constexpr (ISSUE == 2 && kSpreadV) {
      rsV = uniform(buffer_rsrc(rq.base, (uint32_t)N * TL::kRowV));
      vsoff = __builtin_amdgcn_readfirstlane((uint32_t)rq.kb * TL::kRowV);
      vlds = __builtin_amdgcn_readfirstlane(lds_address(smem) + TL::kOffV + rq.buf * TL::kBytesV +
                                            wg * 1024);
    }
    if constexpr (ISSUE == 2 && !kSpreadV) {
      if (rq.on) issue_v<D, QK, PV>(smem, wg, rq.kb, rq.buf, rq.base, N, voff);
    }
    if constexpr (kFenced) {
      // The whole half-step in program order, fenced so that the scheduler
      // keeps it: product i is followed by the LDS reads of product
      // i + kAhead, so every operand is requested kAhead products (about
      // kAhead * 32 cycles, more than the LDS latency) before its use, also
      // across the switch from the P.V products to the S products.  The
      // loads of the next tiles are spread over the products.  No VALU
      // instruction sits in this stream: the wave sharing the SIMD runs a
      // dense VALU stream meanwhile, and an in-order wave whose VALU
      // instruction waits for the VALU port also holds back the products
      // behind it.  Four products ahead (~130 cycles) already cover the LDS
      // latency; at d = 128 the registers eight would hold cost spills, at
      // d = 64 eight measure faster.
      constexpr int kAhead = D == 128 ? 4 : 8;
      constexpr int NPV = DO_PV ? DT * (BC / 16) : 0;  // P.V products, u-major
      // fp8: one 32x32x64 product takes two 16-byte chunks of the row
      constexpr int SPC = QK == QK_F8 ? 2 : 1;         // chunks per S product
      constexpr int QSP = QST / SPC;                   // S products per 32-key subtile
      constexpr int NSM = DO_S ? NKS * QSP : 0;        // S products, chain by chain
      const char* vl = (const char*)smem + TL::kOffV + ((jg - 1) & 1) * TL::kBytesV + v_lane;
      const char* k0 = (const char*)smem + (jg & 1) * TL::kBytesK + k_lane + 16 * g;
      i16x4 vlo[NPV > 0 ? NPV : 1], vhi[NPV > 0 ? NPV : 1];
      i32x4 kf[NSM > 0 ? NSM : 1][SPC];
      // the S products accumulate straight into the score registers X
      // reads (a separate accumulator made the compiler copy all of them)
      if constexpr (DO_S) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) s[ks] = f32x16{};
      }
      auto load = [&](const int i) __attribute__((always_inline)) {
        if (i < NPV) {
          const char* src = vl + 16 * (i / DT) * TL::kStrV + 64 * (i % DT);
          vlo[i] = lds_read_tr16(src);
          vhi[i] = lds_read_tr16(src + 4 * TL::kStrV);
        } else {
          const int t = i - NPV;
#pragma unroll
          for (int c = 0; c < SPC; ++c)
            kf[t][c] = *(const i32x4*)(k0 + (t / QSP) * 32 * TL::kStrK + 32 * ((t % QSP) * SPC + c));
        }
      };
      auto product = [&](const int i) __attribute__((always_inline)) {
        if (i < NPV) {
          oacc[i % DT] = mfma_bf16(join_bf16x8(vlo[i], vhi[i]), pb[i / DT], oacc[i % DT]);
        } else {
          // 8-bit Q/K: raw int32 (or fp32 fp8) products; the end of the
          // half-step applies the key scales
          const int t = i - NPV;
          if constexpr (QK == QK_BF16)
            s[t / QST] = mfma_bf16(__builtin_bit_cast(bf16x8, kf[t][0]),
                                   __builtin_bit_cast(bf16x8, qv[t % QST]), s[t / QST]);
          else if constexpr (QK == QK_I8)
            s[t / QST] = __builtin_bit_cast(
                f32x16, mfma_i8(kf[t][0], qv[t % QST], __builtin_bit_cast(i32x16, s[t / QST])));
          else
            s[t / QSP] = mfma_fp8x4(kf[t][0], kf[t][1], qv[(t % QSP) * 2], qv[(t % QSP) * 2 + 1],
                                    s[t / QSP]);
        }
      };
      // The wave sharing this SIMD runs its softmax meanwhile; a dense VALU
      // stream would win the issue arbitration against the products, so
      // this wave raises its priority for the products and drops it after.
      __builtin_amdgcn_s_setprio(kPrioMfma);
#pragma unroll
      for (int i = 0; i < kAhead && i < NPV + NSM; ++i) load(i);
#pragma unroll
      for (int i = 0; i < NPV + NSM; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        product(i);
        if (i + kAhead < NPV + NSM) load(i + kAhead);
        if constexpr (ISSUE == 1) {
          static_for<NSEG>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            if ((2 * q + 1) * (NPV + NSM) / (2 * NSEG) == i) issue_one(qc, rq);
          });
        }
        if constexpr (ISSUE == 2 && kSpreadV) {
          static_for<NSEGV>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            if ((2 * q + 1) * (NPV + NSM) / (4 * NSEGV) == i && rq.on &&
                (TL::kSegV % TL::kIssuers == 0 || wg + q * TL::kIssuers < TL::kSegV))
              lds_load16<q * TL::kIssuers * 1024>(rsV, voff[q], vsoff, vlds);
          });
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (DEBUG_S && DO_S) {
        if (qvalid) {
          int32_t* dst = p.s_dbg + ((int64_t)bh * N + qrow) * (int64_t)N;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            // whole-vector cast: a bit_cast of one element of a vector
            // register is lowered as a read of element 0
            const i32x16 si = __builtin_bit_cast(i32x16, s[ks]);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = jl * BC + 32 * ks + elem_of_reg(r, g);
              if (key < N) dst[key] = si[r];
            }
          }
        }
      }
      if constexpr (DO_S && QK == QK_I8) {
        // exact int32 -> fp32 (|products| < 2^24) while the other wave of the
        // SIMD still runs its softmax
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const i32x16 si = __builtin_bit_cast(i32x16, s[ks]);  // whole-vector cast
#pragma unroll
          for (int r = 0; r < 16; ++r) s[ks][r] = (float)si[r];
        }
      }
      if constexpr (DO_S && kScaleInX) {
        // t = code product * key scale, here rather than in the softmax
        // half-step, which bounds the 8-bit steps (the matrix half-step has
        // the slack: its score products are a quarter (fp8) or half (int8)
        // as many instructions as bf16's)
        const float* skt = (const float*)(smem + TL::kOffSk + (jg & 1) * TL::kBytesSk);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const f32x4 a0 = *(const f32x4*)(skt + 32 * ks + 8 * g);
          const f32x4 a1 = *(const f32x4*)(skt + 32 * ks + 8 * g + 4);
          const f32x4 b0 = *(const f32x4*)(skt + 32 * ks + 16 + 8 * g);
          const f32x4 b1 = *(const f32x4*)(skt + 32 * ks + 16 + 8 * g + 4);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float sk = r < 4 ? a0[r] : r < 8 ? a1[r - 4] : r < 12 ? b0[r - 8] : b1[r - 12];
            s[ks][r] *= sk;
          }
        }
      }
      if constexpr (DO_S) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) pin(s[ks]);  // q.k (int8: times the key scale)
      }
      if constexpr (DO_PV) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) pin(oacc[dt]);
      }
#pragma unroll
      for (int u = 0; u < BC / 16; ++u) forget(pb[u]);
      if constexpr (!DO_S) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) forget(s[ks]);
      }
    } else {
      if constexpr (ISSUE == 1) {
        if (rq.on) issue_k<D, QK, PV>(smem, wg, lane, rq.kb, rq.buf, rq.skbuf, rq.base, rq.sbase, N, voff);
      }
      if constexpr (DO_PV) {
        const char* vt = (const char*)smem + TL::kOffV + ((jg - 1) & 1) * TL::kBytesV;
        if constexpr (PV == PV_BF16) {
          // key-group-outer order: P_{j-1} registers die group by group, so
          // they are gone before the new scores are born
          const char* vl = vt + v_lane;
#pragma unroll
          for (int u = 0; u < BC / 16; ++u)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const char* src = vl + 16 * u * TL::kStrV + 64 * dt;
              const i16x4 lo = lds_read_tr16(src);
              const i16x4 hi = lds_read_tr16(src + 4 * TL::kStrV);
              oacc[dt] = mfma_bf16(join_bf16x8(lo, hi), pb[u], oacc[dt]);
            }
#pragma unroll
          for (int u = 0; u < BC / 16; ++u) forget(pb[u]);
          pv_schedule<DT * (BC / 16)>();
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const VT* vr = (const VT*)(vt + (32 * ks + elem_of_reg(r, g)) * TL::kStrV) + n;
#pragma unroll
              for (int dt = 0; dt < DT; ++dt)
                oacc[dt] = mfma_f32(to_f32<VT>(vr[32 * dt]), pf[ks][r], oacc[dt]);
            }
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int r = 0; r < 16; ++r) forget(pf[ks][r]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < (PV == PV_BF16 ? BC / 16 : 1); ++u) forget(pb[u]);
#pragma unroll
        for (int ks = 0; ks < (PV == PV_BF16 ? 1 : NKS); ++ks)
#pragma unroll
          for (int r = 0; r < (PV == PV_BF16 ? 1 : 16); ++r) forget(pf[ks][r]);
      }
      if constexpr (!DO_S) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) forget(s[ks]);
      }
      if constexpr (DO_S) {
        const char* kt = (const char*)smem + (jg & 1) * TL::kBytesK;
        if constexpr (QK == QK_BF16) {
          f32x16 acc[NKS];
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) acc[ks] = f32x16{};
          // one accumulator chain at a time (back-to-back dependent products
          // issue at full rate), so that the score registers fill up gradually
          const char* k0 = kt + k_lane + 16 * g;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int st = 0; st < QST; ++st) {
              const i32x4 a = *(const i32x4*)(k0 + ks * 32 * TL::kStrK + 32 * st);
              acc[ks] = mfma_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qv[st]),
                                  acc[ks]);
            }
          s_schedule<NKS * QST>();
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[ks][r] = acc[ks][r];  // raw q.k; scaled inside exp2
        } else if constexpr (QK == QK_I8) {
          const float* skt = (const float*)(smem + TL::kOffSk + (jg & 1) * TL::kBytesSk);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const char* krow = kt + ks * 32 * TL::kStrK + k_lane + 16 * g;
            i32x16 acc = {};
#pragma unroll
            for (int st = 0; st < QST; ++st)
              acc = mfma_i8(*(const i32x4*)(krow + 32 * st), qv[st], acc);
            if constexpr (DEBUG_S) {
              if (qvalid) {
                int32_t* dst = p.s_dbg + ((int64_t)bh * N + qrow) * (int64_t)N;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const int key = jl * BC + 32 * ks + elem_of_reg(r, g);
                  if (key < N) dst[key] = acc[r];
                }
              }
            }
            // exact int32 -> fp32 (|acc| < 2^24), then the per-row scales
#pragma unroll
            for (int r = 0; r < 16; ++r)
              s[ks][r] = (float)acc[r] * (skt[32 * ks + elem_of_reg(r, g)] * sq_log2);
          }
        } else if constexpr (QK == QK_F8) {
          // E4M3 codes in the int8 layout: two fp8 products per 32-byte
          // chunk of the row, then the per-row scales as for int8
          const float* skt = (const float*)(smem + TL::kOffSk + (jg & 1) * TL::kBytesSk);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const char* krow = kt + ks * 32 * TL::kStrK + k_lane + 16 * g;
            f32x16 acc = {};
#pragma unroll
            for (int st = 0; st < QST; ++st)
              acc = mfma_fp8x2(*(const i32x4*)(krow + 32 * st), qv[st], acc);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              s[ks][r] = acc[r] * (skt[32 * ks + elem_of_reg(r, g)] * sq_log2);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const char* krow = kt + ks * 32 * TL::kStrK + k_lane;
            f32x16 acc = {};
#pragma unroll
            for (int st = 0; st < QST; ++st)
              acc = mfma_f32(*(const float*)(krow + 4 * (2 * st + g)), qf[st], acc);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[ks][r] = acc[r];
          }
        }
      }
    }
  };
  // ================= X_j: online softmax of block j
  auto half_x = [&](const int j) __attribute__((always_inline)) {
    const int kb = j * BC;
    // causal diagonal and ragged tail: invisible keys score -inf.  The test
    // is per 32-key subtile first (uniform across the wave): subtiles wholly
    // visible are left alone, wholly invisible ones are set to -inf, and
    // only a subtile the diagonal or the sequence end crosses is masked
    // element by element.
    // Without the causal mask the diagonal row is N (no key lies beyond
    // it), kept opaque so that both variants compile to the same code
    // shape (the optimiser's own specialisation of the non-causal one
    // spills registers).
    int diag0 = CAUSAL ? q0w : N;  // first query row of this wave
    int diag = CAUSAL ? qrow : N;  // this lane's query row
    asm volatile("" : "+s"(diag0), "+v"(diag));
    const bool need_mask = (kb + BC > N) || (kb + BC - 1 > diag0);
    if (need_mask) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int k0s = kb + 32 * ks;
        const bool all_vis = (k0s + 31 < N) && (k0s + 31 <= diag0);
        const bool none_vis = (k0s >= N) || (k0s > diag0 + 31);
        if (none_vis) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[ks][r] = -INFINITY;
        } else if (!all_vis) {
          // key of register r = k0s + 8g + c_r with c_r = 16(r/8) + r%8: the
          // tests compare the constant c_r with per-lane thresholds
          int lim_diag = diag - k0s - 8 * g;  // visible iff c_r <= lim_diag
          int lim_end = N - k0s - 8 * g;      // in range iff c_r < lim_end
          // opaque to the optimiser: otherwise it hoists the sixteen
          // compares of each subtile out of the loop as lane masks held in
          // scalar registers
          asm volatile("" : "+v"(lim_diag), "+v"(lim_end));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 16 * (r >> 3) + (r & 7);
            if (c >= lim_end || c > lim_diag) s[ks][r] = -INFINITY;
          }
        }
      }
    }
    // bf16/fp32 Q,K: s holds raw dot products; int8/fp8 Q,K with bf16 P:
    // code products times key scales.  The max is taken on them (the row
    // factor c is positive) and P = exp2(fma(s, c, -m)) with m = c * max:
    // one fma and one v_exp per score.  int8/fp8 with fp32 P: s is already
    // in log2 units, P = exp2(s - m).
    float flat[NKS * 16];
#pragma unroll
    for (int i = 0; i < NKS * 16; ++i) flat[i] = s[i / 16][i % 16];
    float mx = tree_max(flat);
    mx = pair32_max(mx);
    const float mraw_new = fmaxf(mraw_run, mx);
    // normaliser m of this block's probabilities P = exp2(s*c - m), in log2
    // units (int8: s is already scaled)
    // score factor: scale * log2(e) (bf16/fp32 Q, K), the row's
    // q_scale * scale * log2(e) (8-bit Q/K scaled here), none (8-bit Q/K
    // scaled in the matrix half-step)
    const float row_c = kScaleInX ? sq_log2 : p.scale_log2;
    float m_use = (kScaledQK<QK> && !kScaleInX) ? mraw_new : mraw_new * row_c;
    if constexpr (STAB) {
      // Stabilised variant ("Why Low-Precision Transformer Training Fails",
      // Figure 7 and Algorithm 1): when the row maximum r_m occurs more than
      // once, the normaliser becomes beta*r_m (r_m > 0) or 0 (r_m < 0), so
      // that no probability is exactly 1.  Occurrences are counted online:
      // those of this block's max in this block, added to the running count
      // while the running max is unchanged.
      int cnt = 0;
      if (mx != -INFINITY) {
#pragma unroll
        for (int i = 0; i < NKS * 16; ++i) cnt += (flat[i] == mx) ? 1 : 0;
      }
      cnt = pair32_isum(cnt);
      nmax_run = (mx > mraw_run) ? cnt : (mx == mraw_run ? nmax_run + cnt : nmax_run);
      if (nmax_run >= 2) {
        const float m_max = m_use;  // the running max in log2 units
        if (mraw_new > 0.f) m_use *= p.beta;
        else if (mraw_new < 0.f) m_use = 0.f;
        // Range guard: the page's rule puts the normaliser (beta-1)|r_m|
        // (r_m > 0) or |r_m| (r_m < 0) above the row max, which for large
        // |r_m| underflows every exp2 in fp32 and leaves l = 0, O = 0/0.
        // The shift is capped at kStabMaxShift, so the largest P stays at
        // or above 2^-kStabMaxShift (still below 1, as the variant wants);
        // inside the cap the rule applies unchanged.
        m_use = fminf(m_use, m_max + kStabMaxShift);
      }
    }
    mraw_run = mraw_new;
    if (m_use == -INFINITY) m_use = 0.f;  // every score so far masked
    const float alpha = exp2_approx(m_run - m_use);
    m_run = (mraw_new == -INFINITY) ? -INFINITY : m_use;
    // four independent partial row sums (a single += chain would serialise
    // on the add latency)
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (kScaledQK<QK> && !kScaleInX)
          s[ks][r] = exp2_approx(s[ks][r] - m_use);
        else
          s[ks][r] = exp2_approx(__builtin_fmaf(s[ks][r], row_c, -m_use));
        rsum[r & 3] += s[ks][r];
      }
    l_run = l_run * alpha + ((rsum[0] + rsum[1]) + (rsum[2] + rsum[3]));
    // At d = 128, exp(m - m') is often exactly 1 on every lane of a wave
    // late in long rows (no row max of the wave moved): multiplying by 1
    // changes no bit, so the rescale is skipped.  (At d = 64 the rows are
    // short and the test costs more than it saves.)
    if (D == 64 || __builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    if constexpr (PV == PV_BF16) {
#pragma unroll
      for (int u = 0; u < BC / 16; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[u][e] = (__bf16)s[u >> 1][8 * (u & 1) + e];
#pragma unroll
      for (int u = 0; u < BC / 16; ++u) pin(pb[u]);
    } else {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pf[ks][r] = p.p_round ? round_to_bf16(s[ks][r]) : s[ks][r];
          pin(pf[ks][r]);
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) pin(oacc[dt]);
    pin(l_run);
    pin(m_run);
    pin(mraw_run);
    if constexpr (STAB) pin(nmax_run);
  };

  // ---- epilogue of a finished tile: O = O^T / l, stored row-major, and the
  // optional log-sum-exp; then the running state restarts for the next tile
  auto finish = [&](int b, int row) __attribute__((always_inline)) {
    const float l_tot = pair32_sum(l_run);
    const float inv = 1.f / l_tot;
    const int64_t base = (int64_t)b * N * D + (int64_t)row * D;
    // O in fp32 (fp32 V, or asked for: a separate instance, so that the
    // bf16-output kernels carry no trace of it)
    constexpr bool f32out = sizeof(VT) == 4 || OF32;
    if constexpr (f32out) {
      if (row < N) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const int d0 = 32 * dt + 8 * b4 + 4 * g;
            *(float4*)((float*)p.o + base + d0) =
                make_float4(oacc[dt][4 * b4 + 0] * inv, oacc[dt][4 * b4 + 1] * inv,
                            oacc[dt][4 * b4 + 2] * inv, oacc[dt][4 * b4 + 3] * inv);
          }
      }
    } else {
      // Lane (n, g) holds, for each 8-column group b4 of a 32-column
      // subtile, columns 4g..4g+3 of row n (8 bytes once in bf16).  One
      // permlane32 swap per dword pairs the groups up: afterwards lane g
      // holds all eight columns of group 2k + g, so each store writes 16
      // bytes (half the store instructions of 8-byte pieces).  Both lanes
      // of a pair serve the same row, and the swaps run before the row
      // test, with every lane active.
      auto pk = [&](int dt, int r) __attribute__((always_inline)) {
        return (uint32_t)f32_to_bf16(oacc[dt][r] * inv) |
               ((uint32_t)f32_to_bf16(oacc[dt][r + 1] * inv) << 16);
      };
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          // group 2k (X) and 2k + 1 (Y), two dwords each
          const auto s0 = __builtin_amdgcn_permlane32_swap(pk(dt, 8 * k + 0), pk(dt, 8 * k + 4), false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(pk(dt, 8 * k + 2), pk(dt, 8 * k + 6), false, false);
          if (row < N)
            *(uint4*)((uint16_t*)p.o + base + 32 * dt + 16 * k + 8 * g) =
                make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
    }
    if (row < N && p.lse != nullptr && g == 0)
      p.lse[(int64_t)b * N + row] = (m_run + __log2f(l_tot)) * kLn2;
    m_run = -INFINITY;
    mraw_run = -INFINITY;
    l_run = 0.f;
    nmax_run = 0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  };

  // Slots.  Each group runs, tile after tile, the sequence
  //     M_0 X_0 M_1 X_1 ... M_{n-1} X_{n-1} M_n
  // (2n+1 slots, one workgroup barrier each; M_0 has no P.V part, M_n no S
  // part), group 1 one slot behind group 0: the two waves of a SIMD always
  // run opposite half-steps, except at a tile switch, where group 1's M_n
  // (P.V only) meets group 0's M_0 of the next tile (S only) -- the two
  // together are one full step of matrix work.  Group 1 starts with an idle
  // slot and group 0 ends with one, so both pass the same barriers.
  //
  // Blocks are numbered globally across the workgroup's tiles (jg); block
  // jg's K and V sit in buffers jg%2.  Only matrix half-steps issue loads:
  // group 0 issues the K loads of block jg+1 spread over its M of block jg
  // and awaits them at the end of the following X; group 1 issues the V
  // loads of block jg at the start of its M of block jg and awaits them at
  // the end of that M.  Either way the loads land before the first slot
  // that reads them, and the buffer they overwrite was last read in the
  // slot before the issuing one.  (Issued from the vector half-steps
  // instead, the loads measurably slow the kernel down.)  The next
  // tile's first K block continues this numbering, and its Q rows are
  // loaded at the start of X_{n-1}, after the last S products of the
  // current tile read Q.  A finished tile's O is stored at the start of the
  // next tile's X_0 (O, l and m are not touched by M_0).
  constexpr BoolC<true> kYes{};
  constexpr BoolC<false> kNo{};
  constexpr IntC<0> kIssueNone{};
  constexpr IntC<1> kIssueK{};
  constexpr IntC<2> kIssueV{};
  const Prefetch kNone{nullptr, nullptr, 0, 0, 0, false};
  bool pending = false;    // a finished tile's O waits in the registers
  int pend_bh = 0;
  int pend_row = 0;
  // the K (or V) block following local block j of the current tile
  auto next_k = [&](int j) __attribute__((always_inline)) {
    const bool same = j + 1 < cur.nblk;
    const int b = same ? cur.bh : nxt.bh;
    return Prefetch{head_ptr(p.k, b, sizeof(QT)),
                    kScaledQK<QK> ? (const void*)(p.k_scale + (int64_t)b * N) : nullptr,
                    same ? (j + 1) * BC : 0, (jg0 + j + 1) & 1, (jg0 + j + 1) & 1,
                    same || nxt.valid};
  };
  // the V block of local block j of the current tile
  auto this_v = [&](int j) __attribute__((always_inline)) {
    return Prefetch{head_ptr(p.v, cur.bh, sizeof(VT)), nullptr, j * BC, (jg0 + j) & 1, 0, true};
  };
  // start of X_j: the finished tile's output, the next tile's Q rows
  auto x_prologue = [&](int j) __attribute__((always_inline)) {
    if (j == 0 && pending) {
      finish(pend_bh, pend_row);
      pending = false;
    }
    if (j == cur.nblk - 1 && nxt.valid) load_q(nxt.bh, nxt.q0 + wave * 32 + n);
  };
  // after M_n: the next tile becomes current
  auto advance = [&]() __attribute__((always_inline)) {
    pending = true;
    pend_bh = bh;
    pend_row = qrow;
    jg0 += cur.nblk;
    cur = nxt;
    ++round;
    nxt = tile_of<CAUSAL, BC>(p, round + 1);
    bh = cur.bh;
    q0w = cur.q0 + wave * 32;
    qrow = q0w + n;
    qvalid = qrow < N;
    sq_log2 = sq_pend * p.scale_log2;
  };

  // end of group 0's X_j: the K loads issued in M_j (and any O stores) are
  // awaited; after the last X of a tile, which loads the next tile's Q rows,
  // those Q loads stay in flight (they are awaited at the end of M_n).
  // Top of a block loop.  Nothing is in flight here on any path that
  // reaches it (the last X of a tile, which leaves the next tile's Q loads in
  // flight, also leaves the loop), but the compiler cannot tell: without this
  // wait it assumes those Q loads may be pending and waits for them before
  // the S products, and since it does not count the buffer->LDS loads, that
  // wait would also cover the K/V loads issued earlier in the same half-step.
  auto loop_top_wait = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  };
  auto wait_x0 = [&](int j) __attribute__((always_inline)) {
    if (kQLoads >= 0 && j == cur.nblk - 1 && nxt.valid)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(kQLoads < 0 ? 0 : kQLoads));
    else
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  };
  if (group == 0) {
    while (true) {
      m_body(0, jg0, kNo, kYes, kIssueK, next_k(0));
      block_barrier();
      x_prologue(0);
      half_x(0);
      wait_x0(0);
      block_barrier();
      // Causal tiles: when the last key block lies wholly above group 0's
      // rows (the tile's first half), every score of it is masked for this
      // group, so P = 0 adds nothing to O and m, l stay as they are.  Group 0
      // then skips that block's S products, its softmax and its P.V
      // products, passing the same barriers (and still issuing the next
      // tile's loads).  Its waves' SIMD partners run those slots alone.
      const int nb = cur.nblk;
      const bool skip_last = CAUSAL && nb >= 2 && (nb - 1) * BC > cur.q0 + kBR / 2 - 1;
      for (int j = 1; j < nb - (skip_last ? 1 : 0); ++j) {
        loop_top_wait();
        m_body(j, jg0 + j, kYes, kYes, kIssueK, next_k(j));
        block_barrier();
        x_prologue(j);
        half_x(j);
        wait_x0(j);
        block_barrier();
      }
      if (skip_last) {
        m_body(nb - 1, jg0 + nb - 1, kYes, kNo, kIssueK, next_k(nb - 1));
        block_barrier();
        x_prologue(nb - 1);
        wait_x0(nb - 1);
        block_barrier();
      } else {
        m_body(nb, jg0 + nb, kYes, kNo, kIssueNone, kNone);
      }
      // the next tile's Q rows (loaded in the last X) before its S products
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      block_barrier();
      const bool more = nxt.valid;
      advance();
      if (!more) break;
    }
    finish(pend_bh, pend_row);
    block_barrier();
  } else {
    block_barrier();
    while (true) {
      m_body(0, jg0, kNo, kYes, kIssueV, this_v(0));
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      block_barrier();
      x_prologue(0);
      half_x(0);
      block_barrier();
      for (int j = 1; j < cur.nblk; ++j) {
        loop_top_wait();
        m_body(j, jg0 + j, kYes, kYes, kIssueV, this_v(j));
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        block_barrier();
        x_prologue(j);
        half_x(j);
        block_barrier();
      }
      m_body(cur.nblk, jg0 + cur.nblk, kYes, kNo, kIssueNone, kNone);
      // The next tile's Q rows (loaded in the last X) are awaited here, with
      // no load in flight behind them; otherwise the compiler waits for them
      // at their first use in the next M_0, which by then has issued that
      // tile's first V block, and the wait would cover it too.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      block_barrier();
      const bool more = nxt.valid;
      advance();
      if (!more) break;
    }
    finish(pend_bh, pend_row);
  }
}

template <int D, int QK, int PV, bool CAUSAL, bool DEBUG_S, bool STAB, bool OF32>
hipError_t launch_t(const FlashParams& fp, hipStream_t st) {
  hipLaunchKernelGGL((flash_fwd_kernel<D, QK, PV, CAUSAL, DEBUG_S, STAB, OF32>), dim3(fp.grid),
                     dim3(kThreads), 0, st, fp);
  return hipGetLastError();
}

template <int D, int QK, int PV, bool DEBUG_S, bool STAB, bool OF32>
hipError_t launch_c(const FlashParams& fp, bool causal, hipStream_t st) {
  return causal ? launch_t<D, QK, PV, true, DEBUG_S, STAB, OF32>(fp, st)
                : launch_t<D, QK, PV, false, DEBUG_S, STAB, OF32>(fp, st);
}

// bf16 or fp32 output
template <int D, int QK, int PV, bool STAB = false>
hipError_t launch_o(const FlashParams& fp, bool causal, bool of32, hipStream_t st) {
  return of32 ? launch_c<D, QK, PV, false, STAB, true>(fp, causal, st)
              : launch_c<D, QK, PV, false, STAB, false>(fp, causal, st);
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const FlashParams& fp, hipStream_t st) {
  const bool c = a.causal != 0;
  const bool o = a.o_f32 != 0;
  switch (a.dtype) {
    case kF32:
      return launch_c<D, QK_F32, PV_F32_VF32, false, false, false>(fp, c, st);
    case kBF16:
      if (a.stabilized)
        return a.p_bf16 ? launch_o<D, QK_BF16, PV_BF16, true>(fp, c, o, st)
                        : launch_o<D, QK_BF16, PV_F32_VBF16, true>(fp, c, o, st);
      return a.p_bf16 ? launch_o<D, QK_BF16, PV_BF16>(fp, c, o, st)
                      : launch_o<D, QK_BF16, PV_F32_VBF16>(fp, c, o, st);
    case kINT8:
      if (a.s_dbg != nullptr)
        return a.p_bf16 ? launch_c<D, QK_I8, PV_BF16, true, false, false>(fp, c, st)
                        : launch_c<D, QK_I8, PV_F32_VBF16, true, false, false>(fp, c, st);
      return a.p_bf16 ? launch_o<D, QK_I8, PV_BF16>(fp, c, o, st)
                      : launch_o<D, QK_I8, PV_F32_VBF16>(fp, c, o, st);
    case kFP8:
      return a.p_bf16 ? launch_o<D, QK_F8, PV_BF16>(fp, c, o, st)
                      : launch_o<D, QK_F8, PV_F32_VBF16>(fp, c, o, st);
  }
  return hipErrorInvalidValue;
}

// Compute units of the current device, queried once per device.
hipError_t compute_units(int* cus) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDev) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDev) cache[dev].store(*cus, std::memory_order_relaxed);
  return e;
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
  fp.beta = a.beta;
  const int64_t bh = a.batch * a.heads;
  const int ntiles = (int)((a.seq_len + kBR - 1) / kBR);
  fp.bh_count = bh;
  fp.q_tiles = ntiles;
  fp.tiles = bh * ntiles;
  // one workgroup per compute unit (the LDS footprint allows no second),
  // each walking its share of the tiles
  int cus = 0;
  hipError_t e = compute_units(&cus);
  if (e != hipSuccess) return e;
  fp.grid = (unsigned)(fp.tiles < (int64_t)cus ? fp.tiles : (int64_t)cus);
  // Four heads per XCD at a time keeps the re-read K/V rows of long causal
  // sequences in L2; it needs at least two rounds of tiles.  With fewer, the
  // global longest-first order, the second round dealt in reverse, gives every
  // workgroup a balanced share (e.g. 1.5 rounds of 2/4/6/8-block tiles: at most
  // 8 blocks per workgroup, against 10 in head groups).
  fp.grp4 = (bh % 32 == 0 && fp.grid % 8 == 0 && fp.tiles >= 2 * (int64_t)fp.grid) ? 1 : 0;
  if (a.head_dim == 64) return launch_d<64>(a, fp, stream);
  if (a.head_dim == 128) return launch_d<128>(a, fp, stream);
  return hipErrorInvalidValue;
}

}  // namespace pn
