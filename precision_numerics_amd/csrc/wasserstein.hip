// Wasserstein distances between the empirical distributions of two tensors
// of n values each ("Is Flash Attention Stable?", abstract: the deviation's
// impact measured with the Wasserstein distance; "Statistical Aspects of
// Wasserstein Distances", in its reference list).  On the real line the
// optimal coupling of two uniform n-point distributions pairs equal order
// statistics, so with a_(1) <= ... <= a_(n) and b_(1) <= ... <= b_(n)
//     W_1 = sum_i |a_(i) - b_(i)| / n,   W_2^2 = sum_i (a_(i) - b_(i))^2 / n,
//     W_inf = max_i |a_(i) - b_(i)|.
//
// Both inputs are sorted on the GPU by a stable LSD radix sort (8-bit digits)
// over order-preserving keys of their own width (bf16: 2 passes, fp32: 4,
// fp64: 8): negative values have all bits inverted, non-negative ones the
// sign bit set, so unsigned key order is numeric order.  Every pass is
//   histogram: workgroup g counts the digits of its contiguous chunk
//   offsets:   per digit, the keys of smaller digits plus a scan of that
//              digit's per-chunk counts
//   scatter:   workgroup g walks its chunk in tiles of 4096 elements; an
//              element's rank among equal digits of its wave comes from
//              eight ballots, the runs' counts are prefix-summed per digit
//              in LDS into a digit-sorted copy of the tile, which leaves as
//              one contiguous run per digit; element order is kept
//              throughout, so the sort is stable
// The distances then come from one pass over both sorted key arrays with a
// fixed element-to-thread map and fixed reduction trees (bitwise
// reproducible).  Values are decoded exactly to fp64.  Off the attention hot
// path: HBM-bound, a few full passes over the keys.
#include "device.hpp"
#include "launch.hpp"

namespace pn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBlocks = 1024;

template <typename K> struct KeyTraits;
template <> struct KeyTraits<uint16_t> {
  static constexpr uint16_t kSign = 0x8000u;
  static constexpr uint16_t kExp = 0x7f80u;  // bf16 exponent field
  __device__ static double decode_bits(uint16_t b) { return (double)bf16_to_f32(b); }
};
template <> struct KeyTraits<uint32_t> {
  static constexpr uint32_t kSign = 0x80000000u;
  static constexpr uint32_t kExp = 0x7f800000u;
  __device__ static double decode_bits(uint32_t b) { return (double)__uint_as_float(b); }
};
template <> struct KeyTraits<uint64_t> {
  static constexpr uint64_t kSign = 0x8000000000000000ull;
  static constexpr uint64_t kExp = 0x7ff0000000000000ull;
  __device__ static double decode_bits(uint64_t b) { return __longlong_as_double((long long)b); }
};

template <typename K>
__device__ __forceinline__ K to_key(K bits) {
  return (bits & KeyTraits<K>::kSign) ? (K)~bits : (K)(bits | KeyTraits<K>::kSign);
}
template <typename K>
__device__ __forceinline__ double from_key(K key) {
  const K bits = (key & KeyTraits<K>::kSign) ? (K)(key & (K)~KeyTraits<K>::kSign) : (K)~key;
  return KeyTraits<K>::decode_bits(bits);
}

// keys of the raw values, and per-workgroup counts of non-finite values
template <typename K>
__global__ __launch_bounds__(kThreads) void make_keys(const K* x, int64_t n, int64_t chunk,
                                                      K* keys, uint32_t* nonfinite) {
  __shared__ uint32_t cnt;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  uint32_t bad = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
    const K b = x[i];
    bad += ((b & KeyTraits<K>::kExp) == KeyTraits<K>::kExp) ? 1u : 0u;
    keys[i] = to_key(b);
  }
  if (bad) atomicAdd(&cnt, bad);
  __syncthreads();
  if (threadIdx.x == 0) nonfinite[blockIdx.x] = cnt;
}

// counts[d * G + g] = elements of chunk g whose digit is d
template <typename K>
__global__ __launch_bounds__(kThreads) void digit_histogram(const K* keys, int64_t n,
                                                            int64_t chunk, int shift,
                                                            uint32_t* counts) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads)
    atomicAdd(&h[(uint32_t)(keys[i] >> shift) & 255u], 1u);
  __syncthreads();
  counts[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = h[threadIdx.x];
}

// offsets[d * G + g] = number of keys with a smaller digit, plus those with
// digit d in chunks before g.  digit_totals: workgroup d sums its digit's G
// <= 1024 counts; digit_offsets: workgroup d adds the totals of the smaller
// digits and scans its own counts (one per thread).  Integer sums: exact in
// any order.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void digit_totals(const uint32_t* counts, int G,
                                                             uint32_t* totals) {
  __shared__ uint32_t red[kScanThreads / 64];
  const int d = blockIdx.x, t = threadIdx.x;
  uint32_t c = t < G ? counts[d * G + t] : 0u;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if ((t & 63) == 0) red[t >> 6] = c;
  __syncthreads();
  if (t == 0) {
    uint32_t sum = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) sum += red[w];
    totals[d] = sum;
  }
}
__global__ __launch_bounds__(kScanThreads) void digit_offsets(const uint32_t* counts, int G,
                                                              const uint32_t* totals,
                                                              uint32_t* offsets) {
  __shared__ uint32_t part[kScanThreads];
  __shared__ uint32_t red[kScanThreads / 64];
  const int d = blockIdx.x, t = threadIdx.x;
  uint32_t below = t < d ? totals[t] : 0u;  // d < 256 <= kScanThreads
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) below += __shfl_xor(below, off);
  if ((t & 63) == 0) red[t >> 6] = below;
  const uint32_t c = t < G ? counts[d * G + t] : 0u;
  part[t] = c;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) base += red[w];
  // Hillis-Steele inclusive scan of this digit's counts
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const uint32_t v = t >= off ? part[t - off] : 0u;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  if (t < G) offsets[d * G + t] = base + part[t] - c;
}

// Stable scatter of chunk g by the digit at `shift`.  The chunk is walked in
// tiles of kTileE * kThreads elements (element t + kThreads * s of a tile in
// lane t, sub-tile s):
//   1. every lane ranks its elements among the equal digits of its wave and
//      sub-tile (eight ballots); each run's first lane records the run's
//      length per (sub-tile, wave, digit)
//   2. lane d turns the counts of digit d into starts in (sub-tile, wave)
//      order, i.e. element order, and the tile's digit totals are scanned
//      into the tile's digit-sorted layout
//   3. every element goes to its place in that layout, in LDS
//   4. lanes read the layout in order and write each element to the
//      chunk's current global start of its digit plus its place in the
//      digit's run: the elements of one digit leave as one contiguous run
//      (consecutive lanes, consecutive addresses) instead of one key each
// Within a digit, tiles, sub-tiles, waves and lanes follow element order,
// so the sort stays stable.
constexpr int kTileE = 16;
template <typename K>
__global__ __launch_bounds__(kThreads) void digit_scatter(const K* in, int64_t n, int64_t chunk,
                                                          int shift, const uint32_t* offsets,
                                                          K* out) {
  constexpr int kTile = kTileE * kThreads;
  __shared__ uint32_t gbase[256];                   // global start of the chunk's digit-d run
  __shared__ uint32_t tstart[256];                  // start of digit d in the tile layout
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint16_t cnt[kTileE][kWaves][256];     // run lengths, then run starts
  __shared__ K stage[kTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  gbase[tid] = offsets[(int64_t)tid * gridDim.x + blockIdx.x];
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes below this one
  for (int64_t t0 = lo; t0 < hi; t0 += kTile) {
    K key[kTileE];
    uint32_t dig[kTileE], rank[kTileE];
    bool valid[kTileE];
#pragma unroll
    for (int e = 0; e < kTileE; ++e) {
      const int64_t i = t0 + (int64_t)e * kThreads + tid;
      valid[e] = i < hi;
      key[e] = valid[e] ? in[i] : (K)0;
    }
#pragma unroll
    for (int e = 0; e < kTileE; ++e)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) cnt[e][w][tid] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kTileE; ++e) {
      dig[e] = (uint32_t)(key[e] >> shift) & 255u;
      uint64_t peers = __builtin_amdgcn_ballot_w64(valid[e]);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool on = (dig[e] >> bit) & 1u;
        const uint64_t m = __builtin_amdgcn_ballot_w64(on);
        peers &= on ? m : ~m;
      }
      rank[e] = (uint32_t)__builtin_popcountll(peers & lt);
      if (valid[e] && rank[e] == 0) cnt[e][wave][dig[e]] = (uint16_t)__builtin_popcountll(peers);
    }
    __syncthreads();
    // lane d: starts of digit d's runs inside the digit, in element order,
    // and the digit's total in this tile
    uint32_t run = 0;
#pragma unroll
    for (int e = 0; e < kTileE; ++e)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const uint32_t c = cnt[e][w][tid];
        cnt[e][w][tid] = (uint16_t)run;
        run += c;
      }
    // exclusive scan of the digit totals: in-wave, then across the waves
    uint32_t inc = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(inc, off);
      if (lane >= off) inc += v;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) before += w < wave ? wsum[w] : 0u;
    const uint32_t my_start = before + inc - run;
    tstart[tid] = my_start;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kTileE; ++e)
      if (valid[e]) stage[tstart[dig[e]] + cnt[e][wave][dig[e]] + rank[e]] = key[e];
    __syncthreads();
    const int64_t m = hi - t0 < kTile ? hi - t0 : kTile;   // elements in this tile
#pragma unroll
    for (int e = 0; e < kTileE; ++e) {
      const int p = e * kThreads + tid;
      if (p < m) {
        const K k = stage[p];
        const uint32_t d = (uint32_t)(k >> shift) & 255u;
        // the position lies in [0, n) by construction; the test keeps a
        // counting error from ever writing outside the buffer
        const uint32_t pos = gbase[d] + (uint32_t)p - tstart[d];
        if ((int64_t)pos < n) out[pos] = k;
      }
    }
    __syncthreads();
    gbase[tid] += run;
    // the next tile's first barrier orders this update before its reads
  }
}

struct WPartial {
  double sum_abs, sum_sq, max_abs;
};

__device__ __forceinline__ void wfold(WPartial& a, const WPartial& b) {
  a.sum_abs += b.sum_abs;
  a.sum_sq += b.sum_sq;
  a.max_abs = fmax(a.max_abs, b.max_abs);
}

__device__ void wtree(WPartial& mine, WPartial* lds) {
  lds[threadIdx.x] = mine;
  __syncthreads();
  for (int s = kThreads / 2; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) wfold(lds[threadIdx.x], lds[threadIdx.x + s]);
    __syncthreads();
  }
}

template <typename KA, typename KB>
__global__ __launch_bounds__(kThreads) void quantile_gaps(const KA* a, const KB* b, int64_t n,
                                                          int64_t chunk, WPartial* parts) {
  __shared__ WPartial lds[kThreads];
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  WPartial mine{0.0, 0.0, 0.0};
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
    const double g = fabs(from_key(a[i]) - from_key(b[i]));
    mine.sum_abs += g;
    mine.sum_sq += g * g;
    mine.max_abs = fmax(mine.max_abs, g);
  }
  wtree(mine, lds);
  if (threadIdx.x == 0) parts[blockIdx.x] = lds[0];
}

__global__ __launch_bounds__(kThreads) void gaps_fold(const WPartial* parts, int nparts,
                                                      const uint32_t* nonfinite, int nbad,
                                                      WassersteinRecord* out) {
  __shared__ WPartial lds[kThreads];
  __shared__ uint32_t bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  WPartial mine{0.0, 0.0, 0.0};
  for (int i = threadIdx.x; i < nparts; i += kThreads) wfold(mine, parts[i]);
  uint32_t nb = 0;
  for (int i = threadIdx.x; i < nbad; i += kThreads) nb += nonfinite[i];
  if (nb) atomicAdd(&bad, nb);
  wtree(mine, lds);
  if (threadIdx.x == 0) {
    out->sum_abs = lds[0].sum_abs;
    out->sum_sq = lds[0].sum_sq;
    out->max_abs = lds[0].max_abs;
    out->n_nonfinite = bad;
  }
}

int blocks_for(int64_t n) {
  int64_t b = (n + (int64_t)kThreads * 64 - 1) / ((int64_t)kThreads * 64);
  if (b < 1) b = 1;
  if (b > kMaxBlocks) b = kMaxBlocks;
  return (int)b;
}

size_t key_bytes(int dtype) { return dtype == kBF16 ? 2 : (dtype == kF32 ? 4 : 8); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t a0, a1, b0, b1, counts, totals, offsets, bad, parts, rec, total;
};

Layout layout(int64_t n, int a_dtype, int b_dtype) {
  const size_t G = (size_t)blocks_for(n);
  Layout l;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at = align256(at + bytes);
    return here;
  };
  l.a0 = take((size_t)n * key_bytes(a_dtype));
  l.a1 = take((size_t)n * key_bytes(a_dtype));
  l.b0 = take((size_t)n * key_bytes(b_dtype));
  l.b1 = take((size_t)n * key_bytes(b_dtype));
  l.counts = take(256 * G * 4);
  l.totals = take(256 * 4);
  l.offsets = take(256 * G * 4);
  l.bad = take(2 * G * 4);
  l.parts = take(G * sizeof(WPartial));
  l.rec = take(sizeof(WassersteinRecord));
  l.total = at;
  return l;
}

// sort the n keys of `x` (dtype) into scratch; returns the buffer holding them
template <typename K>
hipError_t sort_keys(const void* x, int64_t n, char* scratch, size_t off0, size_t off1,
                     const Layout& l, uint32_t* bad, hipStream_t st, size_t* result) {
  const int G = blocks_for(n);
  const int64_t chunk = (n + G - 1) / G;
  K* buf[2] = {(K*)(scratch + off0), (K*)(scratch + off1)};
  uint32_t* counts = (uint32_t*)(scratch + l.counts);
  uint32_t* totals = (uint32_t*)(scratch + l.totals);
  uint32_t* offsets = (uint32_t*)(scratch + l.offsets);
  hipLaunchKernelGGL((make_keys<K>), dim3(G), dim3(kThreads), 0, st, (const K*)x, n, chunk,
                     buf[0], bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int cur = 0;
  for (int shift = 0; shift < (int)(8 * sizeof(K)); shift += 8) {
    hipLaunchKernelGGL((digit_histogram<K>), dim3(G), dim3(kThreads), 0, st, buf[cur], n, chunk,
                       shift, counts);
    hipLaunchKernelGGL(digit_totals, dim3(256), dim3(kScanThreads), 0, st, counts, G, totals);
    hipLaunchKernelGGL(digit_offsets, dim3(256), dim3(kScanThreads), 0, st, counts, G, totals, offsets);
    hipLaunchKernelGGL((digit_scatter<K>), dim3(G), dim3(kThreads), 0, st, buf[cur], n, chunk,
                       shift, offsets, buf[cur ^ 1]);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    cur ^= 1;
  }
  *result = cur ? off1 : off0;
  return hipSuccess;
}

hipError_t sort_any(int dtype, const void* x, int64_t n, char* scratch, size_t off0, size_t off1,
                    const Layout& l, uint32_t* bad, hipStream_t st, size_t* result) {
  if (dtype == kBF16) return sort_keys<uint16_t>(x, n, scratch, off0, off1, l, bad, st, result);
  if (dtype == kF32) return sort_keys<uint32_t>(x, n, scratch, off0, off1, l, bad, st, result);
  return sort_keys<uint64_t>(x, n, scratch, off0, off1, l, bad, st, result);
}

template <typename KA, typename KB>
void launch_gaps(const void* a, const void* b, int64_t n, int G, int64_t chunk, WPartial* parts,
                 hipStream_t st) {
  hipLaunchKernelGGL((quantile_gaps<KA, KB>), dim3(G), dim3(kThreads), 0, st, (const KA*)a,
                     (const KB*)b, n, chunk, parts);
}

template <typename KA>
void launch_gaps_b(int b_dtype, const void* a, const void* b, int64_t n, int G, int64_t chunk,
                   WPartial* parts, hipStream_t st) {
  if (b_dtype == kBF16) launch_gaps<KA, uint16_t>(a, b, n, G, chunk, parts, st);
  else if (b_dtype == kF32) launch_gaps<KA, uint32_t>(a, b, n, G, chunk, parts, st);
  else launch_gaps<KA, uint64_t>(a, b, n, G, chunk, parts, st);
}

}  // namespace

size_t wasserstein_scratch_bytes(int64_t n, int a_dtype, int b_dtype) {
  return layout(n, a_dtype, b_dtype).total;
}

hipError_t launch_wasserstein(const void* a, int a_dtype, const void* b, int b_dtype, int64_t n,
                              void* scratch_v, WassersteinRecord* out_host, hipStream_t st) {
  char* scratch = (char*)scratch_v;
  const Layout l = layout(n, a_dtype, b_dtype);
  const int G = blocks_for(n);
  const int64_t chunk = (n + G - 1) / G;
  uint32_t* bad = (uint32_t*)(scratch + l.bad);
  size_t ka = 0, kb = 0;
  hipError_t e = sort_any(a_dtype, a, n, scratch, l.a0, l.a1, l, bad, st, &ka);
  if (e != hipSuccess) return e;
  e = sort_any(b_dtype, b, n, scratch, l.b0, l.b1, l, bad + G, st, &kb);
  if (e != hipSuccess) return e;
  WPartial* parts = (WPartial*)(scratch + l.parts);
  if (a_dtype == kBF16) launch_gaps_b<uint16_t>(b_dtype, scratch + ka, scratch + kb, n, G, chunk, parts, st);
  else if (a_dtype == kF32) launch_gaps_b<uint32_t>(b_dtype, scratch + ka, scratch + kb, n, G, chunk, parts, st);
  else launch_gaps_b<uint64_t>(b_dtype, scratch + ka, scratch + kb, n, G, chunk, parts, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  WassersteinRecord* rec = (WassersteinRecord*)(scratch + l.rec);
  hipLaunchKernelGGL(gaps_fold, dim3(1), dim3(kThreads), 0, st, parts, G, bad, 2 * G, rec);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(out_host, rec, sizeof(WassersteinRecord), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace pn
