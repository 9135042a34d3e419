// Sort of (key, position) pairs by key, positions ascending inside a key, for
// grouping a batch's positions by a 64-bit ID (dedup), where an LSD radix
// sort would need eight passes.  Every pair is distinct (its
// position is), so sorting by the pair itself gives exactly the stable order;
// no pass has to preserve input order.
//
//   tile_sort_kernel    a block sorts a tile of 2048 or 16384 pairs (16 per
//                       thread in registers, then merge levels through LDS),
//                       so runs of a tile are sorted;
//   merge_round_kernel  runs of L are merged pairwise into runs of 2L.  A
//                       block writes kMsOut consecutive outputs: two waves
//                       find where its output range starts and ends in the
//                       two runs (merge path: the count a of first-run
//                       elements among the first o outputs) by a 64-way
//                       search, each round one load per lane, so a run of
//                       2^17 takes three dependent loads, not seventeen; the
//                       block then stages both input pieces in LDS and each
//                       thread merges kMsOut / 256 outputs.  Small output
//                       blocks (256) put many blocks on the GPU per round:
//                       a round is latency-bound (three dependent searches,
//                       then the staging), so more, shorter blocks finish it
//                       sooner.
//
// With a device count of active elements (a compacted input), only the first
// *nact slots take part: tiles and output blocks past it exit at once, so a
// sort costs what it keeps.  The number of merge rounds follows the slot
// count n; the tile sort writes in place or to the other buffer so that the
// result always lands in buffer 1.
#pragma once

#include "hlr_common.hpp"

namespace {

constexpr int kMsThreads = 256;  // merge rounds
constexpr int kMsOut = 256;      // outputs per block in a merge round (one per thread)

// Tile sort: 16 pairs per thread; 1024 threads (16384 pairs) for 32-bit keys,
// 128 (2048 pairs) for 64-bit keys.  A 65,536-ID dedup (32 tiles, five merge
// rounds of 256-output blocks) takes 64.6 us; with tiles of 8192 pairs and
// 2048-output blocks (three rounds of 32 blocks) it took 86.2 us, with tiles
// of 4096 and 256-output blocks 65.4 us, 512-output blocks 67.2 us.
template <typename K>
constexpr int ms_tile_threads() { return sizeof(K) == 4 ? 1024 : 128; }
template <typename K>
constexpr int64_t ms_tile() { return static_cast<int64_t>(ms_tile_threads<K>()) * 16; }
constexpr int kMsResultBuffer = 1;

__device__ __forceinline__ int64_t ms_active(int64_t n, const uint32_t *nact) {
  if (!nact) return n;
  const int64_t m = static_cast<int64_t>(*nact);
  return m < n ? m : n;
}

template <typename K>
__device__ __forceinline__ bool pair_less(K ak, uint32_t av, K bk, uint32_t bv) {
  return ak < bk || (ak == bk && av < bv);
}

inline int merge_rounds(int64_t n, int64_t tile) {
  int r = 0;
  for (int64_t L = tile; L < n; L <<= 1) ++r;
  return r;
}

// Compare-exchange of two pairs into ascending order.
template <typename K>
__device__ __forceinline__ void ms_cx(K &ak, uint32_t &av, K &bk, uint32_t &bv) {
  if (pair_less(bk, bv, ak, av)) {
    const K tk = ak;
    const uint32_t tv = av;
    ak = bk;
    av = bv;
    bk = tk;
    bv = tv;
  }
}

// Sorts a thread's 16 pairs in registers (bitonic network, constant indices).
template <typename K>
__device__ __forceinline__ void ms_sort16(K (&x)[16], uint32_t (&y)[16]) {
#pragma unroll
  for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((e & j) == 0) {
          if ((e & k) == 0) ms_cx(x[e], y[e], x[e | j], y[e | j]);
          else ms_cx(x[e | j], y[e | j], x[e], y[e]);
        }
}

// LDS slot of tile element i: one pad slot after every 16, so that the 16
// stores of a thread's run (lanes 16 apart) fall into different banks.
__device__ __forceinline__ int ms_lds(int i) { return i + (i >> 4); }

// One tile of NT * 16 pairs per block (thread t owns elements 16t .. 16t+15):
// each thread sorts its 16 pairs in registers, then log2(NT) merge levels
// double the sorted runs: the threads write their runs to LDS, and each thread
// finds where its 16 outputs start in the two runs it merges (binary search,
// the merge path) and merges them into its registers.  The input may be the
// output buffer (in place): each block reads its own tile whole before writing it.
// Reads pair g of the input: from a (keys, positions) buffer pair.
template <typename K>
struct PairsIn {
  const K *k;
  const uint32_t *v;
  __device__ __forceinline__ void operator()(int64_t g, K *key, uint32_t *pos) const {
    *key = k[g];
    *pos = v[g];
  }
};

template <typename K, int NT, typename Load>
__global__ void __launch_bounds__(NT)
    tile_sort_kernel(Load load, K *kout, uint32_t *vout, int64_t n, const uint32_t *nact) {
  constexpr int E = 16;
  constexpr int T = NT * E;
  __shared__ K sk[T + T / 16];
  __shared__ uint32_t sv[T + T / 16];
  const int64_t m = ms_active(n, nact);
  const int64_t base = static_cast<int64_t>(blockIdx.x) * T;
  if (base >= m) return;
  const int t = threadIdx.x;
  K x[E];
  uint32_t y[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t g = base + t * E + e;
    x[e] = ~K(0);  // padding sorts last and is never written out
    y[e] = 0xffffffffu;
    if (g < m) load(g, &x[e], &y[e]);
  }
  ms_sort16(x, y);
  for (int R = E; R < T; R <<= 1) {  // runs of R -> runs of 2R
    if (R > E) __syncthreads();        // the previous level has read its runs
#pragma unroll
    for (int e = 0; e < E; ++e) {
      sk[ms_lds(t * E + e)] = x[e];
      sv[ms_lds(t * E + e)] = y[e];
    }
    __syncthreads();
    const int p0 = (t * E) & ~(2 * R - 1);  // the pair of runs: A at p0, B at p0 + R
    const int o = t * E - p0;               // this thread's first output in the pair
    int lo = o > R ? o - R : 0, hi = o < R ? o : R;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const int ia = ms_lds(p0 + mid), ib = ms_lds(p0 + R + o - mid - 1);
      if (pair_less(sk[ia], sv[ia], sk[ib], sv[ib])) lo = mid + 1;
      else hi = mid;
    }
    int ia = lo, ib = o - lo;
    K ak = sk[ms_lds(p0 + (ia < R ? ia : R - 1))], bk = sk[ms_lds(p0 + R + (ib < R ? ib : R - 1))];
    uint32_t av = sv[ms_lds(p0 + (ia < R ? ia : R - 1))], bv = sv[ms_lds(p0 + R + (ib < R ? ib : R - 1))];
    // branch-free steps: one load per output, the index and the register it
    // refills chosen by selects (a per-lane branch would issue and wait for both)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool take_a = ia < R && (ib >= R || pair_less(ak, av, bk, bv));
      x[e] = take_a ? ak : bk;
      y[e] = take_a ? av : bv;
      ia += take_a ? 1 : 0;
      ib += take_a ? 0 : 1;
      const int q = take_a ? ms_lds(p0 + (ia < R ? ia : R - 1)) : ms_lds(p0 + R + (ib < R ? ib : R - 1));
      const K nk = sk[q];
      const uint32_t nv = sv[q];
      ak = take_a ? nk : ak;
      av = take_a ? nv : av;
      bk = take_a ? bk : nk;
      bv = take_a ? bv : nv;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t g = base + t * E + e;
    if (g < m) {
      kout[g] = x[e];
      vout[g] = y[e];
    }
  }
}

// Merge path: the number of elements of run A (at a0, na long) among the first
// o outputs of merge(A, B) (B at b0, nb long), 0 <= o <= na + nb.  For a in
// [lo, hi) the test A[a] < B[o - a - 1] holds exactly for a below the answer;
// each round the 64 lanes test evenly spaced a and the interval shrinks to one
// spacing.  Called by a whole wave; the result is wave-uniform.
template <typename K>
__device__ int64_t corank_wave(const K *__restrict__ k, const uint32_t *__restrict__ v, int64_t a0, int64_t na,
                               int64_t b0, int64_t nb, int64_t o) {
  int64_t lo = o > nb ? o - nb : 0;
  int64_t hi = o < na ? o : na;
  const int lane = hlr::lane_id();
  while (lo < hi) {
    const int64_t span = hi - lo;
    const int64_t step = (span + 63) / 64;
    const int64_t tested = (span + step - 1) / step;  // lanes with a < hi (<= 64)
    const int64_t a = lo + lane * step;
    bool g = false;
    if (lane < tested) {
      const int64_t ia = a0 + a, ib = b0 + (o - a - 1);
      g = pair_less(k[ia], v[ia], k[ib], v[ib]);
    }
    const int64_t t = __popcll(hlr::ballot(g));  // the lanes that hold form a prefix
    const int64_t nlo = t > 0 ? lo + (t - 1) * step + 1 : lo;
    const int64_t nhi = t < tested ? lo + t * step : hi;
    lo = nlo;
    hi = nhi;
  }
  return lo;
}

template <typename K>
__global__ void __launch_bounds__(kMsThreads)
    merge_round_kernel(const K *__restrict__ kin, const uint32_t *__restrict__ vin, K *__restrict__ kout,
                       uint32_t *__restrict__ vout, int64_t n, const uint32_t *nact, int64_t L) {
  constexpr int kPer = kMsOut / kMsThreads;
  __shared__ K sk[kMsOut];
  __shared__ uint32_t sv[kMsOut];
  __shared__ int64_t cr[2];
  const int64_t m = ms_active(n, nact);
  const int64_t out0 = static_cast<int64_t>(blockIdx.x) * kMsOut;
  if (out0 >= m) return;
  const int64_t p0 = out0 / (2 * L) * (2 * L);  // the pair of runs this block's outputs come from
  const int64_t na = L < m - p0 ? L : m - p0;     // >= 1, as m > out0 >= p0
  const int64_t b0 = p0 + na;
  const int64_t nb = m - b0 < L ? (m - b0 > 0 ? m - b0 : 0) : L;
  const int64_t o0 = out0 - p0;
  const int64_t o1 = o0 + kMsOut < na + nb ? o0 + kMsOut : na + nb;
  const int w = threadIdx.x / hlr::kWave;
  if (w < 2) {
    const int64_t a = corank_wave(kin, vin, p0, na, b0, nb, w == 0 ? o0 : o1);
    if (hlr::lane_id() == 0) cr[w] = a;
  }
  __syncthreads();
  const int64_t ca0 = cr[0], ca1 = cr[1];
  const int nA = static_cast<int>(ca1 - ca0);
  const int nB = static_cast<int>((o1 - ca1) - (o0 - ca0));
  const int total = nA + nB;  // = o1 - o0 <= kMsOut
  for (int i = threadIdx.x; i < total; i += kMsThreads) {
    const int64_t g = i < nA ? p0 + ca0 + i : b0 + (o0 - ca0) + (i - nA);
    sk[i] = kin[g];
    sv[i] = vin[g];
  }
  __syncthreads();
  const int x0 = threadIdx.x * kPer;
  if (x0 >= total) return;
  // this thread's start in the staged pieces: A = [0, nA), B = [nA, total)
  int lo = x0 > nB ? x0 - nB : 0, hi = x0 < nA ? x0 : nA;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pair_less(sk[mid], sv[mid], sk[nA + x0 - mid - 1], sv[nA + x0 - mid - 1])) lo = mid + 1;
    else hi = mid;
  }
  // branch-free steps as in the tile sort; A = [0, nA), B = [nA, total) of the staged pieces
  int ia = lo, ib = x0 - lo;
  const int x1 = x0 + kPer < total ? x0 + kPer : total;
  const int last = total - 1;
  int qa = ia < nA ? ia : last, qb = nA + ib < total ? nA + ib : last;
  K ak = sk[qa], bk = sk[qb];
  uint32_t av = sv[qa], bv = sv[qb];
  K ok[kPer];
  uint32_t ov[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const bool take_a = ia < nA && (ib >= nB || pair_less(ak, av, bk, bv));
    ok[u] = take_a ? ak : bk;
    ov[u] = take_a ? av : bv;
    ia += take_a ? 1 : 0;
    ib += take_a ? 0 : 1;
    const int q = take_a ? (ia < nA ? ia : last) : (nA + ib < total ? nA + ib : last);
    const K nk = sk[q];
    const uint32_t nv = sv[q];
    ak = take_a ? nk : ak;
    av = take_a ? nv : av;
    bk = take_a ? bk : nk;
    bv = take_a ? bv : nv;
  }
  const int64_t dst = p0 + o0;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (x0 + u < x1) {
      kout[dst + x0 + u] = ok[u];
      vout[dst + x0 + u] = ov[u];
    }
}

// Sorts the pairs that `load` reads (pair g for g below n, or below *nact when
// given) into (k, v); the result is in buffer kMsResultBuffer.
template <typename K, typename Load>
inline int merge_sort_pairs(Load load, K *const k[2], uint32_t *const v[2], int64_t n, const uint32_t *nact,
                            hipStream_t s) {
  constexpr int64_t tile = ms_tile<K>();
  const int rounds = merge_rounds(n, tile);
  int cur = (rounds % 2 == 0) ? kMsResultBuffer : kMsResultBuffer ^ 1;
  const int tiles = static_cast<int>((n + tile - 1) / tile);
  tile_sort_kernel<K, ms_tile_threads<K>(), Load><<<tiles, ms_tile_threads<K>(), 0, s>>>(load, k[cur], v[cur], n,
                                                                                        nact);
  const int blocks = static_cast<int>((n + kMsOut - 1) / kMsOut);
  int64_t L = tile;
  for (int r = 0; r < rounds; ++r, L <<= 1) {
    merge_round_kernel<K><<<blocks, kMsThreads, 0, s>>>(k[cur], v[cur], k[cur ^ 1], v[cur ^ 1], n, nact, L);
    cur ^= 1;
  }
  return cur;
}

}  // namespace
