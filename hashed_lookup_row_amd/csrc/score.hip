// Serving score: int8 row dequantisation fused with a dot product against the
// request's user vector.  "Memory Layer: Train the In-Model Cache for
// Recommendation Models": sec. 1 (early-stage ranking scores about a thousand
// candidates per request), sec. 5 (the serving side reads int8-quantised rows),
// sec. 2 (a miss zeroes the cached branch: score 0).
//
// sum_d (q_d*scale + bias)*u_d = scale*sum_d q_d*u_d + bias*sum_d u_d, all in
// fp64: q_d*u_d is exact in fp64 (8-bit times 24-bit significands), so each
// candidate costs one fp64 FMA per element plus two per candidate, and the
// only fp32 rounding is the final one.  Layout: 16 lanes per candidate; each
// lane owns 16-byte chunks of the int8 row (lane sub, sub+16, ...), so a
// group's loads cover the row in one pass.  The request's user slice is held
// in fp64 registers and its sum computed once per group.  A group scores
// eight candidates: one vector load fetches their row indices (one per lane),
// then all their row loads are issued before any is used, and each batch of
// four partial sums is combined across the 16 lanes by halving, which leaves
// every candidate's total in the lane that loaded its scale and bias.
//
// Where a candidate's row comes from is a template parameter: a row array
// (gather_dequant_score, after a lookup-only MPZCH call), or the MPZCH probe
// itself (mpzch_score: the lane that owns a candidate reads the ID's bucket of
// the identity tensor and takes the slot holding the ID, the lookup-only rule
// of mpzch_lookup_or_insert), which saves the lookup's own launch and its
// row array's round trip through memory.
//
// A block scores PASSES groups of candidates one after another, with every
// pass's row found first: each candidate is a chain of dependent memory trips
// (ID, bucket, row), and the later passes' ID and bucket trips run while the
// first pass's rows are fetched and scored.  For 8-slot buckets and a
// power-of-two bucket count the probe is branch-free (ProbeIn8), so the
// passes' probes are in flight together (with a branch per probe the
// compiler waits for each one before the next).
#include "hlr_common.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;
constexpr int kCandsPerBlock = 64;

// Candidate rows from a row array.
struct RowsIn {
  const int64_t *rows;
  __device__ __forceinline__ int64_t row(int64_t i, bool) const { return rows[i]; }
  __device__ __forceinline__ void record(int64_t, int64_t) const {}
};

// Candidate rows from the identity tensor (lookup only): bucket mix64(id) mod
// nb, slots bucket * probes + j; the slot holding the ID, or -1.  An ID of -1
// (the empty marker) never has a row.  The owning lane may record the row and
// the hit flag.
struct ProbeIn {
  const int64_t *ids;
  const int64_t *identity;
  uint64_t nb;
  bool pow2;
  int probes;
  int64_t *out_rows;
  int8_t *out_hit;
  __device__ __forceinline__ int64_t row(int64_t i, bool own) const {
    const int64_t id = ids[i];
    const uint64_t h = mix64(static_cast<uint64_t>(id));
    const uint64_t b = pow2 ? (h & (nb - 1)) : (h % nb);
    const int64_t base = static_cast<int64_t>(b) * probes;
    int64_t r = -1;
    if (probes == 8) {  // the bucket as four 16-byte loads (identity 16-byte aligned)
      const longlong2 *q = reinterpret_cast<const longlong2 *>(identity + base);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const longlong2 v = q[j];
        if (v.x == id) r = base + 2 * j;
        if (v.y == id) r = base + 2 * j + 1;
      }
    } else {
      for (int j = 0; j < probes; ++j)
        if (identity[base + j] == id) r = base + j;
    }
    if (id == HLR_EMPTY_ID) r = -1;
    if (own) record(i, r);
    return r;
  }
  __device__ __forceinline__ void record(int64_t i, int64_t r) const {
    if (out_rows) out_rows[i] = r;
    if (out_hit) out_hit[i] = r >= 0 ? 1 : 0;
  }
};

// The same lookup for 8-slot buckets and a power-of-two bucket count, branch
// free (the slot found by selects), so the probes of several passes can be in
// flight together.
struct ProbeIn8 {
  const int64_t *ids;
  const int64_t *identity;
  uint64_t nb;
  int64_t *out_rows;
  int8_t *out_hit;
  __device__ __forceinline__ int64_t row(int64_t i, bool own) const {
    const int64_t id = ids[i];
    const int64_t base = static_cast<int64_t>(mix64(static_cast<uint64_t>(id)) & (nb - 1)) * 8;
    const longlong2 *q = reinterpret_cast<const longlong2 *>(identity + base);
    longlong2 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = q[j];
    int64_t r = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r = v[j].x == id ? base + 2 * j : r;
      r = v[j].y == id ? base + 2 * j + 1 : r;
    }
    r = id == HLR_EMPTY_ID ? -1 : r;
    if (own) record(i, r);
    return r;
  }
  __device__ __forceinline__ void record(int64_t i, int64_t r) const {
    if (out_rows) out_rows[i] = r;
    if (out_hit) out_hit[i] = r >= 0 ? 1 : 0;
  }
};

__device__ __forceinline__ double dot16(const int4 v, const double *u, double s, double b, double acc) {
  const int w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qi = static_cast<int>(static_cast<int8_t>((w[k] >> (8 * e)) & 0xff));
      const double x = __fma_rn(static_cast<double>(qi), s, b);
      acc = __fma_rn(x, u[4 * k + e], acc);
    }
  }
  return acc;
}

// sum of q_e * u_e over a 16-byte chunk, fp64 (each product exact)
__device__ __forceinline__ double qdot16(const int4 v, const double *u, double acc) {
  const int w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qi = static_cast<int>(static_cast<int8_t>((w[k] >> (8 * e)) & 0xff));
      acc = __fma_rn(static_cast<double>(qi), u[4 * k + e], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ double group16_sum(double x) {
  x += __shfl_xor(x, 8, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 1, 16);
  return x;
}

constexpr int kGroups = kThreads / 16;

// Sums four per-lane partials a[0..3] over a 16-lane group by halving: lane
// sub ends up with the full sum of candidate sub >> 2.
__device__ __forceinline__ double group16_scatter4(double a0, double a1, double a2, double a3, int sub) {
  const bool h8 = sub & 8, h4 = sub & 4;
  double k0 = h8 ? a2 : a0, k1 = h8 ? a3 : a1;
  const double s0 = h8 ? a0 : a2, s1 = h8 ? a1 : a3;
  k0 += __shfl_xor(s0, 8, 16);
  k1 += __shfl_xor(s1, 8, 16);
  double k = h4 ? k1 : k0;
  k += __shfl_xor(h4 ? k0 : k1, 4, 16);
  k += __shfl_xor(k, 2, 16);
  k += __shfl_xor(k, 1, 16);
  return k;
}

// CPL 16-byte chunks per lane held in registers: dim = 256 * CPL.  A group
// scores 4*NB consecutive candidates in NB batches of four.  Lane sub owns
// candidate 4*(sub & 3) + (sub >> 2) of the group: it loads that candidate's
// row index, scale and bias, and is the lane that holds the candidate's full
// sum after the halving reduction of batch sub & 3.
template <int CPL, int NB, int PASSES, typename Src>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
    score_kernel(const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
                 int64_t num_rows, int64_t dim, Src src, int64_t cands, const float *__restrict__ user,
                 float *__restrict__ out) {
  constexpr int J = 4 * NB;
  const int64_t req = blockIdx.y;
  const int grp = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  const int kb = sub & 3, kt = sub >> 2;
  // Every pass's row first: the ID and bucket trips of the later passes run
  // while the earlier passes' rows are fetched and scored.
  int64_t cp[PASSES], rp[PASSES];
  bool ownp[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    cp[p] = (static_cast<int64_t>(blockIdx.x) * PASSES + p) * (kGroups * J) + grp * J + 4 * kb + kt;
    ownp[p] = kb < NB && cp[p] < cands;
    rp[p] = src.row(req * cands + (cp[p] < cands ? cp[p] : cands - 1), false);
  }
  // the lookup's outputs after every probe (a store here would hold the next
  // pass's loads behind it: the outputs may alias the inputs)
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
    if (ownp[p]) src.record(req * cands + cp[p], rp[p]);
  const float *u = user + req * dim;
  double ud[CPL][16];
  double usum = 0.0;
#pragma unroll
  for (int m = 0; m < CPL; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      ud[m][e] = static_cast<double>(u[(sub + 16 * m) * 16 + e]);
      usum += ud[m][e];
    }
  const double U = group16_sum(usum);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t c = cp[p];
    const bool own = ownp[p];
    const int64_t r = rp[p];
    const bool ok = own && r >= 0 && r < num_rows;
    const int64_t myrow = ok ? r : 0;
    const double sc = static_cast<double>(scale[myrow]);
    const double bi = static_cast<double>(bias[myrow]);
    int4 v[NB][4][CPL];
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t rr = __shfl(myrow, 4 * t + k, 16);
#pragma unroll
        for (int m = 0; m < CPL; ++m)
          v[k][t][m] = *reinterpret_cast<const int4 *>(q + rr * dim + (sub + 16 * m) * 16);
      }
    double res = 0.0;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      double a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = 0.0;
#pragma unroll
        for (int m = 0; m < CPL; ++m) a[t] = qdot16(v[k][t][m], ud[m], a[t]);
      }
      const double A = group16_scatter4(a[0], a[1], a[2], a[3], sub);
      if (kb == k) res = __fma_rn(sc, A, bi * U);
    }
    if (own) out[req * cands + c] = ok ? static_cast<float>(res) : 0.0f;
  }
}

// Any dim % 16 == 0: chunks walked in a loop, dequantise-then-dot.
template <typename Src>
__global__ void __launch_bounds__(kThreads)
    score_kernel_any(const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
                     int64_t num_rows, int64_t dim, Src src, int64_t cands, const float *__restrict__ user,
                     float *__restrict__ out) {
  const int64_t req = blockIdx.y;
  const int grp = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  const float *u = user + req * dim;
  const int64_t nchunk = dim >> 4;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kCandsPerBlock;
  const int64_t c1 = c0 + kCandsPerBlock < cands ? c0 + kCandsPerBlock : cands;
  for (int64_t c = c0 + grp; c < c1; c += kGroups) {
    const int64_t row = src.row(req * cands + c, sub == 0);
    const bool ok = row >= 0 && row < num_rows;
    double acc = 0.0;
    if (ok) {
      const double s = static_cast<double>(scale[row]);
      const double b = static_cast<double>(bias[row]);
      const int8_t *qr = q + row * dim;
      for (int64_t ch = sub; ch < nchunk; ch += 16) {
        const int4 v = *reinterpret_cast<const int4 *>(qr + ch * 16);
        double uu[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) uu[e] = static_cast<double>(u[ch * 16 + e]);
        acc = dot16(v, uu, s, b, acc);
      }
    }
    acc = group16_sum(acc);
    if (sub == 0) out[req * cands + c] = ok ? static_cast<float>(acc) : 0.0f;
  }
}

// Checks and launches shared by both entry points: src gives each candidate's row.
template <typename Src>
hlr_status score_launch(const int8_t *qtable, const float *scale, const float *bias, int64_t num_rows, int64_t dim,
                        Src src, int64_t num_requests, int64_t cands_per_request, const float *user_vecs,
                        float *out_scores, hipStream_t stream) {
  auto launch = [&](auto kern, int per_block) {
    dim3 grid(static_cast<unsigned>((cands_per_request + per_block - 1) / per_block),
              static_cast<unsigned>(num_requests));
    kern<<<grid, kThreads, 0, stream>>>(qtable, scale, bias, num_rows, dim, src, cands_per_request, user_vecs,
                                        out_scores);
  };
  // Two batches of four candidates per group: enough loads in flight to
  // cover the row fetches, registers for four waves per SIMD.
  if (dim == 256) launch(score_kernel<1, 2, 2, Src>, kGroups * 8 * 2);
  else if (dim == 512) launch(score_kernel<2, 2, 2, Src>, kGroups * 8 * 2);
  else launch(score_kernel_any<Src>, kCandsPerBlock);
  return launch_status();
}

hlr_status score_args(const int8_t *qtable, const float *scale, const float *bias, int64_t num_rows, int64_t dim,
                      int64_t num_requests, int64_t cands_per_request, const float *user_vecs, float *out_scores) {
  if (num_rows < 0 || num_requests < 0 || cands_per_request < 0 || num_requests > 65535) return HLR_INVALID_ARG;
  if (num_requests * cands_per_request > kMaxN) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 16 != 0) return HLR_UNSUPPORTED_DIM;
  if (num_requests == 0 || cands_per_request == 0) return HLR_OK;
  if (!user_vecs || !out_scores || (num_rows > 0 && (!qtable || !scale || !bias))) return HLR_INVALID_ARG;
  if ((qtable && !aligned(qtable, 16)) || !aligned(user_vecs, 4) || !aligned(out_scores, 4) ||
      (scale && !aligned(scale, 4)) || (bias && !aligned(bias, 4)))
    return HLR_MISALIGNED;
  return HLR_OK;
}

}  // namespace

extern "C" hlr_status gather_dequant_score(const int8_t *qtable, const float *scale, const float *bias,
                                           int64_t num_rows, int64_t dim, const int64_t *rows, int64_t num_requests,
                                           int64_t cands_per_request, const float *user_vecs, float *out_scores,
                                           hipStream_t stream) {
  hlr_status st = score_args(qtable, scale, bias, num_rows, dim, num_requests, cands_per_request, user_vecs,
                             out_scores);
  if (st != HLR_OK || num_requests == 0 || cands_per_request == 0) return st;
  if (!rows) return HLR_INVALID_ARG;
  if (!aligned(rows, 8)) return HLR_MISALIGNED;
  if (num_rows == 0) {  // every candidate misses (and the kernels' clamped loads would have no row 0)
    hlr_fill(out_scores, num_requests * cands_per_request, 0.0f, stream);
    return launch_status();
  }
  return score_launch(qtable, scale, bias, num_rows, dim, RowsIn{rows}, num_requests, cands_per_request, user_vecs,
                      out_scores, stream);
}

extern "C" hlr_status mpzch_score(const int64_t *identity, int64_t capacity, int32_t probes, const int64_t *ids,
                                  const int8_t *qtable, const float *scale, const float *bias, int64_t dim,
                                  int64_t num_requests, int64_t cands_per_request, const float *user_vecs,
                                  float *out_scores, int64_t *out_rows, int8_t *out_hit, hipStream_t stream) {
  if (capacity <= 0 || probes < 1 || probes > 32 || capacity % probes != 0) return HLR_INVALID_ARG;
  hlr_status st = score_args(qtable, scale, bias, capacity, dim, num_requests, cands_per_request, user_vecs,
                             out_scores);
  if (st != HLR_OK || num_requests == 0 || cands_per_request == 0) return st;
  if (!identity || !ids || !qtable) return HLR_INVALID_ARG;
  if (!aligned(identity, probes == 8 ? 16 : 8) || !aligned(ids, 8) || (out_rows && !aligned(out_rows, 8)))
    return HLR_MISALIGNED;
  const uint64_t nb = static_cast<uint64_t>(capacity / probes);
  const bool pow2 = (nb & (nb - 1)) == 0;
  if (probes == 8 && pow2)
    return score_launch(qtable, scale, bias, capacity, dim, ProbeIn8{ids, identity, nb, out_rows, out_hit},
                        num_requests, cands_per_request, user_vecs, out_scores, stream);
  const ProbeIn src{ids, identity, nb, pow2, probes, out_rows, out_hit};
  return score_launch(qtable, scale, bias, capacity, dim, src, num_requests, cands_per_request, user_vecs,
                      out_scores, stream);
}
