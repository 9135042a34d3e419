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
#include "hlr_common.hpp"

namespace {
using namespace hlr;

constexpr int kThreads = 256;
constexpr int kCandsPerBlock = 64;

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
template <int CPL, int NB>
__global__ void __launch_bounds__(kThreads)
    score_kernel(const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
                 int64_t num_rows, int64_t dim, const int64_t *__restrict__ rows, int64_t cands,
                 const float *__restrict__ user, float *__restrict__ out) {
  constexpr int J = 4 * NB;
  const int64_t req = blockIdx.y;
  const int grp = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * (kGroups * J) + grp * J;
  const int kb = sub & 3, kt = sub >> 2;
  const int64_t c = c0 + 4 * kb + kt;
  const bool own = kb < NB && c < cands;
  const int64_t r = rows[req * cands + (c < cands ? c : cands - 1)];
  const bool ok = own && r >= 0 && r < num_rows;
  const int64_t myrow = ok ? r : 0;
  const double sc = static_cast<double>(scale[myrow]);
  const double bi = static_cast<double>(bias[myrow]);
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
  int4 v[NB][4][CPL];
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t rr = __shfl(myrow, 4 * t + k, 16);
#pragma unroll
      for (int m = 0; m < CPL; ++m) v[k][t][m] = *reinterpret_cast<const int4 *>(q + rr * dim + (sub + 16 * m) * 16);
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

// Any dim % 16 == 0: chunks walked in a loop, dequantise-then-dot.
__global__ void __launch_bounds__(kThreads)
    score_kernel_any(const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
                     int64_t num_rows, int64_t dim, const int64_t *__restrict__ rows, int64_t cands,
                     const float *__restrict__ user, float *__restrict__ out) {
  const int64_t req = blockIdx.y;
  const int grp = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  const float *u = user + req * dim;
  const int64_t nchunk = dim >> 4;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kCandsPerBlock;
  const int64_t c1 = c0 + kCandsPerBlock < cands ? c0 + kCandsPerBlock : cands;
  for (int64_t c = c0 + grp; c < c1; c += kGroups) {
    const int64_t row = rows[req * cands + c];
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

}  // namespace

extern "C" hlr_status gather_dequant_score(const int8_t *qtable, const float *scale, const float *bias,
                                           int64_t num_rows, int64_t dim, const int64_t *rows, int64_t num_requests,
                                           int64_t cands_per_request, const float *user_vecs, float *out_scores,
                                           hipStream_t stream) {
  if (num_rows < 0 || num_requests < 0 || cands_per_request < 0 || num_requests > 65535) return HLR_INVALID_ARG;
  if (num_requests * cands_per_request > kMaxN) return HLR_INVALID_ARG;
  if (dim <= 0 || dim % 16 != 0) return HLR_UNSUPPORTED_DIM;
  if (num_requests == 0 || cands_per_request == 0) return HLR_OK;
  if (!rows || !user_vecs || !out_scores || (num_rows > 0 && (!qtable || !scale || !bias))) return HLR_INVALID_ARG;
  if ((qtable && !aligned(qtable, 16)) || !aligned(rows, 8) || !aligned(user_vecs, 4) || !aligned(out_scores, 4) ||
      (scale && !aligned(scale, 4)) || (bias && !aligned(bias, 4)))
    return HLR_MISALIGNED;
  if (num_rows == 0) {  // every candidate misses (and the kernels' clamped loads would have no row 0)
    hlr_fill(out_scores, num_requests * cands_per_request, 0.0f, stream);
    return launch_status();
  }
  auto launch = [&](auto kern, int per_block) {
    dim3 grid(static_cast<unsigned>((cands_per_request + per_block - 1) / per_block),
              static_cast<unsigned>(num_requests));
    kern<<<grid, kThreads, 0, stream>>>(qtable, scale, bias, num_rows, dim, rows, cands_per_request, user_vecs,
                                        out_scores);
  };
  // Two batches of four candidates per group: enough loads in flight to
  // cover the row fetches, registers for four waves per SIMD.
  if (dim == 256) launch(score_kernel<1, 2>, kGroups * 8);
  else if (dim == 512) launch(score_kernel<2, 2>, kGroups * 8);
  else launch(score_kernel_any, kCandsPerBlock);
  return launch_status();
}
