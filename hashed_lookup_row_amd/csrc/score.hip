// Serving score: int8 row dequantisation fused with a dot product against the
// request's user vector.  "Memory Layer: Train the In-Model Cache for
// Recommendation Models": sec. 1 (early-stage ranking scores about a thousand
// candidates per request), sec. 5 (the serving side reads int8-quantised rows),
// sec. 2 (a miss zeroes the cached branch: score 0).
//
// Layout: 16 lanes per candidate (one wave scores 4 candidates at a time); each
// lane owns 16-byte chunks of the int8 row (lane sub, sub+16, ...), so a
// group's loads cover the 512-byte row in one pass.  The request's user slice
// is converted to fp64 once per lane and kept in registers.  Dequantisation
// x = q*scale + bias is one fp64 FMA (q*scale is exact in fp64) and the dot
// accumulates in fp64, so the only fp32 rounding is the final one; lanes are
// combined with a 4-step xor-shuffle tree.
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

// CPL: 16-byte chunks per lane held in registers (dim = 256*CPL); 0 = any dim % 16 == 0.
template <int CPL>
__global__ void __launch_bounds__(kThreads)
    score_kernel(const int8_t *__restrict__ q, const float *__restrict__ scale, const float *__restrict__ bias,
                 int64_t num_rows, int64_t dim, const int64_t *__restrict__ rows, int64_t cands,
                 const float *__restrict__ user, float *__restrict__ out) {
  const int64_t req = blockIdx.y;
  const int grp = threadIdx.x >> 4;
  const int sub = threadIdx.x & 15;
  const float *u = user + req * dim;
  const int64_t nchunk = dim >> 4;
  constexpr int CR = CPL > 0 ? CPL : 1;
  double ud[CR][16];
  if (CPL > 0) {
#pragma unroll
    for (int m = 0; m < CR; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) ud[m][e] = static_cast<double>(u[(sub + 16 * m) * 16 + e]);
  }
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kCandsPerBlock;
  const int64_t c1 = c0 + kCandsPerBlock < cands ? c0 + kCandsPerBlock : cands;
  for (int64_t c = c0 + grp; c < c1; c += kThreads / 16) {
    const int64_t row = rows[req * cands + c];
    const bool ok = row >= 0 && row < num_rows;
    double acc = 0.0;
    if (ok) {
      const double s = static_cast<double>(scale[row]);
      const double b = static_cast<double>(bias[row]);
      const int8_t *qr = q + row * dim;
      if (CPL > 0) {
        int4 v[CR];
#pragma unroll
        for (int m = 0; m < CR; ++m) v[m] = *reinterpret_cast<const int4 *>(qr + (sub + 16 * m) * 16);
#pragma unroll
        for (int m = 0; m < CR; ++m) acc = dot16(v[m], ud[m], s, b, acc);
      } else {
        for (int64_t ch = sub; ch < nchunk; ch += 16) {
          const int4 v = *reinterpret_cast<const int4 *>(qr + ch * 16);
          double uu[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) uu[e] = static_cast<double>(u[ch * 16 + e]);
          acc = dot16(v, uu, s, b, acc);
        }
      }
    }
    acc += __shfl_xor(acc, 8, 16);
    acc += __shfl_xor(acc, 4, 16);
    acc += __shfl_xor(acc, 2, 16);
    acc += __shfl_xor(acc, 1, 16);
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
  dim3 grid(static_cast<unsigned>((cands_per_request + kCandsPerBlock - 1) / kCandsPerBlock),
            static_cast<unsigned>(num_requests));
  switch (dim) {
    case 256: score_kernel<1><<<grid, kThreads, 0, stream>>>(qtable, scale, bias, num_rows, dim, rows,
                                                             cands_per_request, user_vecs, out_scores); break;
    case 512: score_kernel<2><<<grid, kThreads, 0, stream>>>(qtable, scale, bias, num_rows, dim, rows,
                                                             cands_per_request, user_vecs, out_scores); break;
    default: score_kernel<0><<<grid, kThreads, 0, stream>>>(qtable, scale, bias, num_rows, dim, rows,
                                                            cands_per_request, user_vecs, out_scores); break;
  }
  return launch_status();
}
