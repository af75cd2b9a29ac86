// Aggregated block scores, Eq. 2 of SparSTAR (review section "What carries
// the argument"): S_ij = tau * qbar_i . kbar_j, per (batch, head).
//
// The selector ranks these scores, and an exact tie rule only means something
// if the GPU and a float64 reference agree on the order of nearly equal
// scores.  Products of two float32 means are exact in float64, so the dot
// product is accumulated in float64 (on the fp64 matrix cores,
// v_mfma_f64_16x16x4f64) and rounded once to float32.
//
// Tiling: one wavefront computes a 64 x 64 tile of S for one (b, h) as 4 x 4
// MFMA tiles of 16 x 16.  Each lane streams float4 slices of its rows of
// qbar and kbar straight from memory (the means are small and L2 resident),
// converts them to float64 and feeds four k-steps from each slice: within a
// 16-dimension chunk, MFMA k-slot s of k-step e is dimension 4*s + e, the
// same on both operands.
#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kTile = 64;

typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(64) void block_scores_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar,
                                                          int nqb, int nkb, int tiles_q,
                                                          int tiles_k, double tau,
                                                          float* __restrict__ S) {
  const int64_t wg = blockIdx.x;
  const int64_t per_head = static_cast<int64_t>(tiles_q) * tiles_k;
  const int64_t bh = wg / per_head;
  const int rem = static_cast<int>(wg - bh * per_head);
  const int i0 = (rem / tiles_k) * kTile;
  const int j0 = (rem % tiles_k) * kTile;
  const float* qh = qbar + bh * static_cast<int64_t>(nqb) * D;
  const float* kh = kbar + bh * static_cast<int64_t>(nkb) * D;
  const int l = threadIdx.x;
  const int lr = l % 16, ls = l / 16;

  // rows (or columns) this lane feeds in each of the 4 sub-tiles; rows past
  // the edge read row 0 and are discarded at the store
  const float* qrow[4];
  const float* krow[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int ii = i0 + 16 * a + lr, jj = j0 + 16 * a + lr;
    qrow[a] = qh + static_cast<int64_t>(ii < nqb ? ii : 0) * D + 4 * ls;
    krow[a] = kh + static_cast<int64_t>(jj < nkb ? jj : 0) * D + 4 * ls;
  }

  f64x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};

#pragma unroll 2
  for (int d0 = 0; d0 < D; d0 += 16) {
    f32x4 qv[4], kv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      qv[a] = *reinterpret_cast<const f32x4*>(qrow[a] + d0);
      kv[a] = *reinterpret_cast<const f32x4*>(krow[a] + d0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double qa[4], kb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        qa[a] = static_cast<double>(qv[a][e]);
        kb[a] = static_cast<double>(kv[a][e]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[a], kb[b], acc[a][b], 0, 0, 0);
    }
  }

  // acc[a][b][r] = S(i0 + 16a + ls + 4r, j0 + 16b + lr)
  float* Sh = S + bh * static_cast<int64_t>(nqb) * nkb;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 16 * a + ls + 4 * r;
      if (i >= nqb) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = j0 + 16 * b + lr;
        if (j < nkb) Sh[static_cast<int64_t>(i) * nkb + j] = static_cast<float>(tau * acc[a][b][r]);
      }
    }
}

}  // namespace

sparstar_status launch_block_scores(const float* qbar, const float* kbar, int64_t BH,
                                    int64_t nqb, int64_t nkb, int64_t D, float tau, float* S,
                                    hipStream_t s) {
  const int64_t tq = (nqb + kTile - 1) / kTile, tk = (nkb + kTile - 1) / kTile;
  if (BH * tq * tk > 2147483647LL) {
    set_error("sparstar_block_scores: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  const dim3 grid(static_cast<uint32_t>(BH * tq * tk)), block(64);
  if (D == 128)
    block_scores_kernel<128><<<grid, block, 0, s>>>(qbar, kbar, (int)nqb, (int)nkb, (int)tq,
                                                    (int)tk, (double)tau, S);
  else
    block_scores_kernel<64><<<grid, block, 0, s>>>(qbar, kbar, (int)nqb, (int)nkb, (int)tq,
                                                   (int)tk, (double)tau, S);
  return check_launch("sparstar_block_scores");
}

}  // namespace sparstar
