// Aggregated block scores, Eq. 2 of SparSTAR (review section "What carries
// the argument"): S_ij = tau * qbar_i . kbar_j, per (batch, head).
//
// The selector ranks these scores, and an exact tie rule only means something
// if the GPU and a float64 reference agree on the order of nearly equal
// scores.  Products of two float32 means are exact in float64, so the dot
// product is accumulated in float64 and rounded once to float32.
//
// Tiling: one workgroup computes a 64 x 64 tile of S for one (b, h).  The
// means are staged through LDS in chunks of 32 dimensions, converted to
// float64 on the way in and stored dimension-major so that every thread of a
// row of 16 reads consecutive words.  Each thread owns a 4 x 4 sub-tile
// (rows 4*ty..4*ty+3, columns tx + 16*c), 16 float64 FMAs per 8 LDS reads.
#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kTile = 64;
constexpr int kChunk = 32;
constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void block_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb,
    int tiles_q, int tiles_k, double tau, float* __restrict__ S) {
  __shared__ double qs[kChunk][kTile + 1];
  __shared__ double ks[kChunk][kTile + 1];

  const int64_t wg = blockIdx.x;
  const int64_t per_head = static_cast<int64_t>(tiles_q) * tiles_k;
  const int64_t bh = wg / per_head;
  const int rem = static_cast<int>(wg - bh * per_head);
  const int i0 = (rem / tiles_k) * kTile;
  const int j0 = (rem % tiles_k) * kTile;
  const float* qh = qbar + bh * static_cast<int64_t>(nqb) * D;
  const float* kh = kbar + bh * static_cast<int64_t>(nkb) * D;

  const int t = threadIdx.x;
  const int tx = t % 16, ty = t / 16;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;

  // loader mapping: 64 rows x 32 dims per operand = 512 float4 chunks
  for (int d0 = 0; d0 < D; d0 += kChunk) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ch = t + kThreads * m;      // 0..511
      const int r = ch / (kChunk / 4);      // row in tile
      const int cc = (ch % (kChunk / 4)) * 4;
      f32x4 vq = {0.f, 0.f, 0.f, 0.f}, vk = {0.f, 0.f, 0.f, 0.f};
      if (i0 + r < nqb) vq = *reinterpret_cast<const f32x4*>(qh + (int64_t)(i0 + r) * D + d0 + cc);
      if (j0 + r < nkb) vk = *reinterpret_cast<const f32x4*>(kh + (int64_t)(j0 + r) * D + d0 + cc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qs[cc + e][r] = static_cast<double>(vq[e]);
        ks[cc + e][r] = static_cast<double>(vk[e]);
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int d = 0; d < kChunk; ++d) {
      double qa[4], kc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[a] = qs[d][4 * ty + a];
#pragma unroll
      for (int c = 0; c < 4; ++c) kc[c] = ks[d][tx + 16 * c];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fma(qa[a], kc[c], acc[a][c]);
    }
    __syncthreads();
  }

  float* Sh = S + bh * static_cast<int64_t>(nqb) * nkb;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + 4 * ty + a;
    if (i >= nqb) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tx + 16 * c;
      if (j < nkb) Sh[static_cast<int64_t>(i) * nkb + j] = static_cast<float>(tau * acc[a][c]);
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
  const dim3 grid(static_cast<uint32_t>(BH * tq * tk)), block(kThreads);
  if (D == 128)
    block_scores_kernel<128><<<grid, block, 0, s>>>(qbar, kbar, (int)nqb, (int)nkb, (int)tq,
                                                    (int)tk, (double)tau, S);
  else
    block_scores_kernel<64><<<grid, block, 0, s>>>(qbar, kbar, (int)nqb, (int)nkb, (int)tq,
                                                   (int)tk, (double)tau, S);
  return check_launch("sparstar_block_scores");
}

}  // namespace sparstar
