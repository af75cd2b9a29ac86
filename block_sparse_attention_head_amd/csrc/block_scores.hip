// Aggregated block scores, Eq. 2 of SparSTAR (review section "What carries
// the argument"): S_ij = tau * qbar_i . kbar_j, per (batch, head).
//
// The selector ranks these scores, and an exact tie rule only means something
// if the GPU and a float64 reference agree on the order of nearly equal
// scores.  Products of two float32 means are exact in float64, so the dot
// product is accumulated in float64 on the fp64 matrix cores
// (score_tile.hpp) and rounded once to float32.
//
// Tiling: a one-wavefront workgroup owns 16 q rows (their operands stay in
// registers) and walks a run of 16-column k tiles two at a time, so two
// independent accumulation chains keep the matrix core busy.
#include "score_tile.hpp"

namespace sparstar {
namespace {

constexpr int kRowsPerWave = 16;
constexpr int kColTilesPerWave = 16;   // 256 columns per wavefront

template <int D>
__global__ __launch_bounds__(64) void block_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb,
    int strips_q, int runs_k, double tau, float* __restrict__ S) {
  const int64_t wg = blockIdx.x;
  const int64_t per_head = static_cast<int64_t>(strips_q) * runs_k;
  const int64_t bh = wg / per_head;
  const int rem = static_cast<int>(wg - bh * per_head);
  const int l = threadIdx.x;
  const int i0 = (rem / runs_k) * kRowsPerWave;
  const int jt0 = (rem % runs_k) * kColTilesPerWave;
  const int ntk = (nkb + 15) / 16;
  const int jt1 = min(ntk, jt0 + kColTilesPerWave);
  const int lr = l % 16, ls = l / 16;

  const float* qh = qbar + bh * static_cast<int64_t>(nqb) * D;
  const float* kh = kbar + bh * static_cast<int64_t>(nkb) * D;
  float* Sh = S + bh * static_cast<int64_t>(nqb) * nkb;
  f32x4 qv[D / 16];
  {
    const int iq = i0 + lr;   // rows past the edge read row 0 and are not stored
    load_operands<D>(qh + static_cast<int64_t>(iq < nqb ? iq : 0) * D + 4 * ls, qv);
  }
  auto krow = [&](int jt) {
    const int jk = 16 * jt + lr;   // columns past the edge read row 0 and are not stored
    return kh + static_cast<int64_t>(jk < nkb ? jk : 0) * D + 4 * ls;
  };
  auto store = [&](const f64x4& acc, int jt) {
    // acc[r] = S(i0 + ls + 4r, 16 jt + lr)
    const int jk = 16 * jt + lr;
    if (jk < nkb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + ls + 4 * r;
        if (i < nqb) Sh[static_cast<int64_t>(i) * nkb + jk] = static_cast<float>(tau * acc[r]);
      }
    }
  };
  for (int jt = jt0; jt < jt1; jt += 2) {
    f32x4 ka[D / 16], kb[D / 16];
    load_operands<D>(krow(jt), ka);
    load_operands<D>(krow(jt + 1 < jt1 ? jt + 1 : jt), kb);
    f64x4 a0, a1;
    score_tiles16x2<D>(qv, ka, kb, a0, a1);
    store(a0, jt);
    if (jt + 1 < jt1) store(a1, jt + 1);
  }
}

}  // namespace

sparstar_status launch_block_scores(const float* qbar, const float* kbar, int64_t BH,
                                    int64_t nqb, int64_t nkb, int64_t D, float tau, float* S,
                                    hipStream_t s) {
  const int64_t strips = (nqb + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t runs = ((nkb + 15) / 16 + kColTilesPerWave - 1) / kColTilesPerWave;
  if (BH * strips * runs > 2147483647LL) {
    set_error("sparstar_block_scores: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  const dim3 grid(static_cast<uint32_t>(BH * strips * runs)), block(64);
  if (D == 128)
    block_scores_kernel<128><<<grid, block, 0, s>>>(qbar, kbar, (int)nqb, (int)nkb, (int)strips,
                                                    (int)runs, (double)tau, S);
  else
    block_scores_kernel<64><<<grid, block, 0, s>>>(qbar, kbar, (int)nqb, (int)nkb, (int)strips,
                                                   (int)runs, (double)tau, S);
  return check_launch("sparstar_block_scores");
}

}  // namespace sparstar
