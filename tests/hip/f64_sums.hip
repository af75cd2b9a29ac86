// Test helper (not part of the library): the library's two fp64 matrix-core
// forms of the score sums, score_tile16 (16 x 16 tile) and score_row16 (one
// row against 16 columns), run on the same operands, so that a test can
// require the same bits from both.  Built beside the tests by
// tests/hip/build_helpers.py.
#include "../../block_sparse_attention_head_amd/csrc/score_tile.hpp"

namespace {

using sparstar::f32x4;
using sparstar::f64x4;

// One wave per case t: Q[t] and K[t] are 16 x D float rows.
// tile[t][i][j] = score_tile16 sum of (Q row i, K row j);
// row[t][i][j]  = score_row16 sum of (Q row i, K row j), for every i.
template <int D>
__global__ __launch_bounds__(64) void sums_kernel(const float* __restrict__ Q,
                                                  const float* __restrict__ K, double* tile,
                                                  double* row) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x, lr = lane % 16, lg = lane / 16;
  const float* q = Q + t * 16 * D;
  const float* k = K + t * 16 * D;
  f32x4 kv[D / 16];
  sparstar::load_operands<D>(k + lr * D + 4 * lg, kv);
  {
    f32x4 qv[D / 16];
    sparstar::load_operands<D>(q + lr * D + 4 * lg, qv);
    const f64x4 acc = sparstar::score_tile16<D>(qv, kv);
#pragma unroll
    for (int r = 0; r < 4; ++r) tile[(t * 16 + lg + 4 * r) * 16 + lr] = acc[r];
  }
  for (int i = 0; i < 16; ++i) {
    f32x4 qv[D / 16];
    sparstar::load_operands<D>(q + i * D + 4 * lg, qv);
    const double acc = sparstar::score_row16<D>(qv, kv);
    if (lane < 16) row[(t * 16 + i) * 16 + lane] = acc;
  }
}

}  // namespace

// Q, K: device float [cases][16][D]; tile, row: device double [cases][16][16].
// D is 64 or 128.  Returns 0, or the HIP error code of the launch.
extern "C" int f64_sums_run(const float* Q, const float* K, int cases, int D, double* tile,
                            double* row, void* stream) {
  if (cases <= 0 || (D != 64 && D != 128)) return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) sums_kernel<128><<<cases, 64, 0, s>>>(Q, K, tile, row);
  else sums_kernel<64><<<cases, 64, 0, s>>>(Q, K, tile, row);
  return static_cast<int>(hipGetLastError());
}
