// The exact block scores on the fp64 matrix cores, in the forms the kernels
// use: a 16 x 16 tile (score_tile16; the score kernel runs two at once,
// score_tiles16x2) and one row against 16 columns (score_row16, for the band
// selection's exact scores).  All form the same float64 sums with the same
// operations in the same order, so every kernel produces the same float32
// scores bit for bit.
//
// v_mfma_f64_16x16x4f64 lane layout (gfx950): A lane l = (row l % 16,
// k l / 16), B lane l = (k l / 16, column l % 16), result lane l register r =
// (row l / 16 + 4 r, column l % 16).  Each lane reads float4 slices of its
// row of qbar and of kbar: within a 16-dimension chunk c, k-step e uses
// dimension 16 c + 4 (l / 16) + e on both operands.  The float32 means become
// float64 exactly, their products are exact, and the 32 (D = 128) k-steps
// accumulate in float64; the caller rounds tau * sum once to float32.
#pragma once

#include "common.hpp"

namespace sparstar {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Operands of one lane for all D dimensions, from the lane's row of qbar or
// kbar (already offset by 4 * (lane / 16)).  They stay float32 in registers
// (half the registers of float64) and are widened exactly at each product;
// loading is separate from the product so that callers can load the next k
// tile while the current one is on the matrix cores.
template <int D>
__device__ __forceinline__ void load_operands(const float* row, f32x4 (&v)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) v[c] = *reinterpret_cast<const f32x4*>(row + 16 * c);
}

// One tile's float64 sums, accumulated over k-steps in ascending dimension
// order.  The q operands pass through an empty asm so that their widening
// stays inside the caller's tile loop: hoisted out of it, the float64 copies
// would double the registers the q operands hold.
template <int D>
__device__ __forceinline__ f64x4 score_tile16(const f32x4 (&qv)[D / 16], const f32x4 (&kv)[D / 16]) {
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    f32x4 q = qv[c];
    asm volatile("" : "+v"(q));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(q[e]),
                                                 static_cast<double>(kv[c][e]), acc, 0, 0, 0);
  }
  return acc;
}

// Two tiles (k operands ka, kb) against the same q rows: each tile's sums are
// formed exactly as score_tile16 forms them (same operations, same order);
// the two independent chains interleave on the matrix core.
template <int D>
__device__ __forceinline__ void score_tiles16x2(const f32x4 (&qv)[D / 16], const f32x4 (&ka)[D / 16],
                                                const f32x4 (&kb)[D / 16], f64x4& a0, f64x4& a1) {
  a0 = f64x4{0.0, 0.0, 0.0, 0.0};
  a1 = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    f32x4 q = qv[c];
    asm volatile("" : "+v"(q));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double qd = static_cast<double>(q[e]);
      a0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qd, static_cast<double>(ka[c][e]), a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qd, static_cast<double>(kb[c][e]), a1, 0, 0, 0);
    }
  }
}

// One row of q against 16 key columns, for a caller that needs a single row:
// v_mfma_f64_4x4x4f64 (four blocks of 4 x 4, K = 4) spends a quarter of the
// matrix-core cycles of a 16 x 16 tile on it.  Lane layout (gfx950): A lane
// i + 4 b + 16 k = (row i, k) of block b, B lane j + 4 b + 16 k = (k, column
// j) of block b, result lane j + 4 b + 16 i = (row i, column j) of block b.
// Every lane passes the same row's slices (qv from the row, offset by
// 4 * (lane / 16) as for score_tile16) and kv from key column 4 b + j =
// lane % 16, so block b holds columns 4 b .. 4 b + 3 in all four rows and
// lane c < 16 receives the sum for column c.  The dimension groups and their
// order are score_tile16's (k-step e of chunk c: dimension 16 c + 4 k + e);
// each step adds a four-product group to the running float64 sum, and the
// two instructions give the same bits for it (checked by a GPU test on
// random, cancelling and wide-range operands).
template <int D>
__device__ __forceinline__ double score_row16(const f32x4 (&qv)[D / 16], const f32x4 (&kv)[D / 16]) {
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    f32x4 q = qv[c];
    asm volatile("" : "+v"(q));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f64_4x4x4f64(static_cast<double>(q[e]),
                                               static_cast<double>(kv[c][e]), acc, 0, 0, 0);
  }
  return acc;
}

}  // namespace sparstar
