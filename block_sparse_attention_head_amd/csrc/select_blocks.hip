// Clip-aware joint Top-K of SparSTAR (review sections "What carries the
// argument" and "Core claim") from a materialised score matrix: per (batch,
// head, query block) keep the forced prefix blocks and the k highest-scoring
// eligible key blocks; write only the forward index list (ascending) and its
// length.  One wavefront per row; the row selection itself is select_row
// (select_row.hpp).
#include "select_row.hpp"

namespace sparstar {
namespace {

constexpr int kWaves = 4;

// C > 0: the row lives in registers (C keys per lane, nkb <= 64*C).
// C == 0: the row is re-read from memory on every pass (any nkb).
template <int C>
__global__ __launch_bounds__(64 * kWaves) void select_kernel(const float* __restrict__ S,
                                                             int64_t rows, int nkb, int nf,
                                                             int k, int32_t* __restrict__ cnt,
                                                             int32_t* __restrict__ idx,
                                                             int max_kept) {
  __shared__ uint32_t cand_lds[kWaves][128];
  const int lane = threadIdx.x % 64;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / 64;
  if (row >= rows) return;  // uniform per wave; no workgroup barrier below
  const float* s = S + row * nkb;

  auto key_at = [&](int j) -> uint32_t {
    return (j >= nf && j < nkb) ? order_key(s[j]) : 0u;
  };
  constexpr int CR = C > 0 ? C : 1;
  uint32_t key[CR];
  if constexpr (C > 0) {
    // All C loads are issued before any is used (clamped, so every one is in
    // bounds); loads under per-key branches would each wait out the latency.
    float v[C];
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = s[min(lane + 64 * c, nkb - 1)];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = lane + 64 * c;
      key[c] = static_cast<unsigned>(j - nf) < static_cast<unsigned>(nkb - nf) ? order_key(v[c]) : 0u;
    }
  }
  const int n = select_row<C>(key, key_at, lane, nkb, nf, k, cand_lds[threadIdx.x / 64],
                              idx + row * static_cast<int64_t>(max_kept), max_kept);
  if (lane == 0) cnt[row] = n;
}

}  // namespace

sparstar_status launch_select_blocks(const float* S, int64_t rows, int64_t nkb, int64_t n_forced,
                                     int64_t k, int32_t* kv_count, int32_t* kv_index,
                                     int64_t max_kept, hipStream_t s) {
  const int64_t wgs = (rows + kWaves - 1) / kWaves;
  if (wgs > 2147483647LL) {
    set_error("sparstar_select_blocks: too many rows");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  const dim3 grid(static_cast<uint32_t>(wgs)), block(64 * kWaves);
  const int n = (int)nkb, f = (int)n_forced, kk = (int)k, mk = (int)max_kept;
  switch (keys_per_lane(nkb)) {
#define SPARSTAR_SELECT_CASE(CC) \
  case CC: select_kernel<CC><<<grid, block, 0, s>>>(S, rows, n, f, kk, kv_count, kv_index, mk); break;
    SPARSTAR_FOR_EACH_C(SPARSTAR_SELECT_CASE)
    SPARSTAR_FOR_EACH_C_LARGE(SPARSTAR_SELECT_CASE)
#undef SPARSTAR_SELECT_CASE
    default: select_kernel<0><<<grid, block, 0, s>>>(S, rows, n, f, kk, kv_count, kv_index, mk);
  }
  return check_launch("sparstar_select_blocks");
}

}  // namespace sparstar
