// Clip-aware joint Top-K of SparSTAR (review sections "What carries the
// argument" and "Core claim"): per (batch, head, query block) keep the forced
// prefix blocks and the k highest-scoring eligible key blocks; write only the
// forward index list (ascending) and its length.
//
// One wavefront per row.  Scores become order-preserving uint32 keys
// (NaN lowest, -0 == +0, forced and out-of-range slots 0).  The k-th largest
// key T is found by a 32-step bisection on the key bits, each step counting
// keys >= candidate with ballots.  Blocks with key > T are kept, and of the
// blocks with key == T the lowest-indexed (k - #greater) are kept, which is
// exactly "ties go to the lower block index".  The index list is then written
// in ascending order with a ballot prefix sum.
#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 1u;  // NaN: below every number
  if (u == 0x80000000u) u = 0u;                     // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // >= 0x007fffff for non-NaN
}

__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// C > 0: the row lives in registers (C keys per lane, nkb <= 64*C).
// C == 0: the row is re-read from memory on every pass (any nkb).
template <int C>
__global__ __launch_bounds__(64 * kWaves) void select_kernel(const float* __restrict__ S,
                                                             int64_t rows, int nkb, int nf,
                                                             int k, int32_t* __restrict__ cnt,
                                                             int32_t* __restrict__ idx,
                                                             int max_kept) {
  const int lane = threadIdx.x % 64;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / 64;
  if (row >= rows) return;  // uniform per wave
  const float* s = S + row * nkb;

  auto key_at = [&](int j) -> uint32_t {
    return (j >= nf && j < nkb) ? order_key(s[j]) : 0u;
  };
  constexpr int CR = C > 0 ? C : 1;
  uint32_t key[CR];
  if constexpr (C > 0) {
#pragma unroll
    for (int c = 0; c < C; ++c) key[c] = key_at(lane + 64 * c);
  }
  auto count_ge = [&](uint32_t cand) -> int {
    int n = 0;
    if constexpr (C > 0) {
#pragma unroll
      for (int c = 0; c < C; ++c) n += wave_count(key[c] >= cand);
    } else {
      for (int j0 = 0; j0 < nkb; j0 += 64) n += wave_count(key_at(j0 + lane) >= cand);
    }
    return n;
  };

  // T = k-th largest eligible key (all eligible keys are >= 1, so T >= 1).
  uint32_t T = 0xffffffffu;
  int need = 0;
  if (k > 0) {
    T = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = T | (1u << b);
      if (count_ge(cand) >= k) T = cand;
    }
    need = k - (T == 0xffffffffu ? 0 : count_ge(T + 1));
  }

  int32_t* out = idx + row * static_cast<int64_t>(max_kept);
  for (int p = lane; p < nf; p += 64) out[p] = p;
  int base = nf, eq_seen = 0;
  const uint64_t lt = lanemask_lt(lane);
  auto emit = [&](uint32_t kk, int j) {
    const bool eq = (k > 0) && (kk == T);
    const uint64_t eqm = __ballot(eq);
    const bool take = (k > 0) && (kk > T || (eq && eq_seen + __popcll(eqm & lt) < need));
    eq_seen += __popcll(eqm);
    const uint64_t tm = __ballot(take);
    const int pos = base + __popcll(tm & lt);
    if (take && pos < max_kept) out[pos] = j;
    base += __popcll(tm);
  };
  if constexpr (C > 0) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (64 * c >= nkb) break;
      emit(key[c], lane + 64 * c);
    }
  } else {
    for (int j0 = 0; j0 < nkb; j0 += 64) emit(key_at(j0 + lane), j0 + lane);
  }
  for (int p = base + lane; p < max_kept; p += 64) out[p] = -1;
  if (lane == 0) cnt[row] = base;
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
#define SPARSTAR_SELECT(CC) select_kernel<CC><<<grid, block, 0, s>>>(S, rows, n, f, kk, kv_count, kv_index, mk)
  // keys per lane = ceil(nkb / 64), rounded up to an instantiated count
  const int64_t c = (nkb + 63) / 64;
  if (c <= 1) SPARSTAR_SELECT(1);
  else if (c <= 2) SPARSTAR_SELECT(2);
  else if (c <= 3) SPARSTAR_SELECT(3);
  else if (c <= 4) SPARSTAR_SELECT(4);
  else if (c <= 6) SPARSTAR_SELECT(6);
  else if (c <= 8) SPARSTAR_SELECT(8);
  else if (c <= 10) SPARSTAR_SELECT(10);
  else if (c <= 12) SPARSTAR_SELECT(12);
  else if (c <= 14) SPARSTAR_SELECT(14);
  else if (c <= 16) SPARSTAR_SELECT(16);
  else if (c <= 18) SPARSTAR_SELECT(18);
  else if (c <= 20) SPARSTAR_SELECT(20);
  else if (c <= 24) SPARSTAR_SELECT(24);
  else if (c <= 28) SPARSTAR_SELECT(28);
  else if (c <= 32) SPARSTAR_SELECT(32);
  else SPARSTAR_SELECT(0);
#undef SPARSTAR_SELECT
  return check_launch("sparstar_select_blocks");
}

}  // namespace sparstar
