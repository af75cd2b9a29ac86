// Selection of one row of block scores, shared by the selection kernels:
// clip-aware joint Top-K of SparSTAR (review sections "What carries the
// argument" and "Core claim"): keep the forced prefix blocks and the k
// highest-scoring eligible key blocks, ties to the lower block index, and
// write the forward index list in ascending order.
//
// Scores become order-preserving uint32 keys (NaN lowest, -0 == +0, forced
// and out-of-range slots 0).  The k-th largest key T is found by bisection on
// the key bits, each step counting keys >= candidate with ballots: the first
// kPrefixBits steps on all keys, the rest on the few keys that still share
// T's prefix (packed into LDS).  Blocks with key > T are kept, and of the
// blocks with key == T the lowest-indexed (k - #greater) are kept, which is
// exactly "ties go to the lower block index".  The index list is then written
// in ascending order with a ballot prefix sum.
#pragma once

#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kPrefixBits = 12;   // bisection steps taken on all keys before packing candidates

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

// Selection of one row.  C > 0: the C keys of each lane are in registers
// (slot j = lane + 64 c); C == 0: keys come from key_at(j) on every pass.
// Writes out[0 .. max_kept) and returns the kept count.
template <int C, typename KeyAt>
__device__ __forceinline__ int select_row(const uint32_t* key, KeyAt key_at, int lane, int nkb,
                                          int nf, int k, uint32_t* cbuf, int32_t* out,
                                          int max_kept) {
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

  // T = k-th largest eligible key (all eligible keys are >= 1, so T >= 1);
  // need = how many keys equal to T are kept, n_eq = how many there are.
  uint32_t T = 0xffffffffu;
  int need = 0, n_eq = 0;
  if (k > 0) {
    T = 0;
    int b = 31;
    if constexpr (C > 0) {
      // The first kPrefixBits bits on all keys; then only the keys that share
      // T's prefix ("candidates", in [lo, hi]) can still move the answer: they
      // are packed into LDS (at most two per lane) and the remaining bits are
      // settled on them alone, counting the keys above hi once.
      for (; b >= 32 - kPrefixBits; --b) {
        const uint32_t cand = T | (1u << b);
        if (count_ge(cand) >= k) T = cand;
      }
      const uint32_t lo = T > 1u ? T : 1u;                         // key 0 never counts
      const uint32_t hi = T | ((1u << (32 - kPrefixBits)) - 1u);   // T's low bits are 0
      int above = 0, ncand = 0;
      const uint64_t lt = lanemask_lt(lane);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        above += wave_count(key[c] > hi);
        const bool in = key[c] >= lo && key[c] <= hi;
        const uint64_t m = __ballot(in);
        const int pos = ncand + __popcll(m & lt);
        if (in && pos < 128) cbuf[pos] = key[c];
        ncand += __popcll(m);
      }
      __builtin_amdgcn_wave_barrier();   // this wave's LDS writes precede its reads
      if (ncand <= 128) {
        // empty slots hold 0, below every threshold tried (all >= 1)
        const uint32_t c0 = lane < ncand ? cbuf[lane] : 0u;
        const uint32_t c1 = lane + 64 < ncand ? cbuf[lane + 64] : 0u;
        auto count_cand = [&](uint32_t v) {
          return above + wave_count(c0 >= v) + wave_count(c1 >= v);
        };
        for (; b >= 0; --b) {
          const uint32_t cand = T | (1u << b);
          if (count_cand(cand) >= k) T = cand;
        }
        const int gt = T == 0xffffffffu ? 0 : count_cand(T + 1);
        need = k - gt;
        n_eq = count_cand(T) - gt;
      }
      __builtin_amdgcn_wave_barrier();   // reads done before the buffer is reused
    }
    if (b >= 0) {   // no candidate pass (or too many candidates): finish on all keys
      for (; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        if (count_ge(cand) >= k) T = cand;
      }
      const int gt = T == 0xffffffffu ? 0 : count_ge(T + 1);
      need = k - gt;
      n_eq = count_ge(T) - gt;
    }
  }

  for (int p = lane; p < nf; p += 64) out[p] = p;
  int base = nf;
  if (k > 0) {
    const uint64_t lt = lanemask_lt(lane);
    auto put = [&](bool take, int j) {
      const uint64_t tm = __ballot(take);
      const int pos = base + __popcll(tm & lt);
      if (take && pos < max_kept) out[pos] = j;
      base += __popcll(tm);
    };
    if (need == n_eq) {
      // every key equal to T is kept (the usual case): keep key >= T
      if constexpr (C > 0) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          if (64 * c >= nkb) break;
          put(key[c] >= T, lane + 64 * c);
        }
      } else {
        for (int j0 = 0; j0 < nkb; j0 += 64) put(key_at(j0 + lane) >= T, j0 + lane);
      }
    } else {
      // ties at T: keep the `need` lowest-indexed keys equal to T
      int eq_seen = 0;
      auto emit = [&](uint32_t kk, int j) {
        const bool eq = kk == T;
        const uint64_t eqm = __ballot(eq);
        const bool take = kk > T || (eq && eq_seen + __popcll(eqm & lt) < need);
        eq_seen += __popcll(eqm);
        put(take, j);
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
    }
  }
  for (int p = base + lane; p < max_kept; p += 64) out[p] = -1;
  return base;
}

// Keys per lane a row of nkb blocks needs, rounded up to an instantiated
// count (0: more than the largest).
// Keys-per-lane instantiations: ceil(nkb / 64) rounded up to one of these.
#define SPARSTAR_FOR_EACH_C(X) X(1) X(2) X(3) X(4) X(6) X(8) X(10) X(12) X(14) X(16) X(18) X(20) X(24) X(28) X(32)
#define SPARSTAR_FOR_EACH_C_LARGE(X) X(40) X(48) X(56) X(64) X(72)

inline int keys_per_lane(int64_t nkb) {
  const int64_t c = (nkb + 63) / 64;
  const int table[] = {1, 2, 3, 4, 6, 8, 10, 12, 14, 16, 18, 20, 24, 28, 32, 40, 48, 56, 64, 72};
  for (int t : table)
    if (c <= t) return t;
  return 0;
}

}  // namespace
}  // namespace sparstar
