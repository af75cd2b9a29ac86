// Clip-aware joint Top-K of SparSTAR (review sections "What carries the
// argument" and "Core claim"): per (batch, head, query block) keep the forced
// prefix blocks and the k highest-scoring eligible key blocks; write only the
// forward index list (ascending) and its length.
//
// One wavefront per row.  Scores become order-preserving uint32 keys
// (NaN lowest, -0 == +0, forced and out-of-range slots 0).  The k-th largest
// key T is found by bisection on the key bits, each step counting keys >=
// candidate with ballots: the first kPrefixBits steps on all keys, the rest on
// the few keys that still share T's prefix (packed into LDS).  Blocks with key
// > T are kept, and of the blocks with key == T the lowest-indexed
// (k - #greater) are kept, which is exactly "ties go to the lower block
// index".  The index list is then written in ascending order with a ballot
// prefix sum.
//
// Two kernels use this: select_kernel reads a row of S from memory;
// scores_select_kernel first computes 16 rows of S into LDS with the same
// fp64 tile code as the score kernel (bit-identical scores) and selects from
// there, so S never reaches HBM.
#include "score_tile.hpp"

namespace sparstar {
namespace {

constexpr int kWaves = 4;
constexpr int kPrefixBits = 12;   // bisection steps taken on all keys before packing candidates
constexpr int kFusedRows = 16;    // q rows per workgroup of the fused kernel
constexpr int kFusedWaves = 8;    // wavefronts per workgroup of the fused kernel

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

// Scores of kFusedRows q rows into LDS, then selection of each row from LDS.
// Score phase: the kFusedWaves wavefronts take the 16-column tiles in turn.
// Selection phase: each wavefront selects rows w, w + kFusedWaves; once a
// row's keys are in registers its LDS slice is free and holds the
// wavefront's candidate keys (row_stride = max(64 C, 128) words).
template <int D, int C>
__global__ __launch_bounds__(64 * kFusedWaves) void scores_select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb, int strips,
    int row_stride, double tau, int nf, int k, int32_t* __restrict__ cnt,
    int32_t* __restrict__ idx, int max_kept) {
  extern __shared__ float s_rows[];          // [kFusedRows][row_stride]
  const int64_t bh = blockIdx.x / strips;
  const int i0 = static_cast<int>(blockIdx.x - bh * strips) * kFusedRows;
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int lr = lane % 16, ls = lane / 16;
  const float* qh = qbar + bh * static_cast<int64_t>(nqb) * D;
  const float* kh = kbar + bh * static_cast<int64_t>(nkb) * D;

  const int ntk = (nkb + 15) / 16;
  if (w < ntk) {
    f32x4 qv[D / 16];
    const int iq = i0 + lr;   // rows past the edge read row 0 and are never selected
    load_operands<D>(qh + static_cast<int64_t>(iq < nqb ? iq : 0) * D + 4 * ls, qv);
    auto krow = [&](int jt) {
      const int jk = 16 * jt + lr;   // columns past the edge read row 0 and are not stored
      return kh + static_cast<int64_t>(jk < nkb ? jk : 0) * D + 4 * ls;
    };
    auto store = [&](const f64x4& acc, int jt) {
      const int jk = 16 * jt + lr;
      if (jk < nkb) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_rows[(ls + 4 * r) * row_stride + jk] = static_cast<float>(tau * acc[r]);
      }
    };
    // wavefront w takes tiles w, w + kFusedWaves, ...; the next one's k
    // operands load while the current one is on the matrix core
    f32x4 kv[D / 16];
    load_operands<D>(krow(w), kv);
    for (int jt = w; jt < ntk; jt += kFusedWaves) {
      f32x4 kn[D / 16];
      load_operands<D>(krow(jt + kFusedWaves < ntk ? jt + kFusedWaves : jt), kn);
      store(score_tile16<D>(qv, kv), jt);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) kv[c] = kn[c];
    }
  }
  __syncthreads();

  for (int rr = w; rr < kFusedRows; rr += kFusedWaves) {
    const int i = i0 + rr;
    if (i >= nqb) break;   // uniform per wave
    const float* s = s_rows + rr * row_stride;
    auto key_at = [&](int j) -> uint32_t {
      return (j >= nf && j < nkb) ? order_key(s[j]) : 0u;
    };
    uint32_t key[C];
    float v[C];   // all reads first (the row spans 64 C slots), then the keys
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = s[lane + 64 * c];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = lane + 64 * c;
      key[c] = static_cast<unsigned>(j - nf) < static_cast<unsigned>(nkb - nf) ? order_key(v[c]) : 0u;
    }
    const int64_t row = bh * nqb + i;
    // LDS returns a wavefront's reads in order: the keys are loaded before the
    // candidate writes into the same slice.
    uint32_t* cbuf = reinterpret_cast<uint32_t*>(s_rows + rr * row_stride);
    const int n = select_row<C>(key, key_at, lane, nkb, nf, k, cbuf,
                                idx + row * static_cast<int64_t>(max_kept), max_kept);
    if (lane == 0) cnt[row] = n;
  }
}

// Keys-per-lane instantiations: ceil(nkb / 64) rounded up to one of these.
#define SPARSTAR_FOR_EACH_C(X) X(1) X(2) X(3) X(4) X(6) X(8) X(10) X(12) X(14) X(16) X(18) X(20) X(24) X(28) X(32)
#define SPARSTAR_FOR_EACH_C_LARGE(X) X(40) X(48) X(56) X(64) X(72)

int keys_per_lane(int64_t nkb) {
  const int64_t c = (nkb + 63) / 64;
  const int table[] = {1, 2, 3, 4, 6, 8, 10, 12, 14, 16, 18, 20, 24, 28, 32, 40, 48, 56, 64, 72};
  for (int t : table)
    if (c <= t) return t;
  return 0;
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

int64_t fused_select_max_nkb() { return 64 * 32; }

sparstar_status launch_scores_select(const float* qbar, const float* kbar, int64_t BH,
                                     int64_t nqb, int64_t nkb, int64_t D, float tau,
                                     int64_t n_forced, int64_t k, int32_t* kv_count,
                                     int32_t* kv_index, int64_t max_kept, hipStream_t s) {
  const int64_t strips = (nqb + kFusedRows - 1) / kFusedRows;
  if (BH * strips > 2147483647LL) {
    set_error("sparstar_select_blocks_from_means: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  const int C = keys_per_lane(nkb);
  // every key slot a lane may read (64 C of them) lies inside the row
  const int row_stride = 64 * C < 128 ? 128 : 64 * C;
  const size_t lds = static_cast<size_t>(kFusedRows) * row_stride * sizeof(float);
  const dim3 grid(static_cast<uint32_t>(BH * strips)), block(64 * kFusedWaves);
  const int n = (int)nkb, nq = (int)nqb, st = (int)strips, f = (int)n_forced, kk = (int)k,
            mk = (int)max_kept;
  hipError_t e = hipSuccess;
#define SPARSTAR_FUSED_CASE_D(DD, CC)                                                             \
  if (lds > 65536)                                                                                \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scores_select_kernel<DD, CC>),        \
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));  \
  if (e == hipSuccess)                                                                            \
    scores_select_kernel<DD, CC><<<grid, block, lds, s>>>(qbar, kbar, nq, n, st, row_stride,     \
                                                          (double)tau, f, kk, kv_count, kv_index, \
                                                          mk);
#define SPARSTAR_FUSED_CASE(CC)            \
  case CC:                                 \
    if (D == 128) {                        \
      SPARSTAR_FUSED_CASE_D(128, CC)       \
    } else {                               \
      SPARSTAR_FUSED_CASE_D(64, CC)        \
    }                                      \
    break;
  switch (C) {
    SPARSTAR_FOR_EACH_C(SPARSTAR_FUSED_CASE)
    default:
      set_error("sparstar_select_blocks_from_means: nkb > %lld is not supported",
                (long long)fused_select_max_nkb());
      return SPARSTAR_ERR_UNSUPPORTED;
  }
#undef SPARSTAR_FUSED_CASE
#undef SPARSTAR_FUSED_CASE_D
  if (e != hipSuccess) {
    set_error("sparstar_select_blocks_from_means: %s", hipGetErrorString(e));
    return SPARSTAR_ERR_HIP;
  }
  return check_launch("sparstar_select_blocks_from_means");
}

}  // namespace sparstar
