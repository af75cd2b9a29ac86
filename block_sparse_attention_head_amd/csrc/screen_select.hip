// Block scores and clip-aware joint Top-K of SparSTAR without the score
// matrix in float32 (review, "What carries the argument": S_ij = tau *
// qbar_i . kbar_j, Eq. 2, then the forced prefix plus the k best eligible
// blocks per query block, ties to the lower index).  The result is the
// selection the two-call route (sparstar_block_scores + sparstar_select_blocks)
// makes, bit for bit.
//
// Screen, then refine.  The two-call route ranks F_ij, the float64 dot
// product of the float32 means rounded once to float32.  Computing every F_ij
// on the fp64 matrix cores costs more than the rest of the selection stage,
// yet only the blocks whose score lies close to a row's k-th largest decide
// anything.  Two kernels:
//  A. screen_kernel: every score approximated on the bf16 matrix cores from
//     a two-term split of each mean (x = hi + lo, both bf16; products
//     hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_bf16, float32
//     accumulation), scaled by tau and stored as float16 in the workspace;
//     work items of 48 query blocks x 32 key blocks, so each key-block mean
//     is read once per 48 query blocks.  The squared norms of the key-block
//     means go to the workspace too.
//  B. band_select_kernel, one wavefront per query block (row): a rigorous
//     bound E on |A_ij - F_ij| (A the stored value): the omitted split terms
//     (<= 3.02 * 2^-16 |q_d k_d|), the float32 accumulation of 3 D products
//     (gamma with u = 2^-23, whatever the hardware's internal rounding), the
//     scaling, the float16 storage (2^-11 relative, 2^-25 absolute) and F's
//     own rounding, the dot-product terms bounded by |qbar_i| max_j |kbar_j|.
//     T = the k-th largest A (radix select on 16-bit order keys); blocks with
//     A > T + 2E are kept and blocks with A < T - 2E dropped, each provably
//     so; the blocks in between ("the band") are decided on their exact F_ij,
//     keeping the best (k - #kept) by (F descending, index ascending).  The
//     exact values come from the score kernel's own fp64 tile code
//     (score_tile.hpp) with this row at its own position in its 16-row tile
//     and the same operations in the same order, hence the same float32
//     values.  A band no larger than what it must supply needs no exact
//     value.  A row whose band exceeds kBandCap, or with a non-finite
//     screened value, takes the exact route: all its exact scores, then the
//     usual row selector.
// The forward index list is written ascending, -1 padded, with its count.
#include <cmath>
#include <mutex>

#include "score_tile.hpp"
#include "select_row.hpp"

namespace sparstar {
namespace {

constexpr int kSWaves = 4;       // wavefronts (rows) per band-selection workgroup
constexpr int kBandCap = 48;     // band blocks per row decided on exact scores
constexpr int kMaxNkb = 2048;    // key blocks per row (a row lives in registers)
constexpr int kBitWords = kMaxNkb / 32;
constexpr int kScreenRowTiles = 3;   // 16-row tiles per screening work item
constexpr int kScreenColTiles = 2;   // 16-column tiles per screening work item

// Order key of float16 bits (NaN excluded beforehand): increasing with the
// value, -0 just below +0 (membership below is decided on float compares).
__device__ __forceinline__ uint32_t key16(uint32_t b) {
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}
__device__ __forceinline__ float half_bits_to_float(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}
__device__ __forceinline__ float value_of_key16(uint32_t key) {
  return half_bits_to_float((key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu));
}

// Eight consecutive floats as bf16 hi and lo parts (x = hi + lo + r with
// |r| <= 2^-16 |x|), and their sum of squares accumulated into ss.
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo,
                                       float& ss) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(x[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
    ss = fmaf(x[e], x[e], ss);
  }
}

// DPP lane moves (GFX9 encodings): row_shr:n = 0x110 + n within rows of 16
// lanes; row_bcast:15 / :31 pass lane 15 of each row (lane 31) on to the
// rows selected by the row mask.  Lanes without a source keep `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += dpp_i<0x111>(0, x);
  x += dpp_i<0x112>(0, x);
  x += dpp_i<0x114>(0, x);
  x += dpp_i<0x118>(0, x);
  x += dpp_i<0x142, 0xa>(0, x);
  x += dpp_i<0x143, 0xc>(0, x);
  return x;
}

// Sum over the 64 lanes (the same order for every lane; the result is used
// only inside an error bound, which carries a relative slack for it).
__device__ __forceinline__ float wave_sum_f(float v) {
  v += __int_as_float(dpp_i<0x111>(0, __float_as_int(v)));
  v += __int_as_float(dpp_i<0x112>(0, __float_as_int(v)));
  v += __int_as_float(dpp_i<0x114>(0, __float_as_int(v)));
  v += __int_as_float(dpp_i<0x118>(0, __float_as_int(v)));
  v += __int_as_float(dpp_i<0x142, 0xa>(0, __float_as_int(v)));
  v += __int_as_float(dpp_i<0x143, 0xc>(0, __float_as_int(v)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Largest value over the 64 lanes of non-negative floats (compared as bits).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int x = __float_as_int(v);
  x = max(x, dpp_i<0x111>(x, x));
  x = max(x, dpp_i<0x112>(x, x));
  x = max(x, dpp_i<0x114>(x, x));
  x = max(x, dpp_i<0x118>(x, x));
  x = max(x, dpp_i<0x142, 0xa>(x, x));
  x = max(x, dpp_i<0x143, 0xc>(x, x));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

// One level of a radix select from the top: hist[b] counts the candidates
// whose digit is 255 - b (so bin 0 holds the largest digit).  Returns the
// digit of the k-th largest candidate and, in *above, how many candidates
// have a larger digit.  Lane l looks after bins 4 l .. 4 l + 3.
__device__ __forceinline__ int radix_level(const uint32_t* hist, int lane, int k, int* above) {
  const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                 h3 = hist[4 * lane + 3];
  const int s = static_cast<int>(h0 + h1 + h2 + h3);
  const int incl = wave_inclusive_scan(s);
  const uint64_t hit = __ballot(incl >= k);       // k <= candidates, so some lane hits
  const int L = __ffsll(static_cast<unsigned long long>(hit)) - 1;
  int excl = incl - s, j = 3;
  if (excl + static_cast<int>(h0) >= k) j = 0;
  else if (excl + static_cast<int>(h0 + h1) >= k) { j = 1; excl += h0; }
  else if (excl + static_cast<int>(h0 + h1 + h2) >= k) { j = 2; excl += h0 + h1; }
  else excl += h0 + h1 + h2;
  *above = __builtin_amdgcn_readlane(excl, L);
  return 255 - __builtin_amdgcn_readlane(4 * lane + j, L);
}

// The k-th largest of the nonzero 16-bit keys of a row (k >= 1 and at most
// that many nonzero keys), by a two-level radix select over per-wave LDS
// histograms of 256 bins.
template <int C>
__device__ __forceinline__ uint32_t kth_largest16(const uint32_t (&key)[C], int k, int lane,
                                                 uint32_t* hist) {
  // level 1: high byte
  *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (key[c] != 0u) atomicAdd(&hist[255 - (key[c] >> 8)], 1u);
  __builtin_amdgcn_wave_barrier();
  int above = 0;
  const uint32_t hi8 = static_cast<uint32_t>(radix_level(hist, lane, k, &above));
  __builtin_amdgcn_wave_barrier();
  // level 2: low byte of the keys in that high-byte bin
  *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (key[c] != 0u && (key[c] >> 8) == hi8) atomicAdd(&hist[255 - (key[c] & 0xffu)], 1u);
  __builtin_amdgcn_wave_barrier();
  int above2 = 0;
  const uint32_t lo8 = static_cast<uint32_t>(radix_level(hist, lane, k - above, &above2));
  __builtin_amdgcn_wave_barrier();
  return (hi8 << 8) | lo8;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) x = fmaxf(x, __shfl_xor(x, d));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) x += __shfl_xor(x, d);
  return x;
}

// ---------------------------------------------------------------------------
// A. screening
// ---------------------------------------------------------------------------
// One wavefront per workgroup, exactly as many as the GPU holds at once; each
// takes a contiguous run of work items (strip-major, so its q operands are
// reloaded only when the 48-row strip changes).  Item = 48 query blocks x 32
// key blocks: per 16-column tile, the key means are split once and multiply
// all three 16-row tiles; the next tile's key means load while the current
// one is on the matrix cores.
template <int D>
__global__ __launch_bounds__(64) void screen_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb, int strips,
    int pairs, int64_t items, float tau, int ws_stride, uint16_t* __restrict__ app,
    float* __restrict__ kn2) {
  constexpr int KS = D / 32;
  const int64_t per = (items + gridDim.x - 1) / gridDim.x;
  const int64_t it0 = blockIdx.x * per;
  const int64_t it1 = it0 + per < items ? it0 + per : items;
  const int lane = threadIdx.x, lr = lane % 16, lg = lane / 16;
  const int ntk = (nkb + 15) / 16;

  // key-mean operands of column tile jt (lane (lr, lg): block 16 jt + lr, the
  // same dimensions as the q operands), clamped to a valid block
  auto load_b = [&](int64_t bh_, int jt, f32x4 (&kr)[2 * KS]) {
    const float* kp = kbar + (bh_ * nkb + min(16 * jt + lr, nkb - 1)) * static_cast<int64_t>(D) + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[2 * ks] = *reinterpret_cast<const f32x4*>(kp + 32 * ks);
      kr[2 * ks + 1] = *reinterpret_cast<const f32x4*>(kp + 32 * ks + 4);
    }
  };
  auto item_start = [&](int64_t it, int64_t& bh_, int& jt) {
    const int64_t hs = it / pairs;
    bh_ = hs / strips;
    jt = kScreenColTiles * static_cast<int>(it - hs * pairs);
  };

  int64_t cur_strip = -1;
  bf16x8 qa_hi[kScreenRowTiles][KS], qa_lo[kScreenRowTiles][KS];
  f32x4 kr[2 * KS];
  if (it0 < it1) {
    int64_t b0;
    int j0;
    item_start(it0, b0, j0);
    load_b(b0, j0, kr);
  }
  for (int64_t it = it0; it < it1; ++it) {
    const int64_t hs = it / pairs;               // (b*h) * strips + strip
    const int pair = static_cast<int>(it - hs * pairs);
    const int64_t bh = hs / strips;
    const int r0 = static_cast<int>(hs - bh * strips) * 16 * kScreenRowTiles;
    if (hs != cur_strip) {
      // A operands: lane (lr, lg) holds row r0 + 16 t + lr, dimensions 32 ks + 8 lg + [0, 8)
#pragma unroll
      for (int t = 0; t < kScreenRowTiles; ++t) {
        const float* qp = qbar + (bh * nqb + min(r0 + 16 * t + lr, nqb - 1)) * static_cast<int64_t>(D) + 8 * lg;
        float ss = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          split8(*reinterpret_cast<const f32x4*>(qp + 32 * ks),
                 *reinterpret_cast<const f32x4*>(qp + 32 * ks + 4), qa_hi[t][ks], qa_lo[t][ks], ss);
      }
      cur_strip = hs;
    }
#pragma unroll 1
    for (int c = 0; c < kScreenColTiles; ++c) {
      const int jt = kScreenColTiles * pair + c;
      if (jt >= ntk) break;
      const int jc = 16 * jt + lr;
      // the next tile of this item, else the first tile of the next item
      f32x4 kn[2 * KS];
      {
        int64_t nbh = bh;
        int njt = jt + 1;
        if (c + 1 == kScreenColTiles || njt >= ntk) item_start(it + 1 < it1 ? it + 1 : it, nbh, njt);
        load_b(nbh, njt, kn);
      }
      f32x4 acc[kScreenRowTiles];
#pragma unroll
      for (int t = 0; t < kScreenRowTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      float kss = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 bh8, bl8;
        split8(kr[2 * ks], kr[2 * ks + 1], bh8, bl8, kss);
#pragma unroll
        for (int t = 0; t < kScreenRowTiles; ++t) {
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa_hi[t][ks], bh8, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa_hi[t][ks], bl8, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa_lo[t][ks], bh8, acc[t], 0, 0, 0);
        }
      }
      if (jc < nkb) {
        // acc[t][r] = A(row r0 + 16 t + 4 lg + r, block jc)
#pragma unroll
        for (int t = 0; t < kScreenRowTiles; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = r0 + 16 * t + 4 * lg + r;
            if (i < nqb)
              app[(bh * nqb + i) * static_cast<int64_t>(ws_stride) + jc] =
                  __builtin_bit_cast(uint16_t, static_cast<_Float16>(tau * acc[t][r]));
          }
      }
      kss += __shfl_xor(kss, 16);
      kss += __shfl_xor(kss, 32);
      if (r0 == 0 && jc < nkb && lg == 0) kn2[bh * nkb + jc] = kss;
#pragma unroll
      for (int x = 0; x < 2 * KS; ++x) kr[x] = kn[x];
    }
  }
}

// ---------------------------------------------------------------------------
// B. band selection
// ---------------------------------------------------------------------------
// One wavefront per query block (row), kSWaves independent rows per
// workgroup.  The row's screened values live in registers (slot c of lane l
// = block l + 64 c).  The exact scores of its band come from fp64 tiles laid
// out as the score kernel lays them out: the A operand holds the 16 rows of
// the row's 16-row tile (this row at its own position), the B operand holds
// band blocks; only this row's results are kept.
template <int D, int C>
__global__ __launch_bounds__(64 * kSWaves, C > 18 ? 2 : 4) void band_select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int64_t rows, int nqb, int nkb,
    float tau, int nf, int k, const uint16_t* __restrict__ app, const float* __restrict__ kn2,
    int ws_stride, int stride, int32_t* __restrict__ cnt, int32_t* __restrict__ idx,
    int max_kept) {
  extern __shared__ float s_exact_rows[];          // [kSWaves][stride]: exact route only
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kSWaves][256];
  __shared__ float s_bandF[kSWaves][kBandCap];
  __shared__ int32_t s_bandC[kSWaves][kBandCap];
  __shared__ uint32_t s_chosen[kSWaves][kBitWords];

  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kSWaves + w;
  if (row >= rows) return;                          // uniform per wave; no workgroup barrier below
  const int64_t bh = row / nqb;
  const int i = static_cast<int>(row - bh * nqb);
  const int lr = lane % 16, lg = lane / 16;
  const float* qh = qbar + bh * static_cast<int64_t>(nqb) * D;
  const float* kh = kbar + bh * static_cast<int64_t>(nkb) * D;
  const uint64_t lt = lanemask_lt(lane);
  int32_t* out = idx + row * static_cast<int64_t>(max_kept);
  const double tau_d = static_cast<double>(tau);

  // all loads first: the row's screened values, the key-block norms of the
  // head, and this query mean
  uint32_t raw[C];
  float kv2[C];
  float qx[D / 64];
  {
    const uint16_t* arow = app + row * static_cast<int64_t>(ws_stride);
#pragma unroll
    for (int c = 0; c < C; ++c) raw[c] = arow[lane + 64 * c];   // inside the workspace row
#pragma unroll
    for (int c = 0; c < C; ++c) kv2[c] = kn2[bh * nkb + min(lane + 64 * c, nkb - 1)];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) qx[e] = qh[static_cast<int64_t>(i) * D + lane + 64 * e];
  }
  // raw[c] becomes the slot's order key (0 for forced and past-the-end
  // slots); its value is recovered from the key when needed
  bool bad = false;
  float amax = 0.f, kmax2 = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = lane + 64 * c;
    const bool el = static_cast<unsigned>(j - nf) < static_cast<unsigned>(nkb - nf);
    const float av = half_bits_to_float(raw[c]);
    kmax2 = fmaxf(kmax2, kv2[c]);
    if (el) {
      bad = bad || !(fabsf(av) <= 65504.f);
      amax = fmaxf(amax, fabsf(av));
    }
    raw[c] = el ? key16(raw[c]) : 0u;
  }
  const uint32_t (&key)[C] = raw;
  auto val = [&](int c) { return value_of_key16(key[c]); };
  float qss = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) qss = fmaf(qx[e], qx[e], qss);

  bool full_exact = __ballot(bad) != 0;             // non-finite screened value
  float lo = INFINITY, hi = INFINITY;
  bool exact = false;
  if (!full_exact && k > 0) {
    amax = wave_max_nonneg(amax);
    const float kmax = sqrtf(wave_max_nonneg(kmax2)) * 1.0001f;
    const float qn = sqrtf(wave_sum_f(qss)) * 1.0001f;
    const float t = value_of_key16(kth_largest16<C>(key, k, lane, s_hist[w]));
    const float E = 1.2e-4f * fabsf(tau) * qn * kmax + 6e-4f * amax + 1e-7f;
    lo = t - 2.f * E;
    hi = t + 2.f * E;
    int n_in = 0, m = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool el = key[c] != 0u;
      const float av = val(c);
      n_in += wave_count(el && av > hi);
      m += wave_count(el && av >= lo && av <= hi);
    }
    const int need = k - n_in;                      // 1 <= need <= m (the k-th lies in the band)
    exact = m > need;
    if (exact && (m > kBandCap || !(E < INFINITY))) {
      full_exact = true;
    } else if (exact) {
      // the band's blocks, ascending, into LDS
      int pos = 0;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float av = val(c);
        const bool in = key[c] != 0u && av >= lo && av <= hi;
        const uint64_t mk = __ballot(in);
        if (in) s_bandC[w][pos + __popcll(mk & lt)] = lane + 64 * c;
        pos += __popcll(mk);
      }
      __builtin_amdgcn_wave_barrier();
      // exact scores of the band, 16 blocks per fp64 tile
      const int i0 = i & ~15, rpos = i - i0;
      f32x4 qv[D / 16];
      load_operands<D>(qh + static_cast<int64_t>(min(i0 + lr, nqb - 1)) * D + 4 * lg, qv);
      for (int c0 = 0; c0 < m; c0 += 16) {
        const int col = s_bandC[w][min(c0 + lr, m - 1)];
        f32x4 kq[D / 16];
        load_operands<D>(kh + static_cast<int64_t>(col) * D + 4 * lg, kq);
        const f64x4 acc = score_tile16<D>(qv, kq);
        // fp64 tile layout: lane (lr, lg) holds rows lg + 4 r of column lr
        if (lg == (rpos & 3) && c0 + lr < m) s_bandF[w][c0 + lr] = static_cast<float>(tau_d * acc[rpos >> 2]);
      }
      __builtin_amdgcn_wave_barrier();
      // keep the best `need` of the band: higher F first, then the lower index
      for (int x = lane; x < kBitWords; x += 64) s_chosen[w][x] = 0u;
      __builtin_amdgcn_wave_barrier();
      const float fe = lane < m ? s_bandF[w][lane] : 0.f;
      const int ce = lane < m ? s_bandC[w][lane] : 0;
      int rank = 0;
      for (int e = 0; e < m; ++e) {
        const float f2 = s_bandF[w][e];
        const int c2 = s_bandC[w][e];
        rank += (f2 > fe || (f2 == fe && c2 < ce)) ? 1 : 0;
      }
      if (lane < m && rank < need) atomicOr(&s_chosen[w][ce >> 5], 1u << (ce & 31));
      __builtin_amdgcn_wave_barrier();
    }
  }

  if (!full_exact) {
    for (int p = lane; p < nf; p += 64) out[p] = p;
    int base = nf;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (64 * c >= nkb) break;
      const int j = lane + 64 * c;
      const float av = val(c);
      const bool take = key[c] != 0u &&
                        (av > hi || (av >= lo && (!exact || ((s_chosen[w][j >> 5] >> (j & 31)) & 1u))));
      const uint64_t tm = __ballot(take);
      const int pos = base + __popcll(tm & lt);
      if (take && pos < max_kept) out[pos] = j;
      base += __popcll(tm);
    }
    for (int p = base + lane; p < max_kept; p += 64) out[p] = -1;
    if (lane == 0) cnt[row] = base;
    return;
  }

  // ---- exact route for this row: every exact score, then the row selector ------
  float* srow = s_exact_rows + w * stride;
  {
    const int i0 = i & ~15, rpos = i - i0;
    f32x4 qv[D / 16];
    load_operands<D>(qh + static_cast<int64_t>(min(i0 + lr, nqb - 1)) * D + 4 * lg, qv);
    const int ntk = (nkb + 15) / 16;
    for (int jt = 0; jt < ntk; ++jt) {
      const int jc = 16 * jt + lr;
      f32x4 kq[D / 16];
      load_operands<D>(kh + static_cast<int64_t>(min(jc, nkb - 1)) * D + 4 * lg, kq);
      const f64x4 acc = score_tile16<D>(qv, kq);
      if (lg == (rpos & 3) && jc < nkb) srow[jc] = static_cast<float>(tau_d * acc[rpos >> 2]);
    }
  }
  __builtin_amdgcn_wave_barrier();
  auto key_at = [&](int j) -> uint32_t { return (j >= nf && j < nkb) ? order_key(srow[j]) : 0u; };
  uint32_t ekey[C];
  float v[C];
#pragma unroll
  for (int c = 0; c < C; ++c) v[c] = srow[lane + 64 * c];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = lane + 64 * c;
    ekey[c] = static_cast<unsigned>(j - nf) < static_cast<unsigned>(nkb - nf) ? order_key(v[c]) : 0u;
  }
  __builtin_amdgcn_wave_barrier();
  // the keys are in registers, so the row's slice holds the candidate keys
  const int n = select_row<C>(ekey, key_at, lane, nkb, nf, k, reinterpret_cast<uint32_t*>(srow), out,
                              max_kept);
  if (lane == 0) cnt[row] = n;
}

// Resident one-wavefront workgroups of `kernel` on the current device.
template <typename K>
sparstar_status resident_waves(K kernel, int64_t& waves) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess ||
      cus < 1 || per_cu < 1) {
    set_error("sparstar_select_blocks_from_means: cannot query the device");
    return SPARSTAR_ERR_HIP;
  }
  waves = static_cast<int64_t>(cus) * per_cu;
  return SPARSTAR_OK;
}

// Workspace layout: screened scores [BH][nqb][ws_stride] float16, then the
// squared norms of the key-block means [BH][nkb] float32 (256-byte aligned).
struct Layout {
  int C, ws_stride;
  int64_t kn2_off, total;
};

Layout layout_of(int64_t BH, int64_t nqb, int64_t nkb) {
  auto up256 = [](int64_t x) { return (x + 255) / 256 * 256; };
  Layout L;
  L.C = keys_per_lane(nkb);
  L.ws_stride = 64 * (L.C > 0 ? L.C : 1);
  L.kn2_off = up256(BH * nqb * L.ws_stride * 2);
  L.total = L.kn2_off + BH * nkb * 4;
  return L;
}

}  // namespace

int64_t fused_select_max_nkb() { return kMaxNkb; }

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: a fixed device array instead of
// a caller workspace.  Each GPU the library runs on holds its own copy until
// the process ends; every call on that GPU uses it, so calls that overlap in
// time on one GPU race.  Nothing in it needs to start at zero (the screening
// kernel writes every entry the band kernel reads for real blocks).
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int64_t select_scratch_bytes() { return kScratchBytes; }

// The current device's address of `scratch`, looked up once per device (the
// array's name is only a host-side stand-in; kernels and copies take this).
sparstar_status select_scratch_pointer(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("sparstar_select_blocks_from_means_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return SPARSTAR_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("sparstar_select_blocks_from_means_noalloc: device %d beyond the %d supported", dev,
              kMaxDevices);
    return SPARSTAR_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("sparstar_select_blocks_from_means_noalloc: hipGetSymbolAddress: %s",
                hipGetErrorString(e));
      return SPARSTAR_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPARSTAR_OK;
}

int64_t select_workspace_bytes(int64_t BH, int64_t nqb, int64_t nkb) {
  return layout_of(BH, nqb, nkb).total;
}

sparstar_status launch_scores_select(const float* qbar, const float* kbar, int64_t BH,
                                     int64_t nqb, int64_t nkb, int64_t D, float tau,
                                     int64_t n_forced, int64_t k, int32_t* kv_count,
                                     int32_t* kv_index, int64_t max_kept, void* workspace,
                                     hipStream_t s) {
  const Layout L = layout_of(BH, nqb, nkb);
  uint16_t* app = static_cast<uint16_t*>(workspace);
  float* kn2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.kn2_off);
  const int n = (int)nkb, nq = (int)nqb, f = (int)n_forced, kk = (int)k, mk = (int)max_kept;

  // A. screening: exactly the resident wavefronts, items split evenly
  const int64_t sstrips = (nqb + 16 * kScreenRowTiles - 1) / (16 * kScreenRowTiles);
  const int64_t pairs = ((nkb + 15) / 16 + kScreenColTiles - 1) / kScreenColTiles;
  const int64_t items = BH * sstrips * pairs;
  int64_t waves = 0;
  sparstar_status st = resident_waves(D == 128 ? screen_kernel<128> : screen_kernel<64>, waves);
  if (st != SPARSTAR_OK) return st;
  const dim3 sgrid(static_cast<uint32_t>(items < waves ? items : waves)), sblock(64);
  if (D == 128)
    screen_kernel<128><<<sgrid, sblock, 0, s>>>(qbar, kbar, nq, n, (int)sstrips, (int)pairs, items,
                                                tau, L.ws_stride, app, kn2);
  else
    screen_kernel<64><<<sgrid, sblock, 0, s>>>(qbar, kbar, nq, n, (int)sstrips, (int)pairs, items,
                                               tau, L.ws_stride, app, kn2);
  if ((st = check_launch("sparstar_select_blocks_from_means")) != SPARSTAR_OK) return st;

  // B. band selection, one wavefront per query block
  const int64_t rows = BH * nqb;
  const int64_t wgs = (rows + kSWaves - 1) / kSWaves;
  if (wgs > 2147483647LL) {
    set_error("sparstar_select_blocks_from_means: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  // the exact route keeps one row of float32 scores per wavefront: every slot
  // a lane reads (64 C of them) lies inside it, and it holds the selector's
  // 128 candidate words
  const int stride = 64 * L.C < 128 ? 128 : 64 * L.C;
  const size_t lds = static_cast<size_t>(kSWaves) * stride * sizeof(float);
  const dim3 grid(static_cast<uint32_t>(wgs)), block(64 * kSWaves);
  hipError_t e = hipSuccess;
#define SPARSTAR_BAND_CASE_D(DD, CC)                                                              \
  if (lds > 49152)                                                                                \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&band_select_kernel<DD, CC>),          \
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));  \
  if (e == hipSuccess)                                                                            \
    band_select_kernel<DD, CC><<<grid, block, lds, s>>>(qbar, kbar, rows, nq, n, tau, f, kk, app, \
                                                        kn2, L.ws_stride, stride, kv_count,       \
                                                        kv_index, mk);
#define SPARSTAR_BAND_CASE(CC)         \
  case CC:                             \
    if (D == 128) {                    \
      SPARSTAR_BAND_CASE_D(128, CC)    \
    } else {                           \
      SPARSTAR_BAND_CASE_D(64, CC)     \
    }                                  \
    break;
  switch (L.C) {
    SPARSTAR_FOR_EACH_C(SPARSTAR_BAND_CASE)
    default:
      set_error("sparstar_select_blocks_from_means: nkb > %lld is not supported",
                (long long)fused_select_max_nkb());
      return SPARSTAR_ERR_UNSUPPORTED;
  }
#undef SPARSTAR_BAND_CASE
#undef SPARSTAR_BAND_CASE_D
  if (e != hipSuccess) {
    set_error("sparstar_select_blocks_from_means: %s", hipGetErrorString(e));
    return SPARSTAR_ERR_HIP;
  }
  return check_launch("sparstar_select_blocks_from_means");
}

}  // namespace sparstar
