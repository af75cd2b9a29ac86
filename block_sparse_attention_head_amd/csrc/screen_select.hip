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
//     hi*hi + hi*lo + lo*hi on v_mfma_f32_32x32x16_bf16, float32
//     accumulation), scaled by tau and stored as float16 in the workspace.
//     Forced blocks and the row padding past nkb get the sentinel 0xffff,
//     and a non-finite value is stored as +NaN (0x7e00), so the selection
//     sees every ineligible slot as key 0 and every non-finite one above
//     +inf.  The largest squared norm of the key-block means of each
//     128-block strip goes to the workspace too.
//  B. band_select_kernel, one wavefront per query block (row): a rigorous
//     bound |A_ij - F_ij| <= e(A_ij) = 1.001 (e1 + 6e-4 |A_ij|) (A the stored
//     value).  e1 = 1.2e-4 |tau| |qbar_i| max_j |kbar_j| covers the omitted
//     split terms (<= 3.02 * 2^-16 |q_d k_d|) and the float32 accumulation of
//     3 D products (gamma with u = 2^-23, whatever the hardware's internal
//     rounding), plus 1e-7 for float16 subnormals; 6e-4 |A| covers the
//     scaling, the float16 storage (2^-11 relative) and F's own rounding.
//     T = the k-th largest A (radix select on 16-bit order keys).  As
//     a -+ 6.006e-4 |a| increase with a, the k blocks with the largest A
//     have F >= T - e(T) and the others F <= T + e(T), so F's k-th largest
//     lies in [T - e(T), T + e(T)]; blocks with A above hi (below lo), set so
//     that F_ij is provably above (below) that interval, are kept (dropped);
//     the blocks in between ("the band") are decided on their exact F_ij,
//     keeping the best (k - #kept) by (F descending, index ascending).  The
//     exact values are the score kernel's fp64 sums (score_tile.hpp): the
//     same dimension groups in the same order, on the one-row 4 x 4 x 4
//     form of its matrix-core step, hence the same float32 values.  A band no larger than what it must supply needs no exact
//     value.  A row whose band exceeds kBandCap, or with a non-finite
//     screened value, takes the exact route: all its exact scores, then the
//     usual row selector.
// The forward index list is written ascending, -1 padded, with its count.
#include <cmath>
#include <mutex>

#include "score_tile.hpp"
#include "select_row.hpp"
#include "tile_common.hpp"

namespace sparstar {
namespace {

// wavefronts (rows) per band-selection workgroup: one, so that a slot frees as
// soon as its row is done (rows differ widely in work: a band decided on exact
// scores takes an fp64 tile; four-row workgroups measured 2 us slower at 72k)
constexpr int kSWaves = 1;
constexpr int kBandCap = 48;     // band blocks per row decided on exact scores
constexpr int kMaxNkb = 2048;    // key blocks per row (a row lives in registers)
constexpr uint32_t kSentinel16 = 0xffffu;   // float16 bits whose order key is 0
constexpr uint32_t kNaN16 = 0x7e00u;        // any non-finite screened value

// Order key of float16 bits: increasing with the value, -0 just below +0.
// Only the sentinel 0xffff maps to 0; +inf maps to 0xfc00 and the stored
// NaN 0x7e00 to 0xfe00, every finite value to [0x0400, 0xfbff].
__device__ __forceinline__ uint32_t key16(uint32_t b) {
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}
__device__ __forceinline__ float half_bits_to_float(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}
__device__ __forceinline__ float value_of_key16(uint32_t key) {
  return half_bits_to_float((key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu));
}

// The smallest key of a finite float16 (in [0x0400, 0xfc00], 0xfc00 = +inf)
// whose value exceeds x (strict) or reaches x (!strict); x finite.  The key
// of the nearest float16 is at most two steps from it.
__device__ __forceinline__ uint32_t key_threshold(float x, bool strict) {
  uint32_t kk = key16(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
  kk = kk < 0x0400u ? 0x0400u : (kk > 0xfc00u ? 0xfc00u : kk);
  auto in = [&](uint32_t q) { return strict ? value_of_key16(q) > x : value_of_key16(q) >= x; };
#pragma unroll
  for (int it = 0; it < 3; ++it)
    if (kk < 0xfc00u && !in(kk)) ++kk;
#pragma unroll
  for (int it = 0; it < 3; ++it)
    if (kk > 0x0400u && in(kk - 1)) --kk;
  return kk;
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

// Largest unsigned value over the 64 lanes.
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  int x = static_cast<int>(v);
  x = static_cast<int>(max(static_cast<uint32_t>(x), static_cast<uint32_t>(dpp_i<0x111>(x, x))));
  x = static_cast<int>(max(static_cast<uint32_t>(x), static_cast<uint32_t>(dpp_i<0x112>(x, x))));
  x = static_cast<int>(max(static_cast<uint32_t>(x), static_cast<uint32_t>(dpp_i<0x114>(x, x))));
  x = static_cast<int>(max(static_cast<uint32_t>(x), static_cast<uint32_t>(dpp_i<0x118>(x, x))));
  x = static_cast<int>(max(static_cast<uint32_t>(x), static_cast<uint32_t>(dpp_i<0x142, 0xa>(x, x))));
  x = static_cast<int>(max(static_cast<uint32_t>(x), static_cast<uint32_t>(dpp_i<0x143, 0xc>(x, x))));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
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

// The k-th largest of the nonzero 16-bit keys of a row (k >= 1, at most that
// many nonzero keys, all of them >= 0x0400), by a two-level radix select over
// a per-wave LDS histogram of 256 bins plus one spare bin per lane.  Key 0
// lands in bin 255, which holds no nonzero key, so it is never reached.  In
// the second level the keys outside the chosen high-byte bin go to their
// lane's spare bin, so the atomics need no branch and do not collide.
template <int CL>
__device__ __forceinline__ uint32_t kth_largest16(const uint32_t (&key)[CL], int k, int lane,
                                                 uint32_t* hist) {
  // level 1: high byte
  *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  hist[256 + lane] = 0u;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int s = 0; s < CL; ++s) atomicAdd(&hist[255 - (key[s] >> 8)], 1u);
  __builtin_amdgcn_wave_barrier();
  int above = 0;
  const uint32_t hi8 = static_cast<uint32_t>(radix_level(hist, lane, k, &above));
  __builtin_amdgcn_wave_barrier();
  // level 2: low byte of the keys in that high-byte bin
  *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int s = 0; s < CL; ++s) {
    const bool in = (key[s] >> 8) == hi8;
    atomicAdd(&hist[in ? 255 - (key[s] & 0xffu) : 256 + lane], 1u);
  }
  __builtin_amdgcn_wave_barrier();
  int above2 = 0;
  const uint32_t lo8 = static_cast<uint32_t>(radix_level(hist, lane, k - above, &above2));
  __builtin_amdgcn_wave_barrier();
  return (hi8 << 8) | lo8;
}

// ---------------------------------------------------------------------------
// A. screening
// ---------------------------------------------------------------------------
// One workgroup of four wavefronts per tile of 128 query blocks x 128 key
// blocks of one head, on v_mfma_f32_32x32x16_bf16 (S^T = Kbar Qbar^T: the
// key means are the A operand).  Every global access is a run of whole
// 16-byte pieces, consecutive lanes on consecutive bytes, and LDS turns the
// data around:
//  * each wavefront reads its 32 query means (16 KiB, contiguous) into LDS
//    as float32 and takes back its MFMA operand slices, split into bf16 hi
//    and lo parts (x = hi + lo + r, |r| <= 2^-16 |x|);
//  * the workgroup then reads the tile's 128 key means (contiguous) and
//    keeps them in LDS split the same way, rows of one block with an XOR
//    swizzle of the 16-byte chunks;
//  * each lane ends with 4 adjacent key blocks of one query block per
//    register group; two 32 x 32 tiles go through a per-wavefront LDS patch
//    and leave as 128-byte row pieces.
// The workspace rows are 128 * cstrips wide, so the tiles cover every slot.
// Tiles are numbered head-major and dealt out so that the workgroups on one
// XCD (workgroups go round-robin over the 8 XCDs) work on the same heads,
// whose means then sit in that XCD's L2.
constexpr int kScrWaves = 4;
constexpr int kScrRows = 32 * kScrWaves;   // query blocks per tile
constexpr int kScrCols = 128;              // key blocks per tile (one strip)

template <int D>
__global__ __launch_bounds__(64 * kScrWaves) void screen_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb, int nf,
    int rstrips, int cstrips, int tiles, int per_xcd, float tau, int ws_stride,
    uint16_t* __restrict__ app, float* __restrict__ kmaxp) {
  constexpr int NT = 64 * kScrWaves;
  constexpr int KS = D / 16;                    // k-steps of 16 dimensions
  constexpr int CPB = D / 4;                    // float4 chunks per mean (query or key block)
  constexpr int KLOADS = kScrCols * CPB / NT;   // float4 loads per thread, key means
  constexpr int QLOADS = 32 * CPB / 64;         // float4 loads per lane, query means
  constexpr int RB = D * 2;                     // bytes per LDS key row (bf16)
  constexpr int QRB = D * 4;                    // bytes per LDS query row (float32)
  static_assert(kScrWaves * 32 * QRB <= 2 * kScrCols * RB, "query staging fits the key region");
  // key region: hi rows then lo rows; before that it stages the query means
  __shared__ __attribute__((aligned(16))) unsigned char s_key[2 * kScrCols * RB];
  __shared__ __attribute__((aligned(16))) unsigned char s_out[kScrWaves][32 * 128];
  // the strip's largest squared norm, in wavefront 0's patch before its first use
  // (80 KiB in all, so that two workgroups share a CU)
  uint32_t* const s_kmax = reinterpret_cast<uint32_t*>(s_out[0]);
  unsigned char* const s_hi = s_key;
  unsigned char* const s_lo = s_key + kScrCols * RB;

  const int L = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (L >= tiles) return;                       // whole workgroup, before any barrier
  const int per_head = rstrips * cstrips;
  const int64_t bh = L / per_head;
  const int rs = (L - static_cast<int>(bh) * per_head) / cstrips;
  const int cs = L - static_cast<int>(bh) * per_head - rs * cstrips;
  const int t = threadIdx.x, lane = t % 64, w = t / 64;
  const int c0 = cs * kScrCols;
  const int q0 = rs * kScrRows + 32 * w;        // this wavefront's first query block
  if (t == 0) *s_kmax = 0u;

  // global reads, all issued up front: query means (load i, lane l -> chunk
  // 64 i + l of the wavefront's 32 rows) and key means (load i, thread t ->
  // chunk t + NT i of the tile's 128 rows); rows past the end repeat the last
  f32x4 qg[QLOADS], kg[KLOADS];
  {
    const float* qp = qbar + bh * static_cast<int64_t>(nqb) * D;
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int c = 64 * i + lane;
      const int r = min(q0 + c / CPB, nqb - 1);
      qg[i] = *reinterpret_cast<const f32x4*>(qp + static_cast<int64_t>(r) * D + 4 * (c % CPB));
    }
    const float* kp = kbar + bh * static_cast<int64_t>(nkb) * D;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int c = t + NT * i;
      const int b = min(c0 + c / CPB, nkb - 1);
      kg[i] = *reinterpret_cast<const f32x4*>(kp + static_cast<int64_t>(b) * D + 4 * (c % CPB));
    }
  }

  // query means through LDS (float32 rows, chunk ^ (row % 16)) into the
  // operand layout: lane l holds query block q0 + l % 32, dimensions
  // 16 ks + 8 (l / 32) + [0, 8)
  bf16x8 a_hi[KS], a_lo[KS];
  {
    unsigned char* qs = s_key + w * 32 * QRB;
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      const int c = 64 * i + lane, r = c / CPB, ch = c % CPB;
      *reinterpret_cast<f32x4*>(qs + r * QRB + (ch ^ (r & 15)) * 16) = qg[i];
    }
    __syncthreads();
    const int r = lane % 32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 4 * ks + 2 * (lane / 32);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(qs + r * QRB + (ch ^ (r & 15)) * 16);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(qs + r * QRB + ((ch + 1) ^ (r & 15)) * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? x0[e] : x1[e - 4];
        const __bf16 hb = static_cast<__bf16>(x);
        a_hi[ks][e] = hb;
        a_lo[ks][e] = static_cast<__bf16>(x - static_cast<float>(hb));
      }
    }
    __syncthreads();                            // the region is the key tile's next
  }

  float ssmax = 0.f;                            // largest squared norm seen (rs == 0)
  // key means split into LDS (bf16 rows, 16-byte chunk ^ (row % 16) for
  // D = 128, ^ ((row / 2) % 8) for D = 64); from the first row strip, the
  // largest squared norm of the strip (rows past nkb repeat the last block)
#pragma unroll
  for (int i = 0; i < KLOADS; ++i) {
    const int c = t + NT * i, bl = c / CPB, ch = c % CPB;
    bf16x4 h, l;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = kg[i][e];
      const __bf16 hb = static_cast<__bf16>(x);
      h[e] = hb;
      l[e] = static_cast<__bf16>(x - static_cast<float>(hb));
      ss = fmaf(x, x, ss);
    }
    const int sw = D == 128 ? (bl & 15) : ((bl >> 1) & 7);
    const int off = bl * RB + ((ch / 2) ^ sw) * 16 + (ch & 1) * 8;
    *reinterpret_cast<bf16x4*>(s_hi + off) = h;
    *reinterpret_cast<bf16x4*>(s_lo + off) = l;
    if (rs == 0) {
      // squared norm of the block: its CPB chunks sit in CPB consecutive
      // lanes (one or two 16-lane rows); prefix sums within each row, then
      // row 2r's total added to row 2r + 1, leave it in the block's last lane
      float v = ss;
      v += __int_as_float(dpp_i<0x111>(0, __float_as_int(v)));
      v += __int_as_float(dpp_i<0x112>(0, __float_as_int(v)));
      v += __int_as_float(dpp_i<0x114>(0, __float_as_int(v)));
      v += __int_as_float(dpp_i<0x118>(0, __float_as_int(v)));
      if constexpr (CPB == 32) v += __int_as_float(dpp_i<0x142, 0xa>(0, __float_as_int(v)));
      ssmax = fmaxf(ssmax, v);
    }
  }
  if (rs == 0) {
    static_assert(CPB == 16 || CPB == 32, "a key-block mean spans one or two 16-lane rows");
    float m2 = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ssmax), 31)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ssmax), 63)));
    if constexpr (CPB == 16)
      m2 = fmaxf(m2, fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ssmax), 15)),
                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ssmax), 47))));
    if (lane == 0) atomicMax(s_kmax, __float_as_uint(m2));   // m2 >= 0: bits order as values
  }
  __syncthreads();
  if (rs == 0 && t == 0) kmaxp[bh * cstrips + cs] = __uint_as_float(*s_kmax);

  // pairs of 32 x 32 tiles of S^T: tile u, lane l, register 4 j + e = key
  // block 32 u + 8 j + 4 (l / 32) + e of the pair, query block q0 + l % 32
  unsigned char* const os = s_out[w];
#pragma unroll 1
  for (int p = 0; p < kScrCols / 64; ++p) {
    f32x16 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int bl = 64 * p + 32 * u + lane % 32;
      const int sw = D == 128 ? (bl & 15) : ((bl >> 1) & 7);
      bf16x8 kh[KS], kl[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = bl * RB + ((2 * ks + lane / 32) ^ sw) * 16;
        kh[ks] = *reinterpret_cast<const bf16x8*>(s_hi + off);
        kl[ks] = *reinterpret_cast<const bf16x8*>(s_lo + off);
      }
      acc[u] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh[ks], a_hi[ks], acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl[ks], a_hi[ks], acc[u], 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh[ks], a_lo[ks], acc[u], 0, 0, 0);
      }
      // the LDS reads two k-steps ahead of the MFMAs that use them (left
      // alone the compiler reads each k-step just before its MFMAs and every
      // third MFMA waits out the LDS latency); 0x100 = LDS reads, 0x008 = MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int x = 0; x < KS - 2; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    }
    // patch: 32 query rows x 64 keys of float16 (128 bytes), chunk ^ (row % 8);
    // forced blocks and blocks past nkb (only in the pairs that hold any)
    // become the sentinel
    const bool edge = c0 + 64 * p < nf || c0 + 64 * p + 64 > nkb;
    {
      const int r = lane % 32;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kb0 = c0 + 64 * p + 32 * u + 8 * j + 4 * (lane / 32);
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t b = __builtin_bit_cast(uint16_t, static_cast<_Float16>(tau * acc[u][4 * j + e]));
            h[e] = (b & 0x7c00u) == 0x7c00u ? kNaN16 : b;       // inf or NaN
          }
          if (edge) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kb0 + e < nf || kb0 + e >= nkb) h[e] = kSentinel16;
          }
          const int ch = 4 * u + j;
          *reinterpret_cast<u32x2*>(os + r * 128 + (ch ^ (r & 7)) * 16 + 8 * (lane / 32)) =
              u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);         // lgkmcnt(0): the patch is written
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 64 * i + lane, r = c / 8, ch = c % 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(os + r * 128 + (ch ^ (r & 7)) * 16);
      const int iq = q0 + r;
      if (iq < nqb)
        *reinterpret_cast<u32x4*>(app + (bh * nqb + iq) * static_cast<int64_t>(ws_stride) + c0 +
                                  64 * p + 8 * ch) = v;
    }
    __builtin_amdgcn_wave_barrier();            // the patch is read before the next pair
  }
}

// ---------------------------------------------------------------------------
// B. band selection
// ---------------------------------------------------------------------------
// One wavefront per query block (row), one row per workgroup.  Lane l owns the CL consecutive blocks CL l .. CL l + CL - 1 of
// the row (keys in registers, sets of them as CL-bit masks), so counts and
// the ascending output need one prefix sum over lanes, not one per slot.
// The exact scores (of the band, and of every block on the exact route) come
// from the score kernel's fp64 sums in their one-row form (score_row16: this
// row against 16 blocks per chain).
template <int D, int CL>
// At most 96 registers (second bound: five waves per SIMD): a row is a
// latency chain, so more rows in flight shorten the kernel.
__global__ __launch_bounds__(64 * kSWaves, 5) void band_select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int64_t rows, int nqb, int nkb,
    float tau, int nf, int k, const uint16_t* __restrict__ app, const float* __restrict__ kmaxp,
    int cstrips, int ws_stride, int stride, int32_t* __restrict__ cnt, int32_t* __restrict__ idx,
    int max_kept) {
  static_assert(CL % 2 == 0 && CL <= 32, "keys per lane: even, one 32-bit mask");
  extern __shared__ float s_exact_rows[];          // [kSWaves][stride]: exact route only
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kSWaves][256 + 64];
  __shared__ float s_bandF[kSWaves][kBandCap];
  __shared__ int32_t s_bandC[kSWaves][kBandCap];
  __shared__ uint32_t s_chosen[kSWaves][64];

  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kSWaves + w;
  if (row >= rows) return;                          // uniform per wave; no workgroup barrier below
  const int64_t bh = row / nqb;
  const int i = static_cast<int>(row - bh * nqb);
  const int lr = lane % 16, lg = lane / 16;
  const float* qh = qbar + bh * static_cast<int64_t>(nqb) * D;
  const float* kh = kbar + bh * static_cast<int64_t>(nkb) * D;
  int32_t* out = idx + row * static_cast<int64_t>(max_kept);
  const double tau_d = static_cast<double>(tau);
  const int j0 = CL * lane;                         // this lane's first block

  // all loads first: the lane's screened values (CL / 2 words), the strip
  // maxima of the squared key norms, this query mean
  uint32_t wv[CL / 2];
  {
    const uint32_t* arow = reinterpret_cast<const uint32_t*>(app + row * static_cast<int64_t>(ws_stride)) +
                           (CL / 2) * lane;
#pragma unroll
    for (int s = 0; s < CL / 2; ++s) wv[s] = arow[s];
  }
  const float kmx2 = lane < cstrips ? kmaxp[bh * cstrips + lane] : 0.f;
  float qx[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) qx[e] = qh[static_cast<int64_t>(i) * D + lane + 64 * e];

  // order keys (0 = ineligible) and the largest of them
  uint32_t key[CL];
  uint32_t kbig = 0u;
#pragma unroll
  for (int s = 0; s < CL; ++s) {
    key[s] = key16((s & 1) ? (wv[s / 2] >> 16) : (wv[s / 2] & 0xffffu));
    kbig = max(kbig, key[s]);
  }
  float qss = 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) qss = fmaf(qx[e], qx[e], qss);

  kbig = wave_max_u(kbig);
  bool full_exact = kbig >= 0xfc00u;                 // a non-finite screened value
  uint32_t above_m = 0u, band_m = 0u;                // CL-bit masks of this lane's blocks
  bool exact = false;
  if (!full_exact && k > 0) {
    const float kmax = sqrtf(__uint_as_float(wave_max_u(__float_as_uint(kmx2)))) * 1.0001f;
    const float qn = sqrtf(wave_sum_f(qss)) * 1.0001f;
    const float t = value_of_key16(kth_largest16<CL>(key, k, lane, s_hist[w]));
    // |A_j - F_j| <= 1.001 (e1 + 6e-4 |A_j|) =: e(A_j); then F's k-th largest
    // lies in [t - e(t), t + e(t)], and A_j > hi (A_j < lo) puts F_j above
    // (below) that interval, because a -+ 6.006e-4 |a| increase with a
    const float e1 = 1.2e-4f * fabsf(tau) * qn * kmax + 1e-7f;
    const float X = t + 2.002f * e1 + 6.006e-4f * fabsf(t);
    const float Y = t - 2.002f * e1 - 6.006e-4f * fabsf(t);
    const float hi = X + 7e-4f * fabsf(X) + 1e-7f, lo = Y - 7e-4f * fabsf(Y) - 1e-7f;
    if (!(fabsf(lo) < INFINITY) || !(fabsf(hi) < INFINITY)) {
      full_exact = true;
    } else {
      // keys of values > hi, and of values >= lo (klo >= 0x0400 > key 0)
      const uint32_t khi = key_threshold(hi, true), klo = key_threshold(lo, false);
      uint32_t ge_m = 0u;
#pragma unroll
      for (int s = 0; s < CL; ++s) {
        above_m |= (key[s] >= khi ? 1u : 0u) << s;
        ge_m |= (key[s] >= klo ? 1u : 0u) << s;
      }
      band_m = ge_m & ~above_m;
      const int packed = wave_inclusive_scan(__popc(above_m) | (__popc(band_m) << 16));
      const int tot = __builtin_amdgcn_readlane(packed, 63);
      const int n_in = tot & 0xffff, m = tot >> 16;
      const int need = k - n_in;                     // 1 <= need <= m (the k-th lies in the band)
      exact = m > need;
      if (exact && m > kBandCap) {
        full_exact = true;
      } else if (exact) {
        // the band's blocks into LDS, each lane's in order after those of the lanes below
        int pos = ((packed >> 16) & 0xffff) - __popc(band_m);
        for (uint32_t x = band_m; x; x &= x - 1u) s_bandC[w][pos++] = j0 + __builtin_ctz(x);
        s_chosen[w][lane] = 0u;
        __builtin_amdgcn_wave_barrier();
        // exact scores of the band, 16 blocks per row chain (lane c < 16: block c0 + c)
        f32x4 qv[D / 16];
        load_operands<D>(qh + static_cast<int64_t>(i) * D + 4 * lg, qv);
        for (int c0 = 0; c0 < m; c0 += 16) {
          const int col = s_bandC[w][min(c0 + lr, m - 1)];
          f32x4 kq[D / 16];
          load_operands<D>(kh + static_cast<int64_t>(col) * D + 4 * lg, kq);
          const double acc = score_row16<D>(qv, kq);
          if (lane < 16 && c0 + lane < m) s_bandF[w][c0 + lane] = static_cast<float>(tau_d * acc);
        }
        __builtin_amdgcn_wave_barrier();
        // keep the best `need` of the band: higher F first, then the lower index
        // (lane e holds band block e; the others are broadcast from their lanes)
        const float fe = lane < m ? s_bandF[w][lane] : 0.f;
        const int ce = lane < m ? s_bandC[w][lane] : 0;
        int rank = 0;
        for (int e = 0; e < m; ++e) {
          const float f2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fe), e));
          const int c2 = __builtin_amdgcn_readlane(ce, e);
          rank += (f2 > fe || (f2 == fe && c2 < ce)) ? 1 : 0;
        }
        if (lane < m && rank < need) atomicOr(&s_chosen[w][ce / CL], 1u << (ce % CL));
        __builtin_amdgcn_wave_barrier();
        band_m = s_chosen[w][lane];
      }
    }
  }

  if (!full_exact) {
    for (int p = lane; p < nf; p += 64) out[p] = p;
    const uint32_t keep = above_m | band_m;
    const int incl = wave_inclusive_scan(__popc(keep));
    int pos = nf + incl - __popc(keep);
    for (uint32_t x = keep; x; x &= x - 1u) {
      if (pos < max_kept) out[pos] = j0 + __builtin_ctz(x);
      ++pos;
    }
    const int base = nf + __builtin_amdgcn_readlane(incl, 63);
    for (int p = base + lane; p < max_kept; p += 64) out[p] = -1;
    if (lane == 0) cnt[row] = base;
    return;
  }

  // ---- exact route for this row: every exact score, then the row selector ------
  float* srow = s_exact_rows + w * stride;
  {
    f32x4 qv[D / 16];
    load_operands<D>(qh + static_cast<int64_t>(i) * D + 4 * lg, qv);
    const int ntk = (nkb + 15) / 16;
    for (int jt = 0; jt < ntk; ++jt) {
      const int jc = 16 * jt + lr;
      f32x4 kq[D / 16];
      load_operands<D>(kh + static_cast<int64_t>(min(jc, nkb - 1)) * D + 4 * lg, kq);
      const double acc = score_row16<D>(qv, kq);   // lane c < 16: block 16 jt + c
      if (lane < 16 && jc < nkb) srow[jc] = static_cast<float>(tau_d * acc);
    }
  }
  __builtin_amdgcn_wave_barrier();
  auto key_at = [&](int j) -> uint32_t { return (j >= nf && j < nkb) ? order_key(srow[j]) : 0u; };
  // slot c of lane l = block l + 64 c (the row selector's layout)
  uint32_t ekey[CL];
  float v[CL];
#pragma unroll
  for (int c = 0; c < CL; ++c) v[c] = srow[lane + 64 * c];
#pragma unroll
  for (int c = 0; c < CL; ++c) {
    const int j = lane + 64 * c;
    ekey[c] = static_cast<unsigned>(j - nf) < static_cast<unsigned>(nkb - nf) ? order_key(v[c]) : 0u;
  }
  __builtin_amdgcn_wave_barrier();
  // the keys are in registers, so the row's slice holds the candidate keys
  const int n = select_row<CL>(ekey, key_at, lane, nkb, nf, k, reinterpret_cast<uint32_t*>(srow), out,
                               max_kept);
  if (lane == 0) cnt[row] = n;
}

// Workspace layout: screened scores [BH][nqb][ws_stride] float16 with
// ws_stride = 128 * cstrips (cstrips = ceil(nkb / 128), CL = 2 cstrips keys
// per lane), then the strip maxima of the squared key norms [BH][cstrips]
// float32 (256-byte aligned).
struct Layout {
  int cstrips, CL, ws_stride;
  int64_t kmax_off, total;
};

Layout layout_of(int64_t BH, int64_t nqb, int64_t nkb) {
  auto up256 = [](int64_t x) { return (x + 255) / 256 * 256; };
  Layout L;
  L.cstrips = static_cast<int>((nkb + kScrCols - 1) / kScrCols);
  L.CL = 2 * L.cstrips;
  L.ws_stride = kScrCols * L.cstrips;
  L.kmax_off = up256(BH * nqb * L.ws_stride * 2);
  L.total = L.kmax_off + BH * L.cstrips * 4;
  return L;
}

}  // namespace

int64_t fused_select_max_nkb() { return kMaxNkb; }

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: a fixed device array instead of
// a caller workspace.  Each GPU the library runs on holds its own copy until
// the process ends; every call on that GPU uses it, so calls that overlap in
// time on one GPU race.  Nothing in it needs to start at zero (the screening
// kernel writes every entry the band kernel reads).
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
  float* kmaxp = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.kmax_off);
  const int n = (int)nkb, nq = (int)nqb, f = (int)n_forced, kk = (int)k, mk = (int)max_kept;

  // A. screening: one workgroup per 128 x 128 tile, dealt out per XCD
  const int64_t rstrips = (nqb + kScrRows - 1) / kScrRows;
  const int64_t tiles = BH * rstrips * L.cstrips;
  if (tiles > 2147483647LL - kXcds) {
    set_error("sparstar_select_blocks_from_means: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  const int per_xcd = static_cast<int>((tiles + kXcds - 1) / kXcds);
  const dim3 sgrid(static_cast<uint32_t>(per_xcd) * kXcds), sblock(64 * kScrWaves);
  if (D == 128)
    screen_kernel<128><<<sgrid, sblock, 0, s>>>(qbar, kbar, nq, n, f, (int)rstrips, L.cstrips,
                                                (int)tiles, per_xcd, tau, L.ws_stride, app, kmaxp);
  else
    screen_kernel<64><<<sgrid, sblock, 0, s>>>(qbar, kbar, nq, n, f, (int)rstrips, L.cstrips,
                                               (int)tiles, per_xcd, tau, L.ws_stride, app, kmaxp);
  sparstar_status st = check_launch("sparstar_select_blocks_from_means");
  if (st != SPARSTAR_OK) return st;

  // B. band selection, one wavefront per query block
  const int64_t rows = BH * nqb;
  const int64_t wgs = (rows + kSWaves - 1) / kSWaves;
  if (wgs > 2147483647LL) {
    set_error("sparstar_select_blocks_from_means: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  // the exact route keeps one row of float32 scores per wavefront: every slot
  // a lane reads (64 CL of them) lies inside it, and it holds the selector's
  // 128 candidate words
  const int stride = 64 * L.CL < 128 ? 128 : 64 * L.CL;
  const size_t lds = static_cast<size_t>(kSWaves) * stride * sizeof(float);
  const dim3 grid(static_cast<uint32_t>(wgs)), block(64 * kSWaves);
  hipError_t e = hipSuccess;
#define SPARSTAR_BAND_CASE_D(DD, CC)                                                              \
  if (lds > 49152)                                                                                \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&band_select_kernel<DD, CC>),          \
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));  \
  if (e == hipSuccess)                                                                            \
    band_select_kernel<DD, CC><<<grid, block, lds, s>>>(qbar, kbar, rows, nq, n, tau, f, kk, app, \
                                                        kmaxp, L.cstrips, L.ws_stride, stride,    \
                                                        kv_count, kv_index, mk);
#define SPARSTAR_BAND_CASE(CC)         \
  case CC:                             \
    if (D == 128) {                    \
      SPARSTAR_BAND_CASE_D(128, CC)    \
    } else {                           \
      SPARSTAR_BAND_CASE_D(64, CC)     \
    }                                  \
    break;
  switch (L.CL) {
    SPARSTAR_BAND_CASE(2) SPARSTAR_BAND_CASE(4) SPARSTAR_BAND_CASE(6) SPARSTAR_BAND_CASE(8)
    SPARSTAR_BAND_CASE(10) SPARSTAR_BAND_CASE(12) SPARSTAR_BAND_CASE(14) SPARSTAR_BAND_CASE(16)
    SPARSTAR_BAND_CASE(18) SPARSTAR_BAND_CASE(20) SPARSTAR_BAND_CASE(22) SPARSTAR_BAND_CASE(24)
    SPARSTAR_BAND_CASE(26) SPARSTAR_BAND_CASE(28) SPARSTAR_BAND_CASE(30) SPARSTAR_BAND_CASE(32)
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
