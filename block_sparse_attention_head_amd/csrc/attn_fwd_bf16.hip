// Block-sparse flash-attention forward for bf16 on gfx950 MFMA.
//
// Operation (SparSTAR review, "What carries the argument"): each query block
// attends only to the key blocks its forward index list names; the softmax
// runs over the valid keys of those blocks.
//
// Design (gfx950, wave64):
//  * One workgroup per (b*h, query block) = 128 queries, 4 waves x 32
//    queries.  Every row keeps the same number of blocks, so the grid is
//    evenly loaded; workgroups are numbered head-major so the ones resident
//    together walk the same head's K/V (which then stays in L2 / MALL).
//  * Key tiles of 64 tokens (half a selected block) go through LDS, double
//    buffered.  The next tile is fetched with gfx950's direct-to-LDS loads
//    (global_load_lds_dwordx4: no staging registers) while the current one is
//    computed; one barrier per tile.  LDS rows are unpadded and their 16-byte
//    chunks XOR-swizzled per row, which keeps both LDS read patterns below
//    free of bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in registers).
//    The output layout then gives every lane ONE query and 16 keys of a
//    32-key tile, so the running max / sum / rescale of the online softmax
//    are per-lane scalars; only one exchange between lane l and l^32 per
//    tile is needed (v_permlane32_swap).
//  * The output is accumulated transposed too, O^T += V^T P^T: P (bf16) is
//    the B operand straight from the score registers (the MFMA k index is
//    permuted to match the score layout), and V^T is read from the natural
//    [key][d] LDS tile with ds_read_b64_tr_b16, gfx950's transposing LDS
//    load, using the same key permutation.
//  * Keys past Nk (partial last block) are zero-filled on load and masked to
//    -inf before the softmax.  Index entries outside [0, nkb) are skipped.
#include <cmath>

#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;  // keys per LDS tile
#ifndef SPARSTAR_ATTN_WAVES_PER_EU
#define SPARSTAR_ATTN_WAVES_PER_EU 2
#endif
// The running max only moves when a tile's max exceeds it by more than this
// many log2 units; until then probabilities are taken against the old max
// (so they stay below 2^8) and the output needs no rescale.
constexpr float kRescaleSlack = 8.f;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

__device__ __forceinline__ float partner_lane32(float x) {
  // v_permlane32_swap(x, x): lanes < 32 receive [x[l], x[l+32]], lanes >= 32
  // receive [x[l-32], x[l]]; pick the other half's value.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// XOR swizzle of the 16-byte chunk index of LDS row r.  Chosen so that
//  (a) 16 consecutive rows reading the same chunk (the K operand reads) hit
//      16 different bank groups, and
//  (b) 4 consecutive rows reading 2 or 4 adjacent chunks (the transposing V
//      reads) never share a bank group.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);   // 16 chunks per row
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);                // 8 chunks, 2 rows per 256 B
}

template <int D>
__global__ __launch_bounds__(kThreads, SPARSTAR_ATTN_WAVES_PER_EU) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int Nq, int Nk, int nqb,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_index, int max_kept,
    float sl2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int ROWB = 2 * D;                 // bytes per token row
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILEB = kBK * ROWB;           // bytes per K (or V) tile
  constexpr int RPI = 1024 / ROWB;            // rows per 1 KB wave-wide DMA instruction
  constexpr int DMA_PER_WAVE = TILEB / 1024 / (kThreads / 64);
  constexpr int KSTEPS = D / 16;              // MFMA k-steps over d for S^T
  constexpr int DT = D / 32;                  // 32-row d tiles of O^T
  __shared__ __attribute__((aligned(1024))) char lds[2][2][TILEB];  // [buffer][K, V]

  const int64_t row = blockIdx.x;             // (bh, i), head-major
  const int64_t bh = row / nqb;
  const int i = static_cast<int>(row - bh * nqb);
  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64, h = l / 32, n = l % 32;
  const int g = l / 16, L = l % 16;
  const int nkb = (Nk + kBlock - 1) / kBlock;
  const int tok = i * kBlock + 32 * w + n;
  const bool qvalid = tok < Nq;

  // Q as the B operand of S^T = K Q^T: lane l holds query n, d = 16*ks + 8*h + [0, 8).
  bf16x8 qop[KSTEPS];
  {
    const uint16_t* qp = q + (bh * Nq + (qvalid ? tok : 0)) * static_cast<int64_t>(D) + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 x = qvalid ? *reinterpret_cast<const u32x4*>(qp + 16 * ks) : u32x4{0, 0, 0, 0};
      qop[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  int count = kv_count[row];
  count = count < 0 ? 0 : (count > max_kept ? max_kept : count);
  const int32_t* list = kv_index + row * static_cast<int64_t>(max_kept);
  const uint16_t* kh = k + bh * static_cast<int64_t>(Nk) * D;
  const uint16_t* vh = v + bh * static_cast<int64_t>(Nk) * D;
  const int ntiles = 2 * count;

  // valid keys in tile t (0 if its block index is out of range)
  auto tile_keys = [&](int t, int& key0) -> int {
    const int j = list[t >> 1];
    key0 = j * kBlock + (t & 1) * kBK;
    if (j < 0 || j >= nkb) return 0;
    return min(kBK, Nk - key0);
  };

  // Direct-to-LDS fetch of tile t into buffer buf.  Wave w's m-th DMA fills
  // 1 KB of LDS = rows [RPI*u, RPI*u + RPI), u = 4*m + w; lane i lands in
  // LDS slot i % CPR of row RPI*u + i / CPR and so fetches global chunk
  // (slot ^ swizzle(row)).  Rows past Nk re-read row Nk-1: finite values
  // whose scores are masked to -inf below.
  auto fetch_tile = [&](int t, int buf) {
    int key0;
    const int nv = tile_keys(t, key0);
    if (nv <= 0) return;
#pragma unroll
    for (int m = 0; m < DMA_PER_WAVE; ++m) {
      const int u = 4 * m + w;
      const int r = RPI * u + l / CPR;
      const int c = (l % CPR) ^ chunk_swizzle<D>(r);
      const int64_t off = static_cast<int64_t>(min(key0 + r, Nk - 1)) * D + 8 * c;
      __builtin_amdgcn_global_load_lds((const global_void*)(kh + off),
                                       (lds_void*)(&lds[buf][0][1024 * u]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const global_void*)(vh + off),
                                       (lds_void*)(&lds[buf][1][1024 * u]), 16, 0, 0);
    }
  };

  // per-lane LDS byte offsets of the operand reads (buffer-relative)
  int koff[KSTEPS];                 // K operand: row n, chunk 2*ks + h
  {
    const int sw = chunk_swizzle<D>(n);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) koff[ks] = n * ROWB + 16 * ((2 * ks + h) ^ sw);
  }
  int voff[2][DT];                  // V^T operand (transposing read), lo/hi key quad
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int r = 4 * h + 8 * hi + L / 4;      // row within a 16-key step
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int chunk = 4 * dt + 2 * (g % 2) + (L % 4) / 2;
      voff[hi][dt] = r * ROWB + 16 * (chunk ^ chunk_swizzle<D>(r)) + 8 * (L % 2);
    }
  }

  if (ntiles > 0) {
    fetch_tile(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    int key0;
    const int nv = tile_keys(t, key0);
    if (t + 1 < ntiles) fetch_tile(t + 1, buf ^ 1);

    if (nv > 0) {
      const char* Kl = lds[buf][0];
      const char* Vl = lds[buf][1];
      // ---- S^T = K Q^T : two 32-key sub-tiles --------------------------------
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 a[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          a[ks] = *reinterpret_cast<const bf16x8*>(Kl + 32 * kt * ROWB + koff[ks]);
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qop[ks], sacc[kt], 0, 0, 0);
      }
      // sacc[kt][r] = S(key 32*kt + (r%4) + 8*(r/4) + 4*h, query n)
      if (nv < kBK) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kt + (r % 4) + 8 * (r / 4) + 4 * h >= nv) sacc[kt][r] = -INFINITY;
      }
      // ---- online softmax (per lane = per query) ------------------------------
      float mx = sacc[0][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
      mx = fmaxf(mx, partner_lane32(mx));
      const float mt = mx * sl2;  // tile max, log2 units
      const bool grow = mt > m_run + kRescaleSlack;  // true on the first non-empty tile
      if (__ballot(grow)) {
        const float m_new = grow ? mt : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], sl2, -m_use));
          sacc[kt][r] = p;
          ls += p;
        }
      l_run += ls;
      // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kt = c / 2, r0 = 8 * (c % 2);
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(sacc[kt][r0 + e]);
        const char* vbase = Vl + 16 * c * ROWB;   // keys [16c, 16c + 16)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + voff[0][dt]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + voff[1][dt]));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[dt], 0, 0, 0);
        }
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA for tile t+1 landed
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE ----------------------------------------------
  const float l_tot = l_run + partner_lane32(l_run);
  if (qvalid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = o + (bh * Nq + tok) * static_cast<int64_t>(D);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * h;
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = static_cast<__bf16>(oacc[dt][4 * r4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + d) = pk;
      }
    if (lse && h == 0)
      lse[bh * Nq + tok] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

sparstar_status launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     int64_t BH, int64_t Nq, int64_t Nk, int64_t D,
                                     const int32_t* kv_count, const int32_t* kv_index,
                                     int64_t max_kept, float scale, uint16_t* o, float* lse,
                                     hipStream_t s) {
  const int64_t nqb = (Nq + kBlock - 1) / kBlock;
  const dim3 grid(static_cast<uint32_t>(BH * nqb)), block(kThreads);
  const float sl2 = scale * 1.4426950408889634f;
  if (D == 128)
    attn_fwd_bf16_kernel<128><<<grid, block, 0, s>>>(q, k, v, (int)Nq, (int)Nk, (int)nqb,
                                                     kv_count, kv_index, (int)max_kept, sl2, o, lse);
  else
    attn_fwd_bf16_kernel<64><<<grid, block, 0, s>>>(q, k, v, (int)Nq, (int)Nk, (int)nqb,
                                                    kv_count, kv_index, (int)max_kept, sl2, o, lse);
  return check_launch("sparstar_block_sparse_attn_fwd");
}

}  // namespace sparstar
