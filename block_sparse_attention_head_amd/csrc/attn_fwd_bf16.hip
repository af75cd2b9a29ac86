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
//    buffered: the next tile's global loads are issued before the current
//    tile's MFMAs and written to the other buffer afterwards; one barrier per
//    tile.  LDS rows are padded by 16 bytes so the MFMA operand reads below
//    are bank-conflict free.
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

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ float partner_lane32(float x) {
  // v_permlane32_swap(x, x): lanes < 32 receive [x[l], x[l+32]], lanes >= 32
  // receive [x[l-32], x[l]]; pick the other half's value.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int Nq, int Nk, int nqb,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_index, int max_kept,
    float sl2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int LD = D + 8;            // padded LDS row, elements
  constexpr int KSTEPS = D / 16;       // MFMA k-steps over d for S^T
  constexpr int DT = D / 32;           // 32-row d tiles of O^T
  constexpr int CPR = D / 8;           // 16-byte chunks per token row
  constexpr int LPT = kBK * CPR / kThreads;  // 16-byte loads per thread per tensor
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kBK * LD];

  const int64_t row = blockIdx.x;      // (bh, i), head-major
  const int64_t bh = row / nqb;
  const int i = static_cast<int>(row - bh * nqb);
  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64, h = l / 32, n = l % 32;
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

  u32x4 kreg[LPT], vreg[LPT];
  auto load_tile = [&](int t) {
    int key0;
    const int nv = tile_keys(t, key0);
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int ch = tid + kThreads * m;
      const int r = ch / CPR, c = ch % CPR;
      if (r < nv) {
        const int64_t off = static_cast<int64_t>(key0 + r) * D + 8 * c;
        kreg[m] = *reinterpret_cast<const u32x4*>(kh + off);
        vreg[m] = *reinterpret_cast<const u32x4*>(vh + off);
      } else {
        kreg[m] = u32x4{0, 0, 0, 0};
        vreg[m] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int m = 0; m < LPT; ++m) {
      const int ch = tid + kThreads * m;
      const int r = ch / CPR, c = ch % CPR;
      *reinterpret_cast<u32x4*>(&lds[buf][0][r * LD + 8 * c]) = kreg[m];
      *reinterpret_cast<u32x4*>(&lds[buf][1][r * LD + 8 * c]) = vreg[m];
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    int key0;
    const int nv = tile_keys(t, key0);
    if (t + 1 < ntiles) load_tile(t + 1);

    if (nv > 0) {
      const uint16_t* Kl = lds[buf][0];
      const uint16_t* Vl = lds[buf][1];
      // ---- S^T = K Q^T : two 32-key sub-tiles --------------------------------
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kl + (32 * kt + n) * LD + 16 * ks + 8 * h);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], sacc[kt], 0, 0, 0);
        }
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
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], sl2, -m_use));
          sacc[kt][r] = p;
          ls += p;
        }
      l_run = l_run * alpha + ls;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      m_run = m_new;
      // ---- O^T += V^T P^T ---------------------------------------------------
      const int g = l / 16, L = l % 16;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kt = c / 2, r0 = 8 * (c % 2);
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(sacc[kt][r0 + e]);
        const int key_base = 32 * kt + 16 * (c % 2) + 4 * h;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int dbase = 32 * dt + 16 * (g % 2);
          const uint16_t* p1 = Vl + (key_base + L / 4) * LD + dbase + 4 * (L % 4);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1 + 8 * LD));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[dt], 0, 0, 0);
        }
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
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
        u32x2 pk;
        pk[0] = static_cast<uint32_t>(f32_to_bf16(oacc[dt][4 * r4 + 0] * inv)) |
                (static_cast<uint32_t>(f32_to_bf16(oacc[dt][4 * r4 + 1] * inv)) << 16);
        pk[1] = static_cast<uint32_t>(f32_to_bf16(oacc[dt][4 * r4 + 2] * inv)) |
                (static_cast<uint32_t>(f32_to_bf16(oacc[dt][4 * r4 + 3] * inv)) << 16);
        *reinterpret_cast<u32x2*>(op + d) = pk;
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
