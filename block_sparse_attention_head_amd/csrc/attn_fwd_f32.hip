// Block-sparse forward attention, float32 inputs (plain VALU arithmetic).
//
// Same operation as the bf16 MFMA kernel (forward attention over the kept
// key blocks of each query block, SparSTAR review "What carries the
// argument"), for float32 workloads where exact float32 products are wanted.
// One workgroup per (b*h, query block): 2 * kBlock threads, two per query, each
// owning half of the head dimension of q and of the output.  Key/value tiles
// of 32 tokens are staged through LDS; the softmax is the usual online
// (running max and sum) form.
#include <cmath>

#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kTileK = 32;

template <int D, int kBlock>
__global__ __launch_bounds__(2 * kBlock) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    int Nq, int Nk, int nqb, const int32_t* __restrict__ kv_count,
    const int32_t* __restrict__ kv_index, int max_kept, float scale_log2, float* __restrict__ o,
    float* __restrict__ lse) {
  constexpr int DH = D / 2;
  constexpr int kThreads = 2 * kBlock;
  __shared__ float ks[kTileK][D];
  __shared__ float vs[kTileK][D];

  const int64_t row = blockIdx.x;  // (bh, i)
  const int64_t bh = row / nqb;
  const int i = static_cast<int>(row - bh * nqb);
  const int t = threadIdx.x;
  const int qi = t >> 1, half = t & 1;
  const int tok = i * kBlock + qi;
  const bool qvalid = tok < Nq;
  const int nkb = (Nk + kBlock - 1) / kBlock;

  float qr[DH], acc[DH];
  const float* qp = q + (bh * Nq + (qvalid ? tok : 0)) * static_cast<int64_t>(D) + half * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qr[d] = qvalid ? qp[d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int count = kv_count[row];
  count = count < 0 ? 0 : (count > max_kept ? max_kept : count);
  const int32_t* list = kv_index + row * static_cast<int64_t>(max_kept);
  const float* kh = k + bh * static_cast<int64_t>(Nk) * D;
  const float* vh = v + bh * static_cast<int64_t>(Nk) * D;

  for (int e = 0; e < count; ++e) {
    const int j = list[e];
    if (j < 0 || j >= nkb) continue;  // uniform: skipped entries cost nothing
    for (int sub = 0; sub < kBlock / kTileK; ++sub) {
      const int key0 = j * kBlock + sub * kTileK;
      const int nvalid = min(kTileK, Nk - key0);
      if (nvalid <= 0) break;
      __syncthreads();
      for (int x = t; x < kTileK * D; x += kThreads) {
        const int r = x / D, c = x % D;
        const bool ok = r < nvalid;
        ks[r][c] = ok ? kh[static_cast<int64_t>(key0 + r) * D + c] : 0.f;
        vs[r][c] = ok ? vh[static_cast<int64_t>(key0 + r) * D + c] : 0.f;
      }
      __syncthreads();
      float s[kTileK];
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < kTileK; ++r) {
        float p = 0.f;
#pragma unroll
        for (int d = 0; d < DH; ++d) p = fmaf(qr[d], ks[r][half * DH + d], p);
        p += __shfl_xor(p, 1);
        s[r] = (r < nvalid) ? p * scale_log2 : -INFINITY;
        mt = fmaxf(mt, s[r]);
      }
      const float mn = fmaxf(m, mt);
      const float alpha = exp2f(m - mn);  // m = -inf at start -> 0
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < kTileK; ++r) {
        s[r] = exp2f(s[r] - mn);
        ls += s[r];
      }
      l = l * alpha + ls;
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        float a = acc[d] * alpha;
#pragma unroll
        for (int r = 0; r < kTileK; ++r) a = fmaf(s[r], vs[r][half * DH + d], a);
        acc[d] = a;
      }
      m = mn;
    }
  }

  if (qvalid) {
    float* op = o + (bh * Nq + tok) * static_cast<int64_t>(D) + half * DH;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) op[d] = acc[d] * inv;
    if (lse && half == 0)
      lse[bh * Nq + tok] = l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int B>
sparstar_status launch_b(const float* q, const float* k, const float* v, int64_t BH, int64_t Nq,
                         int64_t Nk, int64_t D, const int32_t* kv_count, const int32_t* kv_index,
                         int64_t max_kept, float scale, float* o, float* lse, hipStream_t s) {
  const int64_t nqb = (Nq + B - 1) / B;
  const dim3 grid(static_cast<uint32_t>(BH * nqb)), block(2 * B);
  const float sl2 = scale * 1.4426950408889634f;
  if (D == 128)
    attn_fwd_f32_kernel<128, B><<<grid, block, 0, s>>>(q, k, v, (int)Nq, (int)Nk, (int)nqb, kv_count,
                                                       kv_index, (int)max_kept, sl2, o, lse);
  else
    attn_fwd_f32_kernel<64, B><<<grid, block, 0, s>>>(q, k, v, (int)Nq, (int)Nk, (int)nqb, kv_count,
                                                      kv_index, (int)max_kept, sl2, o, lse);
  return check_launch("sparstar_block_sparse_attn_fwd");
}

}  // namespace

sparstar_status launch_attn_fwd_f32(const float* q, const float* k, const float* v, int64_t BH,
                                    int64_t Nq, int64_t Nk, int64_t D, int64_t block,
                                    const int32_t* kv_count, const int32_t* kv_index,
                                    int64_t max_kept, float scale, float* o, float* lse,
                                    hipStream_t s) {
  if (block == 32)
    return launch_b<32>(q, k, v, BH, Nq, Nk, D, kv_count, kv_index, max_kept, scale, o, lse, s);
  if (block == 64)
    return launch_b<64>(q, k, v, BH, Nq, Nk, D, kv_count, kv_index, max_kept, scale, o, lse, s);
  return launch_b<128>(q, k, v, BH, Nq, Nk, D, kv_count, kv_index, max_kept, scale, o, lse, s);
}

}  // namespace sparstar
