// Block means of Q or K over contiguous blocks of kBlock tokens (SparSTAR
// review, "What carries the argument": queries and keys are averaged per
// block of 128 tokens; 32 and 64 are instantiated as well).
//
// One workgroup of 256 threads per (b*h, block): the kBlock x D slab is one
// contiguous chunk of HBM, read once with 16-byte loads by consecutive
// threads (fully coalesced).  Each thread sums its rows column-wise in
// registers; the per-thread partials meet in LDS as float64 and are added in
// a fixed order, so the result is the float32 rounding of the (nearly exact)
// mean.  A partial last block divides by its own token count.
#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kThreads = 256;

template <int D, bool kBf16, int kBlock>
__global__ __launch_bounds__(kThreads) void block_means_kernel(const void* __restrict__ xv,
                                                               int N, int nb,
                                                               float* __restrict__ out) {
  constexpr int VEC = kBf16 ? 8 : 4;        // elements per 16-byte load
  constexpr int CPR = D / VEC;              // 16-byte chunks per token row
  constexpr int G = kThreads / CPR;         // row groups
  constexpr int RPT = kBlock / G;           // rows per thread
  __shared__ double part[G][D];

  const int64_t blk = blockIdx.x;           // (bh, i) flattened
  const int64_t bh = blk / nb;
  const int i = static_cast<int>(blk - bh * nb);
  const int t = threadIdx.x;
  const int c = t % CPR, g = t / CPR;
  const int row0 = i * kBlock;
  const int nvalid = min(kBlock, N - row0);

  const u32x4* base = reinterpret_cast<const u32x4*>(
      static_cast<const char*>(xv) +
      ((bh * N + row0) * static_cast<int64_t>(D)) * (kBf16 ? 2 : 4));

  u32x4 raw[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = g + G * m;
    raw[m] = (r < nvalid) ? __builtin_nontemporal_load(base + r * CPR + c) : u32x4{0, 0, 0, 0};
  }

  if constexpr (kBf16) {
    // Sums of <= 8 bf16 values in float32 are exact unless their exponents
    // span more than ~13 binades.
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const uint32_t w[4] = {raw[m].x, raw[m].y, raw[m].z, raw[m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) part[g][c * VEC + e] = static_cast<double>(acc[e]);
  } else {
    double acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      acc[0] += static_cast<double>(__uint_as_float(raw[m].x));
      acc[1] += static_cast<double>(__uint_as_float(raw[m].y));
      acc[2] += static_cast<double>(__uint_as_float(raw[m].z));
      acc[3] += static_cast<double>(__uint_as_float(raw[m].w));
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) part[g][c * VEC + e] = acc[e];
  }
  __syncthreads();
  if (t < D) {
    double s = 0.0;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) s += part[gg][t];
    out[(bh * nb + i) * D + t] = static_cast<float>(s / static_cast<double>(nvalid));
  }
}

template <int B>
sparstar_status launch_b(const void* x, sparstar_dtype dt, int64_t BH, int64_t N, int64_t D,
                         float* out, hipStream_t s) {
  const int64_t nb = (N + B - 1) / B;
  if (BH * nb > 2147483647LL) {
    set_error("sparstar_block_means: B*H*nblocks exceeds the grid limit");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  const dim3 grid(static_cast<uint32_t>(BH * nb)), block(kThreads);
  const int n = static_cast<int>(N), nbi = static_cast<int>(nb);
  if (dt == SPARSTAR_BF16) {
    if (D == 128) block_means_kernel<128, true, B><<<grid, block, 0, s>>>(x, n, nbi, out);
    else block_means_kernel<64, true, B><<<grid, block, 0, s>>>(x, n, nbi, out);
  } else {
    if (D == 128) block_means_kernel<128, false, B><<<grid, block, 0, s>>>(x, n, nbi, out);
    else block_means_kernel<64, false, B><<<grid, block, 0, s>>>(x, n, nbi, out);
  }
  return check_launch("sparstar_block_means");
}

}  // namespace

sparstar_status launch_block_means(const void* x, sparstar_dtype dt, int64_t BH, int64_t N,
                                   int64_t D, int64_t block, float* out, hipStream_t s) {
  if (block == 32) return launch_b<32>(x, dt, BH, N, D, out, s);
  if (block == 64) return launch_b<64>(x, dt, BH, N, D, out, s);
  return launch_b<128>(x, dt, BH, N, D, out, s);
}

}  // namespace sparstar
