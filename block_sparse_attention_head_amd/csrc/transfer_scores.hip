// Score transfer between scales: the mask-reuse baseline (SparSTAR review,
// "Extended reading notes" / "Core claim": a selection carried over from
// another scale or across a clip boundary; abstract: the analyses set a
// carried-over selection against one computed anew per scale).
//
// S_dst[bh, i, j] = S_src[bh, qmap(i), kmap(j)].  A block stands for the
// centre of its valid tokens; doubled, that centre is the integer
// C2 = first + last + 1 = b*j + min(b*j + b, n).  The segment holding it
// (2*start <= C2 < 2*(start + len)) is mapped by relative position onto the
// same segment of the source scale:
//   token = start_src + floor((C2 - 2*start_dst) * len_src / (2*len_dst)),
// exact in int64 (scales stay below 2^30 tokens, so the numerator stays below
// 2^61), and token / b is the block.
// The query map is the same with the current segment alone.
//
// Memory-bound gather: each workgroup takes 256 target columns and kRows
// target rows of one head; the key map is computed once per column (one lane
// each) and the query map once per row (into LDS), then reused; writes are
// coalesced, reads follow the key map (non-decreasing, so neighbouring lanes
// read neighbouring or equal addresses).
#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kRows = 32;

// floor(num / den) for 0 <= num < 2^62, 0 < den < 2^32: a double-precision
// estimate (off by at most one: each of the two conversions and the division
// is correctly rounded, a relative error below 2^-51 of a quotient below
// 2^31) corrected with exact integer products.
__device__ __forceinline__ int64_t floor_div(int64_t num, int64_t den) {
  int64_t t = static_cast<int64_t>(static_cast<double>(num) / static_cast<double>(den));
  if (t * den > num) --t;
  else if ((t + 1) * den <= num) ++t;
  return t;
}

struct SegMap {
  int64_t dst_start[3], dst_len[3], src_start[3], src_len[3];
  int64_t dst_n;
};

__device__ __forceinline__ int64_t doubled_centre(int64_t j, int64_t block, int64_t n) {
  const int64_t end = (j + 1) * block < n ? (j + 1) * block : n;
  return j * block + end;
}

__global__ __launch_bounds__(256) void transfer_scores_kernel(
    const float* __restrict__ S_src, int64_t nqb_src, int64_t nkb_src, int64_t nqb_dst,
    int64_t nkb_dst, int64_t block, int log2_block, int64_t src_ncur, int64_t dst_ncur, SegMap m,
    int64_t col_chunks, int64_t row_groups, float* __restrict__ S_dst) {
  const int64_t p = blockIdx.x;
  const int64_t chunk = p % col_chunks;
  const int64_t rg = (p / col_chunks) % row_groups;
  const int64_t bh = p / (col_chunks * row_groups);
  // source query block of each of this workgroup's target rows, once
  __shared__ int32_t qsrc[kRows];
  if (threadIdx.x < kRows) {
    const int64_t i = rg * kRows + threadIdx.x;
    qsrc[threadIdx.x] = i < nqb_dst ? static_cast<int32_t>(
        floor_div(doubled_centre(i, block, dst_ncur) * src_ncur, 2 * dst_ncur) >> log2_block) : 0;
  }
  __syncthreads();
  const int64_t j = chunk * 256 + threadIdx.x;
  if (j >= nkb_dst) return;
  const int64_t c2 = doubled_centre(j, block, m.dst_n);
  int64_t tok = 0;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int64_t lo = 2 * m.dst_start[s], hi = 2 * (m.dst_start[s] + m.dst_len[s]);
    if (c2 >= lo && c2 < hi)
      tok = m.src_start[s] + floor_div((c2 - lo) * m.src_len[s], 2 * m.dst_len[s]);
  }
  const int64_t kj = tok >> log2_block;
  const float* src_head = S_src + bh * nqb_src * nkb_src;
  float* dst_head = S_dst + bh * nqb_dst * nkb_dst;
  const int rows = static_cast<int>(nqb_dst - rg * kRows < kRows ? nqb_dst - rg * kRows : kRows);
#pragma unroll 8
  for (int r = 0; r < rows; ++r) {
    const int64_t i = rg * kRows + r;
    dst_head[i * nkb_dst + j] = src_head[qsrc[r] * nkb_src + kj];
  }
}

}  // namespace

sparstar_status launch_transfer_scores(const float* S_src, int64_t BH, int64_t block,
                                       const int64_t src_geom[3], const int64_t dst_geom[3],
                                       float* S_dst, hipStream_t s) {
  SegMap m;
  int64_t a = 0, b = 0;
  for (int k = 0; k < 3; ++k) {
    m.dst_start[k] = a;
    m.dst_len[k] = dst_geom[k];
    m.src_start[k] = b;
    m.src_len[k] = src_geom[k];
    a += dst_geom[k];
    b += src_geom[k];
  }
  m.dst_n = a;
  const int64_t nqb_src = (src_geom[2] + block - 1) / block, nkb_src = (b + block - 1) / block;
  const int64_t nqb_dst = (dst_geom[2] + block - 1) / block, nkb_dst = (a + block - 1) / block;
  const int64_t col_chunks = (nkb_dst + 255) / 256, row_groups = (nqb_dst + kRows - 1) / kRows;
  const int64_t blocks = BH * row_groups * col_chunks;
  if (blocks > 2147483647LL) {
    set_error("sparstar_transfer_scores: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  transfer_scores_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s>>>(
      S_src, nqb_src, nkb_src, nqb_dst, nkb_dst, block, block == 32 ? 5 : (block == 64 ? 6 : 7),
      src_geom[2], dst_geom[2], m, col_chunks,
      row_groups, S_dst);
  return check_launch("sparstar_transfer_scores");
}

}  // namespace sparstar
