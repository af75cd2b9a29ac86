// Pieces shared by the kernels that stream K (and V) tiles through LDS and
// compute S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (attention forward and
// the token-wise Top-K bound): lane exchange, the LDS row swizzle, the
// scheduling of LDS-fed MFMA chains, and small constants.
#pragma once

#include "common.hpp"

namespace sparstar {
namespace {

constexpr int kXcds = 8;                   // XCDs of an MI355X; workgroups go round-robin
constexpr uint32_t kBufferRsrcWord3 = 0x00020000u;  // raw buffer descriptor, gfx9 family

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Byte offset of token row `row` inside one head's K or V slab, as a buffer
// load takes it: an unsigned 32-bit value passed through an int argument.
// The API admits N * D < 2^31 per head, so a bf16 slab holds fewer than
// 2^32 bytes and the unsigned product cannot wrap (a signed one would from
// row 2^31 / (2 D) on).
__device__ __forceinline__ int row_offset_bytes(int row, int row_bytes) {
  return static_cast<int>(static_cast<uint32_t>(row) * static_cast<uint32_t>(row_bytes));
}

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

// Scheduling of an MFMA chain fed from LDS: N MFMAs, each consuming DSPER
// LDS reads, with the reads kept AHEAD MFMAs in front (instruction-group
// barriers: 0x100 = LDS reads, 0x008 = MFMAs).  Left to itself the compiler
// issues the K reads only one or two MFMAs ahead, so each MFMA waits for
// the LDS latency; reading further ahead costs a few registers and removes
// most of those waits (the arithmetic and its order are unchanged).
template <int R, int DSPER>
__device__ __forceinline__ void mfma_ds_interleave() {
  if constexpr (R > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, DSPER, 0);
    mfma_ds_interleave<R - 1, DSPER>();
  }
}
template <int AHEAD, int N, int DSPER>
__device__ __forceinline__ void schedule_mfma_chain() {
  constexpr int A = AHEAD < N ? AHEAD : N;
  __builtin_amdgcn_sched_group_barrier(0x100, A * DSPER, 0);
  mfma_ds_interleave<N - A, DSPER>();
  __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
}

}  // namespace
}  // namespace sparstar
