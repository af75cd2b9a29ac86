// Shared host/device helpers of the SparSTAR HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/sparstar.h"

namespace sparstar {

// ---------------------------------------------------------------------------
// Host-side error reporting (thread-local message, see sparstar_last_error).
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);
void clear_error();

// Kernel launchers (one per source file).  Each returns SPARSTAR_OK or
// SPARSTAR_ERR_HIP after checking hipGetLastError; arguments are validated
// by the callers in api.hip.
sparstar_status launch_block_means(const void* x, sparstar_dtype dt, int64_t BH, int64_t N,
                                   int64_t D, int64_t block, float* out, hipStream_t s);
sparstar_status launch_block_scores(const float* qbar, const float* kbar, int64_t BH,
                                    int64_t nqb, int64_t nkb, int64_t D, float tau, float* S,
                                    hipStream_t s);
sparstar_status launch_select_blocks(const float* S, int64_t rows, int64_t nkb, int64_t n_forced,
                                     int64_t k, int32_t* kv_count, int32_t* kv_index,
                                     int64_t max_kept, hipStream_t s);
sparstar_status launch_scores_select(const float* qbar, const float* kbar, int64_t BH,
                                     int64_t nqb, int64_t nkb, int64_t D, float tau,
                                     int64_t n_forced, int64_t k, int32_t* kv_count,
                                     int32_t* kv_index, int64_t max_kept, void* workspace,
                                     hipStream_t s);
// Largest nkb the screened score + selection route takes (a row lives in registers).
int64_t fused_select_max_nkb();
// Workspace bytes of the screened route for BH heads of nqb x nkb blocks.
int64_t select_workspace_bytes(int64_t BH, int64_t nqb, int64_t nkb);
// The allocation-free route's device scratch: its size, and its address on
// the current device (looked up once per device).
int64_t select_scratch_bytes();
sparstar_status select_scratch_pointer(void** out);
sparstar_status launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t block,
                                     const int32_t* kv_count, const int32_t* kv_index,
                                     int64_t max_kept, float scale, uint16_t* o, float* lse,
                                     hipStream_t s);
sparstar_status launch_attn_fwd_f32(const float* q, const float* k, const float* v, int64_t BH,
                                    int64_t Nq, int64_t Nk, int64_t D, int64_t block,
                                    const int32_t* kv_count,
                                    const int32_t* kv_index, int64_t max_kept, float scale,
                                    float* o, float* lse, hipStream_t s);

sparstar_status launch_retained_mass(const float* lse_sel, const float* lse_dense, int64_t n,
                                     float* mass, hipStream_t s);

sparstar_status launch_transfer_scores(const float* S_src, int64_t BH, int64_t block,
                                       const int64_t src_geom[3], const int64_t dst_geom[3],
                                       float* S_dst, hipStream_t s);

sparstar_status launch_token_topk_bound(const uint16_t* q, const uint16_t* k, int64_t BH, int64_t Nq,
                                        int64_t Nk, int64_t D, int64_t f_tok, int64_t m_tok,
                                        float scale, float* bound, hipStream_t s);

sparstar_status check_launch(const char* what);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
// Block sizes (tokens) the kernels are instantiated for; 128 is the pages'.
inline bool block_supported(int64_t b) { return b == 32 || b == 64 || b == 128; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

}  // namespace sparstar
