// C ABI of the SparSTAR hot path: argument checks, then one launcher call.
// Every check happens before anything is enqueued, so a failed call writes
// nothing.  The operations are defined in include/sparstar.h.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "common.hpp"

namespace sparstar {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

sparstar_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return SPARSTAR_ERR_HIP;
  }
  return SPARSTAR_OK;
}

}  // namespace sparstar

using namespace sparstar;

namespace {

constexpr int64_t kMaxI32 = 2147483647LL;

sparstar_status invalid(const char* fn, const char* msg) {
  set_error("%s: %s", fn, msg);
  return SPARSTAR_ERR_INVALID_ARGUMENT;
}

sparstar_status unsupported(const char* fn, const char* msg) {
  set_error("%s: %s", fn, msg);
  return SPARSTAR_ERR_UNSUPPORTED;
}

// Common shape checks for a [B,H,N,D] tensor handled per (b,h) slice.
sparstar_status check_bhnd(const char* fn, int64_t B, int64_t H, int64_t N, int64_t D) {
  if (B < 1 || H < 1) return invalid(fn, "B and H must be >= 1");
  if (N < 1) return invalid(fn, "sequence length must be >= 1");
  if (D < 1) return invalid(fn, "D must be >= 1");
  if (D != 64 && D != 128) return unsupported(fn, "D must be 64 or 128");
  if (B > kMaxI32 / H) return invalid(fn, "B*H too large");
  if (N > kMaxI32 / D) return invalid(fn, "N*D per head must fit in int32");
  return SPARSTAR_OK;
}

sparstar_status check_block(const char* fn, int64_t block) {
  if (block < 1) return invalid(fn, "block must be >= 1");
  if (!block_supported(block)) return unsupported(fn, "block must be 32, 64 or 128");
  return SPARSTAR_OK;
}

bool density_ok(double d) { return std::isfinite(d) && d >= 0.0 && d <= 1.0; }

// Kernels move 16-byte vectors; device allocations are at least 256-byte aligned.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

namespace {
// Arguments of the screened score + selection route (every entry point to it).
sparstar_status check_select_from_means(const char* fn, const float* qbar, const float* kbar,
                                        int64_t B, int64_t H, int64_t nqb, int64_t nkb,
                                        int64_t D, float tau, int64_t n_forced_blocks,
                                        double density, const int32_t* kv_count,
                                        const int32_t* kv_index, int64_t max_kept,
                                        int64_t* kept_out) {
  if (!qbar || !kbar || !kv_count || !kv_index) return invalid(fn, "null pointer");
  if (!aligned16(qbar) || !aligned16(kbar)) return invalid(fn, "qbar and kbar must be 16-byte aligned");
  if (nqb < 1 || nkb < 1) return invalid(fn, "nqb and nkb must be >= 1");
  sparstar_status st = check_bhnd(fn, B, H, nqb > nkb ? nqb : nkb, D);
  if (st != SPARSTAR_OK) return st;
  if (nqb > kMaxI32 / nkb || B * H > kMaxI32 / nqb) return invalid(fn, "sizes too large");
  if (!std::isfinite(tau)) return invalid(fn, "tau must be finite");
  if (n_forced_blocks < 0 || n_forced_blocks > nkb)
    return invalid(fn, "n_forced_blocks must lie in [0, nkb]");
  if (!density_ok(density)) return invalid(fn, "density must lie in [0, 1]");
  const int64_t kept = sparstar_kept_blocks(nkb, n_forced_blocks, density);
  if (max_kept < kept) {
    set_error("%s: max_kept (%lld) < kept blocks per row (%lld)", fn, (long long)max_kept,
              (long long)kept);
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  if (max_kept > kMaxI32) return invalid(fn, "max_kept too large");
  if (nkb > fused_select_max_nkb()) {
    set_error("%s: nkb > %lld is not supported (use sparstar_block_scores + "
              "sparstar_select_blocks)", fn, (long long)fused_select_max_nkb());
    return SPARSTAR_ERR_UNSUPPORTED;
  }
  *kept_out = kept;
  return SPARSTAR_OK;
}

// The caller workspace of the screened route: present, 256-byte aligned, large enough.
sparstar_status check_workspace(const char* fn, const void* workspace, int64_t workspace_bytes,
                                int64_t BH, int64_t nqb, int64_t nkb) {
  if (!workspace) return invalid(fn, "null pointer");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return invalid(fn, "workspace must be 256-byte aligned");
  const int64_t need = select_workspace_bytes(BH, nqb, nkb);
  if (workspace_bytes < need) {
    set_error("%s: workspace_bytes (%lld) < %lld (sparstar_select_workspace_bytes)", fn,
              (long long)workspace_bytes, (long long)need);
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  return SPARSTAR_OK;
}
}  // namespace

extern "C" {

int32_t sparstar_version(void) { return 10400; }

const char* sparstar_last_error(void) { return g_err; }

int64_t sparstar_forced_blocks(int64_t n_forced_tokens, int64_t block) {
  if (n_forced_tokens < 0 || block < 1) return -1;
  return (n_forced_tokens + block - 1) / block;
}

int64_t sparstar_kept_blocks(int64_t nkb, int64_t n_forced_blocks, double density) {
  if (nkb < 0 || n_forced_blocks < 0 || n_forced_blocks > nkb || !density_ok(density)) return -1;
  // k = ceil(density * E): one rounded double product, then ceil.
  const double prod = density * static_cast<double>(nkb - n_forced_blocks);
  int64_t k = static_cast<int64_t>(std::ceil(prod));
  if (k > nkb - n_forced_blocks) k = nkb - n_forced_blocks;  // density <= 1 keeps this exact
  return n_forced_blocks + k;
}

sparstar_status sparstar_block_means(const void* x, sparstar_dtype dtype, int64_t B, int64_t H,
                                     int64_t N, int64_t D, int64_t block, float* out,
                                     void* stream) {
  const char* fn = "sparstar_block_means";
  clear_error();
  if (!x || !out) return invalid(fn, "null pointer");
  if (!aligned16(x)) return invalid(fn, "x must be 16-byte aligned");
  if (dtype != SPARSTAR_FP32 && dtype != SPARSTAR_BF16) return invalid(fn, "unknown dtype");
  sparstar_status st = check_bhnd(fn, B, H, N, D);
  if (st != SPARSTAR_OK) return st;
  if ((st = check_block(fn, block)) != SPARSTAR_OK) return st;
  return launch_block_means(x, dtype, B * H, N, D, block, out, static_cast<hipStream_t>(stream));
}

sparstar_status sparstar_block_scores(const float* qbar, const float* kbar, int64_t B, int64_t H,
                                      int64_t nqb, int64_t nkb, int64_t D, float tau, float* S,
                                      void* stream) {
  const char* fn = "sparstar_block_scores";
  clear_error();
  if (!qbar || !kbar || !S) return invalid(fn, "null pointer");
  if (!aligned16(qbar) || !aligned16(kbar)) return invalid(fn, "qbar and kbar must be 16-byte aligned");
  if (nqb < 1 || nkb < 1) return invalid(fn, "nqb and nkb must be >= 1");
  sparstar_status st = check_bhnd(fn, B, H, nqb > nkb ? nqb : nkb, D);
  if (st != SPARSTAR_OK) return st;
  if (nqb > kMaxI32 / nkb) return invalid(fn, "nqb*nkb per head must fit in int32");
  if (!std::isfinite(tau)) return invalid(fn, "tau must be finite");
  return launch_block_scores(qbar, kbar, B * H, nqb, nkb, D, tau, S,
                             static_cast<hipStream_t>(stream));
}

sparstar_status sparstar_select_blocks(const float* S, int64_t B, int64_t H, int64_t nqb,
                                       int64_t nkb, int64_t n_forced_blocks, double density,
                                       int32_t* kv_count, int32_t* kv_index, int64_t max_kept,
                                       void* stream) {
  const char* fn = "sparstar_select_blocks";
  clear_error();
  if (!S || !kv_count || !kv_index) return invalid(fn, "null pointer");
  if (B < 1 || H < 1 || nqb < 1 || nkb < 1) return invalid(fn, "B, H, nqb, nkb must be >= 1");
  if (nkb > kMaxI32 || B > kMaxI32 / H || B * H > kMaxI32 / nqb)
    return invalid(fn, "sizes too large");
  if (n_forced_blocks < 0 || n_forced_blocks > nkb)
    return invalid(fn, "n_forced_blocks must lie in [0, nkb]");
  if (!density_ok(density)) return invalid(fn, "density must lie in [0, 1]");
  const int64_t kept = sparstar_kept_blocks(nkb, n_forced_blocks, density);
  if (max_kept < kept) {
    set_error("%s: max_kept (%lld) < kept blocks per row (%lld)", fn, (long long)max_kept,
              (long long)kept);
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  if (max_kept > kMaxI32) return invalid(fn, "max_kept too large");
  return launch_select_blocks(S, B * H * nqb, nkb, n_forced_blocks, kept - n_forced_blocks,
                              kv_count, kv_index, max_kept, static_cast<hipStream_t>(stream));
}

int64_t sparstar_select_workspace_bytes(int64_t B, int64_t H, int64_t nqb, int64_t nkb) {
  if (B < 1 || H < 1 || nqb < 1 || nkb < 1 || nkb > fused_select_max_nkb()) return -1;
  if (B > kMaxI32 / H || nqb > kMaxI32 / (B * H)) return -1;
  return select_workspace_bytes(B * H, nqb, nkb);
}

sparstar_status sparstar_select_blocks_from_means(const float* qbar, const float* kbar,
                                                  int64_t B, int64_t H, int64_t nqb, int64_t nkb,
                                                  int64_t D, float tau, int64_t n_forced_blocks,
                                                  double density, int32_t* kv_count,
                                                  int32_t* kv_index, int64_t max_kept,
                                                  void* workspace, int64_t workspace_bytes,
                                                  void* stream) {
  const char* fn = "sparstar_select_blocks_from_means";
  clear_error();
  int64_t kept = 0;
  sparstar_status st = check_select_from_means(fn, qbar, kbar, B, H, nqb, nkb, D, tau,
                                               n_forced_blocks, density, kv_count, kv_index,
                                               max_kept, &kept);
  if (st != SPARSTAR_OK) return st;
  if ((st = check_workspace(fn, workspace, workspace_bytes, B * H, nqb, nkb)) != SPARSTAR_OK)
    return st;
  return launch_scores_select(qbar, kbar, B * H, nqb, nkb, D, tau, n_forced_blocks,
                              kept - n_forced_blocks, kv_count, kv_index, max_kept, workspace,
                              static_cast<hipStream_t>(stream));
}

sparstar_status sparstar_select_blocks_from_qk(const void* q, const void* k, sparstar_dtype dtype,
                                               int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                               int64_t D, int64_t block, float tau,
                                               int64_t n_forced_blocks, double density,
                                               float* qbar, float* kbar, int32_t* kv_count,
                                               int32_t* kv_index, int64_t max_kept,
                                               void* workspace, int64_t workspace_bytes,
                                               void* stream) {
  const char* fn = "sparstar_select_blocks_from_qk";
  clear_error();
  if (!q || !k) return invalid(fn, "null pointer");
  if (!aligned16(q) || !aligned16(k)) return invalid(fn, "q and k must be 16-byte aligned");
  if (dtype != SPARSTAR_FP32 && dtype != SPARSTAR_BF16) return invalid(fn, "unknown dtype");
  sparstar_status st = check_bhnd(fn, B, H, Nq, D);
  if (st != SPARSTAR_OK) return st;
  if ((st = check_bhnd(fn, B, H, Nk, D)) != SPARSTAR_OK) return st;
  if ((st = check_block(fn, block)) != SPARSTAR_OK) return st;
  const int64_t nqb = (Nq + block - 1) / block, nkb = (Nk + block - 1) / block;
  int64_t kept = 0;
  if ((st = check_select_from_means(fn, qbar, kbar, B, H, nqb, nkb, D, tau, n_forced_blocks,
                                    density, kv_count, kv_index, max_kept, &kept)) != SPARSTAR_OK)
    return st;
  if ((st = check_workspace(fn, workspace, workspace_bytes, B * H, nqb, nkb)) != SPARSTAR_OK)
    return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // two launches: one launch over both tensors measured slower on MI355X
  if ((st = launch_block_means(q, dtype, B * H, Nq, D, block, qbar, s)) != SPARSTAR_OK) return st;
  if ((st = launch_block_means(k, dtype, B * H, Nk, D, block, kbar, s)) != SPARSTAR_OK) return st;
  return launch_scores_select(qbar, kbar, B * H, nqb, nkb, D, tau, n_forced_blocks,
                              kept - n_forced_blocks, kv_count, kv_index, max_kept, workspace, s);
}

sparstar_status sparstar_select_blocks_from_means_noalloc(const float* qbar, const float* kbar,
                                                          int64_t B, int64_t H, int64_t nqb,
                                                          int64_t nkb, int64_t D, float tau,
                                                          int64_t n_forced_blocks, double density,
                                                          int32_t* kv_count, int32_t* kv_index,
                                                          int64_t max_kept, void* stream) {
  const char* fn = "sparstar_select_blocks_from_means_noalloc";
  clear_error();
  int64_t kept = 0;
  sparstar_status st = check_select_from_means(fn, qbar, kbar, B, H, nqb, nkb, D, tau,
                                               n_forced_blocks, density, kv_count, kv_index,
                                               max_kept, &kept);
  if (st != SPARSTAR_OK) return st;
  const int64_t need = select_workspace_bytes(B * H, nqb, nkb);
  if (need > select_scratch_bytes()) {
    set_error("%s: these sizes need %lld bytes of scratch, more than the %lld this entry point "
              "holds (use sparstar_select_blocks_from_means with a workspace)", fn,
              (long long)need, (long long)select_scratch_bytes());
    return SPARSTAR_ERR_UNSUPPORTED;
  }
  void* scratch = nullptr;
  if ((st = select_scratch_pointer(&scratch)) != SPARSTAR_OK) return st;
  return launch_scores_select(qbar, kbar, B * H, nqb, nkb, D, tau, n_forced_blocks,
                              kept - n_forced_blocks, kv_count, kv_index, max_kept, scratch,
                              static_cast<hipStream_t>(stream));
}

sparstar_status sparstar_retained_mass(const float* lse_sel, const float* lse_dense, int64_t n,
                                      float* mass, void* stream) {
  const char* fn = "sparstar_retained_mass";
  clear_error();
  if (n < 0) return invalid(fn, "n must be >= 0");
  if (n == 0) return SPARSTAR_OK;
  if (!lse_sel || !lse_dense || !mass) return invalid(fn, "null pointer");
  return launch_retained_mass(lse_sel, lse_dense, n, mass, static_cast<hipStream_t>(stream));
}

sparstar_status sparstar_transfer_scores(const float* S_src, int64_t B, int64_t H, int64_t block,
                                         int64_t src_n_text, int64_t src_n_ref, int64_t src_n_cur,
                                         int64_t dst_n_text, int64_t dst_n_ref, int64_t dst_n_cur,
                                         float* S_dst, void* stream) {
  const char* fn = "sparstar_transfer_scores";
  clear_error();
  if (!S_src || !S_dst) return invalid(fn, "null pointer");
  if (S_src == S_dst) return invalid(fn, "S_src and S_dst must not overlap");
  if (B < 1 || H < 1) return invalid(fn, "B and H must be >= 1");
  if (B > kMaxI32 / H) return invalid(fn, "B*H too large");
  sparstar_status st;
  if ((st = check_block(fn, block)) != SPARSTAR_OK) return st;
  const int64_t src[3] = {src_n_text, src_n_ref, src_n_cur};
  const int64_t dst[3] = {dst_n_text, dst_n_ref, dst_n_cur};
  constexpr int64_t kMaxScale = int64_t(1) << 30;
  int64_t ns = 0, nd = 0;
  for (int k = 0; k < 3; ++k) {
    if (src[k] < 0 || dst[k] < 0) return invalid(fn, "segment lengths must be >= 0");
    if (src[k] >= kMaxScale || dst[k] >= kMaxScale) return invalid(fn, "a scale must hold fewer than 2^30 tokens");
    if (dst[k] > 0 && src[k] == 0)
      return invalid(fn, "a non-empty target segment has an empty source segment");
    ns += src[k];
    nd += dst[k];
  }
  if (ns >= kMaxScale || nd >= kMaxScale) return invalid(fn, "a scale must hold fewer than 2^30 tokens");
  if (src_n_cur < 1 || dst_n_cur < 1) return invalid(fn, "n_cur must be >= 1 on both scales");
  const int64_t nqs = (src_n_cur + block - 1) / block, nks = (ns + block - 1) / block;
  const int64_t nqd = (dst_n_cur + block - 1) / block, nkd = (nd + block - 1) / block;
  if (nqs > kMaxI32 / nks || nqd > kMaxI32 / nkd)
    return invalid(fn, "nqb*nkb per head must fit in int32");
  return launch_transfer_scores(S_src, B * H, block, src, dst, S_dst,
                                static_cast<hipStream_t>(stream));
}

sparstar_status sparstar_token_topk_bound(const void* q, const void* k, sparstar_dtype dtype,
                                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                          int64_t block, int64_t n_forced_blocks, int64_t k_blocks,
                                          float scale, float* bound, void* stream) {
  const char* fn = "sparstar_token_topk_bound";
  clear_error();
  if (!q || !k || !bound) return invalid(fn, "null pointer");
  if (dtype != SPARSTAR_BF16 && dtype != SPARSTAR_FP32) return invalid(fn, "unknown dtype");
  if (dtype != SPARSTAR_BF16) return unsupported(fn, "only bf16 inputs are supported");
  if (!aligned16(q) || !aligned16(k)) return invalid(fn, "q and k must be 16-byte aligned");
  if (Nq < 1 || Nk < 1) return invalid(fn, "sequence lengths must be >= 1");
  sparstar_status st = check_bhnd(fn, B, H, Nq > Nk ? Nq : Nk, D);
  if (st != SPARSTAR_OK) return st;
  if ((st = check_block(fn, block)) != SPARSTAR_OK) return st;
  if (n_forced_blocks < 0 || k_blocks < 0) return invalid(fn, "block counts must be >= 0");
  if (!std::isfinite(scale) || !(scale > 0.f)) return invalid(fn, "scale must be finite and > 0");
  // token budget of the block policy (counts clamped to nkb first, so the
  // products stay small)
  const int64_t nkb = (Nk + block - 1) / block;
  const int64_t fb = n_forced_blocks < nkb ? n_forced_blocks : nkb;
  const int64_t kb = k_blocks < nkb ? k_blocks : nkb;
  const int64_t f_tok = fb * block < Nk ? fb * block : Nk;
  const int64_t m_tok = kb * block < Nk - f_tok ? kb * block : Nk - f_tok;
  return launch_token_topk_bound(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                 B * H, Nq, Nk, D, f_tok, m_tok, scale, bound,
                                 static_cast<hipStream_t>(stream));
}

sparstar_status sparstar_block_sparse_attn_fwd(const void* q, const void* k, const void* v,
                                               sparstar_dtype dtype, int64_t B, int64_t H,
                                               int64_t Nq, int64_t Nk, int64_t D, int64_t block,
                                               const int32_t* kv_count, const int32_t* kv_index,
                                               int64_t max_kept, float scale, void* o, float* lse,
                                               void* stream) {
  const char* fn = "sparstar_block_sparse_attn_fwd";
  clear_error();
  if (!q || !k || !v || !o || !kv_count) return invalid(fn, "null pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return invalid(fn, "q, k, v and o must be 16-byte aligned");
  if (max_kept < 0 || max_kept > kMaxI32) return invalid(fn, "max_kept must lie in [0, 2^31)");
  if (max_kept > 0 && !kv_index) return invalid(fn, "null kv_index");
  if (dtype != SPARSTAR_FP32 && dtype != SPARSTAR_BF16) return invalid(fn, "unknown dtype");
  sparstar_status st = check_bhnd(fn, B, H, Nq, D);
  if (st != SPARSTAR_OK) return st;
  if ((st = check_bhnd(fn, B, H, Nk, D)) != SPARSTAR_OK) return st;
  if ((st = check_block(fn, block)) != SPARSTAR_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.f)) return invalid(fn, "scale must be finite and > 0");
  const int64_t nqb = (Nq + block - 1) / block;
  if (B * H > kMaxI32 / nqb) return invalid(fn, "B*H*nqb too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == SPARSTAR_BF16)
    return launch_attn_fwd_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                static_cast<const uint16_t*>(v), B * H, Nq, Nk, D, block, kv_count,
                                kv_index, max_kept, scale, static_cast<uint16_t*>(o), lse, s);
  return launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                             static_cast<const float*>(v), B * H, Nq, Nk, D, block, kv_count, kv_index,
                             max_kept, scale, static_cast<float*>(o), lse, s);
}

}  // extern "C"
