/*
 * sparstar.h -- C ABI of the SparSTAR selected-block attention hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources: the review "Pith review of SparSTAR: Sparse
 * Attention for SpaceTime AutoRegressive Video Synthesis", pith.science, and
 * the SparSTAR abstract on mlsanity.com):
 *
 *   separately for every costly refinement scale and every attention head
 *   (abstract), i.e. per (batch, head):
 *     1. qbar_i, kbar_j: means of Q and K over runs of 128 consecutive
 *        tokens ("What carries the argument");
 *     2. S_ij = tau * qbar_i . kbar_j with tau = D^-1/2 (Eq. 2, same section);
 *     3. keep the forced context blocks (text; for Clip 1 also the final
 *        image-pyramid reference) and jointly rank every other key block
 *        (preceding-clip reference and current scale) under the scale's
 *        density budget ("What carries the argument", "Core claim");
 *     4. run forward attention over the kept blocks only, from a forward
 *        index list with no reverse index ("What carries the argument").
 *
 * Layout conventions (all entry points):
 *   - Tensors are dense, row-major, head-major: Q [B,H,Nq,D], K and V
 *     [B,H,Nk,D], O [B,H,Nq,D], means [B,H,nblocks,D], S [B,H,nqb,nkb],
 *     kv_count [B,H,nqb], kv_index [B,H,nqb,max_kept], lse [B,H,Nq].
 *   - Key tokens are in the order text | reference | current, so the forced
 *     context is a prefix and is given as a number of leading key blocks.
 *   - Every pointer is DEVICE memory owned by the caller; the library
 *     allocates nothing and keeps no state besides a per-thread error string.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; nothing is synchronised.
 *
 * Errors: arguments are checked on the host before anything is enqueued.  A
 * status other than SPARSTAR_OK means nothing was enqueued and no output was
 * written; sparstar_last_error() then describes the problem.  A failed kernel
 * launch returns SPARSTAR_ERR_HIP.
 */
#ifndef SPARSTAR_H_
#define SPARSTAR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARSTAR_OK = 0,
  SPARSTAR_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad density, ... */
  SPARSTAR_ERR_UNSUPPORTED = 2,      /* valid but not implemented (block not 32/64/128, D not 64/128) */
  SPARSTAR_ERR_HIP = 3               /* the HIP runtime refused a launch */
} sparstar_status;

typedef enum {
  SPARSTAR_FP32 = 0, /* IEEE float32 */
  SPARSTAR_BF16 = 1  /* bfloat16 bit patterns (uint16) */
} sparstar_dtype;

/* The pages' block size of 128 tokens (review, "Assumptions & free
 * parameters").  The means and attention entry points
 * also take block = 64 or 32: the review notes that smaller blocks improve
 * fidelity but had no efficient kernel in the authors' environment
 * ("Assumptions & free parameters", "Referee Report" minor comment 4). */
#define SPARSTAR_BLOCK 128

/*
 * Block means (review, "What carries the argument": queries and keys are
 * averaged over runs of consecutive tokens, one run per block).
 *   x    [B,H,N,D] of `dtype`.
 *   out  [B,H,ceil(N/block),D] float32.  out[b,h,i,:] is the mean of tokens
 *        [i*block, min((i+1)*block, N)); a partial last block is divided by
 *        its own token count.  Sums are accumulated exactly enough that the
 *        result is the fp32 rounding of the exact mean up to ~1 ulp.
 * Requires block in {32, 64, 128}, D in {64,128}, N >= 1.
 */
sparstar_status sparstar_block_means(const void* x, sparstar_dtype dtype, int64_t B, int64_t H,
                                     int64_t N, int64_t D, int64_t block, float* out,
                                     void* stream);

/*
 * Aggregated block scores, Eq. 2 ("What carries the argument"):
 *   S[b,h,i,j] = tau * sum_d qbar[b,h,i,d] * kbar[b,h,j,d]
 * qbar [B,H,nqb,D] and kbar [B,H,nkb,D] float32; S [B,H,nqb,nkb] float32.
 * Products and sums are formed in float64 and tau * sum is rounded once to
 * float32, so nearly equal scores keep the order of a float64 reference.
 * Pass tau = 1/sqrt(D) for the method's score.
 * Requires D in {64,128}, nqb >= 1, nkb >= 1.
 */
sparstar_status sparstar_block_scores(const float* qbar, const float* kbar, int64_t B, int64_t H,
                                      int64_t nqb, int64_t nkb, int64_t D, float tau, float* S,
                                      void* stream);

/*
 * Clip-aware joint Top-K ("What carries the argument", "Core claim").
 * For every row (b,h,i) of S [B,H,nqb,nkb]:
 *   - blocks [0, n_forced_blocks) are always kept (text, and for Clip 1 the
 *     image-pyramid reference);
 *   - of the E = nkb - n_forced_blocks eligible blocks, the
 *     k = ceil(density * E) with the largest S are kept (density * E is one
 *     rounded double product); equal scores go to the lower block index;
 *     NaN ranks below every number, -0.0 equals +0.0;
 *   - kv_count[b,h,i] = n_forced_blocks + k;
 *   - kv_index[b,h,i,:] lists the kept blocks in ascending order, then -1
 *     up to max_kept.
 * Requires 0 <= n_forced_blocks <= nkb, 0 <= density <= 1 and
 * max_kept >= sparstar_kept_blocks(nkb, n_forced_blocks, density).
 * The output is the forward index only; no reverse (key -> query) index is
 * built, matching the forward-only path the review describes.
 */
sparstar_status sparstar_select_blocks(const float* S, int64_t B, int64_t H, int64_t nqb,
                                       int64_t nkb, int64_t n_forced_blocks, double density,
                                       int32_t* kv_count, int32_t* kv_index, int64_t max_kept,
                                       void* stream);

/*
 * Scores and selection in one pass (review, "What carries the argument":
 * Eq. 2 scores, then the clip-aware joint Top-K): the same result as
 * sparstar_block_scores(qbar, kbar, ..., tau, S) followed by
 * sparstar_select_blocks(S, ...), bit for bit, without S in device memory.
 * All scores are first screened at reduced precision with a proven error
 * bound; only the blocks whose score lies within that bound of a row's k-th
 * largest are recomputed exactly as sparstar_block_scores forms them, and
 * the ranking uses those exact values, so both routes select identically.
 * Arguments are those of the two calls (qbar [B,H,nqb,D], kbar [B,H,nkb,D]
 * float32; kv_count [B,H,nqb]; kv_index [B,H,nqb,max_kept]) with their
 * requirements, and additionally nkb <= 2048 (a row of screened scores is
 * held in registers); larger nkb returns SPARSTAR_ERR_UNSUPPORTED.
 * workspace: caller-owned device memory of at least
 * sparstar_select_workspace_bytes(B, H, nqb, nkb) bytes, 256-byte aligned,
 * used as scratch (the screened scores as float16, nqb x 128 ceil(nkb / 128)
 * per head, and the largest key-block norm of each strip of 128 blocks); its
 * contents before and after the call carry no meaning.  Two calls in flight
 * at once must not share a workspace.
 */
sparstar_status sparstar_select_blocks_from_means(const float* qbar, const float* kbar,
                                                  int64_t B, int64_t H, int64_t nqb, int64_t nkb,
                                                  int64_t D, float tau, int64_t n_forced_blocks,
                                                  double density, int32_t* kv_count,
                                                  int32_t* kv_index, int64_t max_kept,
                                                  void* workspace, int64_t workspace_bytes,
                                                  void* stream);
/* Workspace bytes sparstar_select_blocks_from_means needs for these sizes;
 * -1 when the sizes are invalid or nkb > 2048.  Host only. */
int64_t sparstar_select_workspace_bytes(int64_t B, int64_t H, int64_t nqb, int64_t nkb);

/*
 * The whole selection stage of one scale from Q and K ("What carries the
 * argument": block means, Eq. 2 scores, clip-aware joint Top-K): the block
 * means of q and of k, as sparstar_block_means computes them, into qbar and
 * kbar (caller buffers, left holding the means), then the selection of
 * sparstar_select_blocks_from_means on them, with the same workspace rules:
 * one call for the stage, four kernel launches.  The result equals
 * sparstar_block_means(q), sparstar_block_means(k) and
 * sparstar_select_blocks_from_means(qbar, kbar, ...) bit for bit.
 *   q [B,H,Nq,D] and k [B,H,Nk,D] of `dtype`, 16-byte aligned; block as for
 *   sparstar_block_means; qbar [B,H,ceil(Nq/block),D] and
 *   kbar [B,H,ceil(Nk/block),D] float32; kv_count [B,H,nqb] and
 *   kv_index [B,H,nqb,max_kept] with nqb = ceil(Nq/block).
 * Requirements: those of sparstar_block_means for q and k and of
 * sparstar_select_blocks_from_means with nkb = ceil(Nk/block); every check is
 * made before anything is enqueued.
 */
sparstar_status sparstar_select_blocks_from_qk(const void* q, const void* k, sparstar_dtype dtype,
                                               int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                               int64_t D, int64_t block, float tau,
                                               int64_t n_forced_blocks, double density,
                                               float* qbar, float* kbar, int32_t* kv_count,
                                               int32_t* kv_index, int64_t max_kept,
                                               void* workspace, int64_t workspace_bytes,
                                               void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments, result and requirements as
 * sparstar_select_blocks_from_means, without the workspace.  In its place
 * the library uses a 64 MiB array of its own in device memory, one per GPU it
 * runs on, held until the process ends; this call allocates nothing.  Sizes
 * whose sparstar_select_workspace_bytes exceeds 64 MiB return
 * SPARSTAR_ERR_UNSUPPORTED before anything is enqueued.  Every call on one
 * GPU uses that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must not be made.
 */
sparstar_status sparstar_select_blocks_from_means_noalloc(const float* qbar, const float* kbar,
                                                          int64_t B, int64_t H, int64_t nqb,
                                                          int64_t nkb, int64_t D, float tau,
                                                          int64_t n_forced_blocks, double density,
                                                          int32_t* kv_count, int32_t* kv_index,
                                                          int64_t max_kept, void* stream);

/*
 * Block-sparse forward attention (review, "What carries the argument": only
 * the selected blocks are computed, by a forward-only operator).
 * For every query token t of query block i of (b,h):
 *   O[b,h,t,:] = sum_s softmax_s(scale * q_t . k_s) * v_s
 *   lse[b,h,t] = log sum_s exp(scale * q_t . k_s)
 * where s runs over the valid keys (s < Nk) of the blocks
 * kv_index[b,h,i,0 .. kv_count[b,h,i]-1].  No causal mask is applied.
 * Index entries outside [0, ceil(Nk/block)) are skipped; kv_count is clamped
 * to [0, max_kept].  A row with no valid block gives O = 0 and lse = -inf.
 *   q [B,H,Nq,D], k, v [B,H,Nk,D] of `dtype`; o [B,H,Nq,D] of `dtype`;
 *   lse [B,H,Nq] float32, may be NULL.
 * bf16 inputs run on bf16 MFMA with float32 accumulation and a float32
 * online softmax; float32 inputs run in float32 throughout.  Query block i
 * is tokens [i*block, (i+1)*block) and key block j tokens [j*block, ...).
 * Requires block in {32, 64, 128}, D in {64,128}.
 */
sparstar_status sparstar_block_sparse_attn_fwd(const void* q, const void* k, const void* v,
                                               sparstar_dtype dtype, int64_t B, int64_t H,
                                               int64_t Nq, int64_t Nk, int64_t D, int64_t block,
                                               const int32_t* kv_count, const int32_t* kv_index,
                                               int64_t max_kept, float scale, void* o, float* lse,
                                               void* stream);

/*
 * Retained attention mass, a diagnostic of a selection (review, "Core
 * claim": fresh block-wise Top-K is judged by the share of dense attention
 * mass it keeps).  For each of the n query tokens:
 *   mass[t] = exp(lse_sel[t] - lse_dense[t])
 * = the dense softmax probability of query t summed over the kept keys, where
 * lse_sel comes from sparstar_block_sparse_attn_fwd with the selection and
 * lse_dense from the same call with every block listed (e.g. the lists of
 * sparstar_select_blocks with n_forced_blocks = 0 and density = 1).  A query
 * with lse_sel or lse_dense equal to -inf gets 0.  All three arrays are
 * float32 device memory of n elements; n = 0 is a no-op.
 */
sparstar_status sparstar_retained_mass(const float* lse_sel, const float* lse_dense, int64_t n,
                                       float* mass, void* stream);

/*
 * Token-wise Top-K upper bound of the retained attention mass (review, "Core
 * claim": block-wise Top-K is measured against the token-wise Top-K upper
 * bound at the same budget).  For every query token t, with p_s the dense
 * softmax probability of key s (scale * q_t . k_s over all Nk keys):
 *   bound[t] = sum of p_s over s < f_tok + sum of the m_tok largest p_s over
 *              s >= f_tok,
 * f_tok = min(n_forced_blocks * block, Nk), m_tok = min(k_blocks * block,
 * Nk - f_tok): the mass kept by the best selection of single keys with as
 * many keys as n_forced_blocks forced and k_blocks ranked blocks hold.  The
 * m_tok-th largest logit is located by bisection to within 1/2^21 of the
 * logit range; the keys inside that last interval are counted at its upper
 * end, so the result errs upwards only, by a relative amount below
 * 2^(range / 2^21) - 1.  Logits are computed with bf16 MFMA and float32
 * accumulation, sums in float32.
 *   q [B,H,Nq,D], k [B,H,Nk,D] bf16 (16-byte aligned); bound [B,H,Nq] float32.
 * Requires bf16 (float32 returns UNSUPPORTED), D in {64, 128}, block in
 * {32, 64, 128}, scale finite and > 0; counts are clamped to nkb.  Runs the
 * key stream of each head several times: a diagnostic, not a hot-path call.
 */
sparstar_status sparstar_token_topk_bound(const void* q, const void* k, sparstar_dtype dtype,
                                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                          int64_t block, int64_t n_forced_blocks, int64_t k_blocks,
                                          float scale, float* bound, void* stream);

/*
 * Mask reuse, the baseline the method argues against (review, "Extended
 * reading notes" / "Core claim": a selection carried over from another scale
 * or across a clip boundary keeps less attention mass than a fresh one;
 * abstract: the analyses compare a selection computed anew per scale with
 * one carried over).  Builds the target scale's score matrix from a source
 * scale's, so that sparstar_select_blocks on it gives the transferred
 * selection under the target scale's own forced set and budget:
 *   S_dst[b,h,i,j] = S_src[b,h, qmap(i), kmap(j)].
 * A scale's geometry is (n_text, n_ref, n_cur): queries are its n_cur
 * current tokens, keys the concatenation [text | ref | cur], both cut into
 * `block`-token blocks from token 0.  A block stands for the centre of its
 * valid tokens (token t covers [t, t+1)); the segment holding that centre is
 * mapped by relative position onto the same segment of the source scale and
 * the source token found there, floor(start_src + (c - start_dst) *
 * len_src / len_dst), names the source block (the pages give no mapping;
 * this is the plain reading of "the same place at the other scale").
 *   S_src [B,H,ceil(src_n_cur/block), ceil(src_n/block)] float32,
 *   S_dst [B,H,ceil(dst_n_cur/block), ceil(dst_n/block)] float32,
 *   src_n = src_n_text + src_n_ref + src_n_cur (likewise dst_n); device
 *   memory, caller-owned, not overlapping.  S_dst is fully overwritten.
 * Errors (nothing written): INVALID_ARGUMENT for null pointers, B or H < 1,
 * negative segment lengths, n_cur < 1, a non-empty target segment whose
 * source segment is empty, a scale of 2^30 tokens or more, or sizes whose
 * element count per head exceeds int32; UNSUPPORTED for block not in
 * {32, 64, 128}.
 */
sparstar_status sparstar_transfer_scores(const float* S_src, int64_t B, int64_t H, int64_t block,
                                         int64_t src_n_text, int64_t src_n_ref, int64_t src_n_cur,
                                         int64_t dst_n_text, int64_t dst_n_ref, int64_t dst_n_cur,
                                         float* S_dst, void* stream);

/* Host-only helpers (no HIP call, no error state). */
/* ceil(n_forced_tokens / block): leading blocks that hold forced tokens; -1 on bad input. */
int64_t sparstar_forced_blocks(int64_t n_forced_tokens, int64_t block);
/* n_forced_blocks + ceil(density * (nkb - n_forced_blocks)); -1 on bad input. */
int64_t sparstar_kept_blocks(int64_t nkb, int64_t n_forced_blocks, double density);
/* Message of the last failed call on this thread ("" if none). */
const char* sparstar_last_error(void);
/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t sparstar_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSTAR_H_ */
