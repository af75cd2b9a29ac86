/*
 * Plain C user of libsparstar.so: one small bf16 scale (means, scores,
 * selection, attention, retained mass) through the C ABI only, with HIP
 * runtime calls for memory.  Checks what holds without a reference:
 * statuses, the kept count and forced prefix of every row, ascending
 * indices and -1 padding, finite outputs, and a retained mass in (0, 1].
 * Prints "abi_smoke ok" and returns 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sparstar.h"

#define CHECK(c)                                                                 \
  do {                                                                           \
    if (!(c)) {                                                                  \
      fprintf(stderr, "abi_smoke: check failed at line %d: %s (%s)\n", __LINE__, \
              #c, sparstar_last_error());                                        \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);   /* round to nearest even (finite inputs) */
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  const int64_t B = 1, H = 2, Nq = 300, Nk = 700, D = 128, blk = SPARSTAR_BLOCK;
  const int64_t n_forced_tokens = 130;
  const double density = 0.25;
  const int64_t nqb = (Nq + blk - 1) / blk, nkb = (Nk + blk - 1) / blk;
  const int64_t F = sparstar_forced_blocks(n_forced_tokens, blk);
  const int64_t kept = sparstar_kept_blocks(nkb, F, density);
  CHECK(sparstar_version() >= 10000);
  CHECK(F == 2 && kept == 3);   /* nkb = 6: 2 forced + ceil(0.25 * 4) */

  const size_t nq = (size_t)(B * H * Nq * D), nk = (size_t)(B * H * Nk * D);
  uint16_t* hq = malloc(nq * 2);
  uint16_t* hk = malloc(nk * 2);
  uint16_t* hv = malloc(nk * 2);
  uint32_t state = 12345u;
  for (size_t i = 0; i < nq; ++i) {
    state = state * 1664525u + 1013904223u;
    hq[i] = to_bf16(((float)(state >> 8) / 16777216.0f - 0.5f) * 2.0f);
  }
  for (size_t i = 0; i < nk; ++i) {
    state = state * 1664525u + 1013904223u;
    hk[i] = to_bf16(((float)(state >> 8) / 16777216.0f - 0.5f) * 2.0f);
    state = state * 1664525u + 1013904223u;
    hv[i] = to_bf16(((float)(state >> 8) / 16777216.0f - 0.5f) * 2.0f);
  }

  void *q, *k, *v, *o;
  float *qbar, *kbar, *S, *lse, *lse_d, *mass;
  int32_t *cnt, *idx, *dcnt, *didx;
  CHECK(hipMalloc(&q, nq * 2) == hipSuccess && hipMalloc(&k, nk * 2) == hipSuccess);
  CHECK(hipMalloc(&v, nk * 2) == hipSuccess && hipMalloc(&o, nq * 2) == hipSuccess);
  CHECK(hipMalloc((void**)&qbar, B * H * nqb * D * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&kbar, B * H * nkb * D * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&S, B * H * nqb * nkb * 4) == hipSuccess);
  float* S2;
  CHECK(hipMalloc((void**)&S2, B * H * nqb * nkb * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&cnt, B * H * nqb * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&idx, B * H * nqb * kept * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&dcnt, B * H * nqb * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&didx, B * H * nqb * nkb * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&lse, B * H * Nq * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&lse_d, B * H * Nq * 4) == hipSuccess);
  CHECK(hipMalloc((void**)&mass, B * H * Nq * 4) == hipSuccess);
  float* bnd;
  CHECK(hipMalloc((void**)&bnd, B * H * Nq * 4) == hipSuccess);
  CHECK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice) == hipSuccess);
  CHECK(hipMemcpy(k, hk, nk * 2, hipMemcpyHostToDevice) == hipSuccess);
  CHECK(hipMemcpy(v, hv, nk * 2, hipMemcpyHostToDevice) == hipSuccess);

  const float tau = 1.0f / sqrtf((float)D);
  CHECK(sparstar_block_means(q, SPARSTAR_BF16, B, H, Nq, D, blk, qbar, NULL) == SPARSTAR_OK);
  CHECK(sparstar_block_means(k, SPARSTAR_BF16, B, H, Nk, D, blk, kbar, NULL) == SPARSTAR_OK);
  CHECK(sparstar_block_scores(qbar, kbar, B, H, nqb, nkb, D, tau, S, NULL) == SPARSTAR_OK);
  CHECK(sparstar_select_blocks(S, B, H, nqb, nkb, F, density, cnt, idx, kept, NULL) == SPARSTAR_OK);
  CHECK(sparstar_block_sparse_attn_fwd(q, k, v, SPARSTAR_BF16, B, H, Nq, Nk, D, blk, cnt, idx,
                                       kept, tau, o, lse, NULL) == SPARSTAR_OK);
  CHECK(sparstar_select_blocks(S, B, H, nqb, nkb, 0, 1.0, dcnt, didx, nkb, NULL) == SPARSTAR_OK);
  CHECK(sparstar_block_sparse_attn_fwd(q, k, v, SPARSTAR_BF16, B, H, Nq, Nk, D, blk, dcnt, didx,
                                       nkb, tau, o, lse_d, NULL) == SPARSTAR_OK);
  CHECK(sparstar_retained_mass(lse, lse_d, B * H * Nq, mass, NULL) == SPARSTAR_OK);
  CHECK(sparstar_token_topk_bound(q, k, SPARSTAR_BF16, B, H, Nq, Nk, D, blk, F, kept - F, tau, bnd,
                                  NULL) == SPARSTAR_OK);
  /* the same geometry on both sides: the transferred scores are the scores */
  CHECK(sparstar_transfer_scores(S, B, H, blk, 130, 270, Nq, 130, 270, Nq, S2, NULL) == SPARSTAR_OK);
  /* a rejected call enqueues nothing and explains itself */
  CHECK(sparstar_block_means(q, SPARSTAR_BF16, B, H, Nq, 96, blk, qbar, NULL) ==
        SPARSTAR_ERR_UNSUPPORTED);
  CHECK(strlen(sparstar_last_error()) > 0);
  CHECK(hipDeviceSynchronize() == hipSuccess);

  int32_t* hc = malloc(B * H * nqb * 4);
  int32_t* hi = malloc(B * H * nqb * kept * 4);
  float* hm = malloc(B * H * Nq * 4);
  uint16_t* ho = malloc(nq * 2);
  CHECK(hipMemcpy(hc, cnt, B * H * nqb * 4, hipMemcpyDeviceToHost) == hipSuccess);
  CHECK(hipMemcpy(hi, idx, B * H * nqb * kept * 4, hipMemcpyDeviceToHost) == hipSuccess);
  CHECK(hipMemcpy(hm, mass, B * H * Nq * 4, hipMemcpyDeviceToHost) == hipSuccess);
  CHECK(hipMemcpy(ho, o, nq * 2, hipMemcpyDeviceToHost) == hipSuccess);
  for (int64_t r = 0; r < B * H * nqb; ++r) {
    CHECK(hc[r] == kept);
    for (int64_t e = 0; e < F; ++e) CHECK(hi[r * kept + e] == e);
    for (int64_t e = 1; e < kept; ++e) CHECK(hi[r * kept + e] > hi[r * kept + e - 1]);
    CHECK(hi[r * kept + kept - 1] < nkb);
  }
  for (int64_t t = 0; t < B * H * Nq; ++t) CHECK(hm[t] > 0.f && hm[t] <= 1.f);
  float* hb = malloc(B * H * Nq * 4);
  CHECK(hipMemcpy(hb, bnd, B * H * Nq * 4, hipMemcpyDeviceToHost) == hipSuccess);
  /* the token-wise bound at the same budget is at least the block selection's mass */
  for (int64_t t = 0; t < B * H * Nq; ++t) CHECK(hb[t] >= hm[t] - 1e-5f && hb[t] <= 1.f);
  float* hs = malloc(B * H * nqb * nkb * 4);
  float* hs2 = malloc(B * H * nqb * nkb * 4);
  CHECK(hipMemcpy(hs, S, B * H * nqb * nkb * 4, hipMemcpyDeviceToHost) == hipSuccess);
  CHECK(hipMemcpy(hs2, S2, B * H * nqb * nkb * 4, hipMemcpyDeviceToHost) == hipSuccess);
  CHECK(memcmp(hs, hs2, B * H * nqb * nkb * 4) == 0);
  for (size_t i = 0; i < nq; ++i) CHECK(isfinite(from_bf16(ho[i])) && fabsf(from_bf16(ho[i])) <= 1.f);
  printf("abi_smoke ok\n");
  return 0;
}
