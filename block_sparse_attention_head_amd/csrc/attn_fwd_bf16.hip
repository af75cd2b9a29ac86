// Block-sparse flash-attention forward for bf16 on gfx950 MFMA.
//
// Operation (SparSTAR review, "What carries the argument"): each query block
// attends only to the key blocks its forward index list names; the softmax
// runs over the valid keys of those blocks.
//
// Design (gfx950, wave64):
//  * One workgroup per (b*h, query block) = kBlock queries, kBlock / 32
//    waves x 32 queries (128-token blocks: 4 waves, two workgroups per CU,
//    two waves per SIMD, so one wave's matrix work overlaps the other's
//    vector work; 64- and 32-token blocks use 32-key tiles).  Every row keeps
//    the same number of blocks, so the grid is evenly loaded.
//  * Grid order: all XCDs work on the same head at a time (its K/V then
//    stays in the MALL), and each XCD takes a contiguous run of that head's
//    query blocks (neighbouring query blocks, which tend to select the same
//    key blocks, then share the XCD's L2).
//  * Each query block streams its selected K/V through a two-slot LDS ring
//    of kBK-key tiles, filled by gfx950's direct-to-LDS buffer loads
//    (buffer_load_dwordx4 ... lds: no staging registers, the tile offset in a
//    scalar, constant per-lane offsets) one tile ahead of use; one barrier
//    per tile.  The kernel is limited by this stream (every query block
//    reads 64 KiB per kept block), so the next tile's transfer must overlap
//    all of the current tile's work: the slots are separate LDS variables
//    (see below) so that no LDS read waits for it.  LDS rows are unpadded and their
//    16-byte chunks XOR-swizzled per row, which keeps both LDS read patterns
//    below free of bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q held in registers).
//    The output layout gives every lane ONE query and 16 keys of a 32-key
//    tile, so all softmax state is per-lane scalars; one exchange between
//    lanes l and l^32 (v_permlane32_swap) completes a row max.
//  * The output is accumulated transposed too, O^T += V^T P^T: P (bf16) is
//    the B operand straight from the score registers (the MFMA k index is
//    permuted to match the score layout), and V^T is read from the natural
//    [key][d] LDS tile with ds_read_b64_tr_b16, gfx950's transposing LDS
//    load, using the same key permutation.
//  * The LDS operand reads of both MFMA chains are issued several MFMAs
//    ahead of their use (instruction-group barriers; left alone the compiler
//    reads just in time and every MFMA waits out the LDS latency).
//  * Vector work per score is kept to one FMA, one exp2, half a bf16 pack
//    and half a v_dot2 (the row sum is taken over the packed bf16 weights the
//    MFMA consumes).  The reference max is set on the first tile and only
//    moved when a tile's weights would exceed 2^16 (detected from the row
//    sum), so the per-tile max and the output rescale are off the common
//    path.
//  * Keys past Nk (partial last block) are masked to -inf before the softmax
//    (their rows are fetched from row Nk-1, so the values are finite).  Index
//    entries outside [0, nkb) contribute nothing.
#include <cmath>

#include "tile_common.hpp"

namespace sparstar {
namespace {

// Keys per LDS tile: 64 for 128-token blocks, 32 for the smaller blocks
// (whose workgroups have fewer waves, so a smaller ring keeps more
// workgroups per CU).
template <int kBlock>
constexpr int tile_keys_of() { return kBlock >= 128 ? 64 : 32; }
// Weights exp2(s - m_ref) may grow up to a row sum of 2^16 before the
// reference max is moved (fp32 accumulators and bf16 weights hold that
// range as exactly as small values).
constexpr float kMaxRowSum = 65536.f;

template <int D, int kBlock>
__global__ __launch_bounds__(64 * (kBlock / 32), 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int Nq, int Nk, int nqb, int BH,
    const int32_t* __restrict__ kv_count, const int32_t* __restrict__ kv_index, int max_kept,
    float sl2, uint16_t* __restrict__ o, float* __restrict__ lse) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource builtins exist only in the device pass
  constexpr int kNW = kBlock / 32;            // waves: 32 queries each
  constexpr int kBK = tile_keys_of<kBlock>();
  constexpr int ROWB = 2 * D;                 // bytes per token row
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILEB = kBK * ROWB;           // bytes per K (or V) tile
  constexpr int RPI = 1024 / ROWB;            // rows per 1 KB wave-wide DMA instruction
  constexpr int DPW = TILEB / 1024 / kNW;     // DMAs per wave per tensor
  constexpr int TPB = kBlock / kBK;           // tiles per selected block
  constexpr int KT = kBK / 32;                // 32-key score sub-tiles per tile
  constexpr int NC = kBK / 16;                // 16-key P*V steps per tile
  constexpr int KSTEPS = D / 16;              // MFMA k-steps over d for S^T
  constexpr int DT = D / 32;                  // 32-row d tiles of O^T
  // Two ring slots of a K and a V tile.  Four separate variables, not one
  // array: each then carries its own alias scope, so the compiler can see
  // that reads of one slot do not touch the slot the DMA is filling and does
  // not make them wait for it (with one array it waits for the in-flight
  // tile before the V reads of every tile).
  __shared__ __attribute__((aligned(1024))) char ldsK0[TILEB];
  __shared__ __attribute__((aligned(1024))) char ldsV0[TILEB];
  __shared__ __attribute__((aligned(1024))) char ldsK1[TILEB];
  __shared__ __attribute__((aligned(1024))) char ldsV1[TILEB];

  // ---- which (b*h, query block) this workgroup owns -----------------------------
  int64_t bh;
  int i;
  {
    // Launch p runs on XCD p % 8.  Per head the query blocks are cut into 8
    // contiguous runs of `run` blocks, run x going to XCD x; consecutive
    // launches still sweep one head after another.
    const int p = blockIdx.x;
    const int run = (nqb + kXcds - 1) / kXcds;
    const int per_head = run * kXcds;
    const int head = p / per_head;
    const int r = p - head * per_head;
    i = (r % kXcds) * run + r / kXcds;
    bh = head;
    if (i >= nqb || head >= BH) return;   // padding launches (whole workgroup)
  }
  const int64_t row = bh * nqb + i;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);  // wave index (uniform)
  const int l = tid % 64, h = l / 32, n = l % 32;
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
  float m_ref = -INFINITY, l_run = 0.f;   // reference max (log2 units) and row sum

  int count = kv_count[row];
  count = count < 0 ? 0 : (count > max_kept ? max_kept : count);
  const int32_t* list = kv_index + row * static_cast<int64_t>(max_kept);
  const uint32_t head_bytes = static_cast<uint32_t>(Nk) * ROWB;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(k + bh * static_cast<int64_t>(Nk) * D), 0, head_bytes, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(v + bh * static_cast<int64_t>(Nk) * D), 0, head_bytes, kBufferRsrcWord3);
  const int T = TPB * count;

  // Tile t = part (t % TPB) of block list[t / TPB]: first key and valid key
  // count (0 when the index is out of range).
  auto tile_keys = [&](int t, int& key0) -> int {
    const int j = list[t / TPB];
    key0 = j * kBlock + (t % TPB) * kBK;
    if (j < 0 || j >= nkb) return 0;
    return min(kBK, Nk - key0);
  };

  // DMA geometry: wave w's m-th transfer fills 1 KB = LDS rows [RPI*u, RPI*u + RPI),
  // u = kNW*m + w; lane l lands in slot l % CPR of row RPI*u + l / CPR and so
  // fetches global chunk (slot ^ swizzle(row)).
  int dma_row[DPW], dma_off[DPW];
#pragma unroll
  for (int m = 0; m < DPW; ++m) {
    dma_row[m] = RPI * (kNW * m + w) + l / CPR;
    dma_off[m] = dma_row[m] * ROWB + 16 * ((l % CPR) ^ chunk_swizzle<D>(dma_row[m]));
  }
  // Every tile issues the same 2 * DPW transfers per wave; a tile with no
  // valid key fetches rows from the start of the sequence, which are finite
  // and never used.
  auto fetch_tile = [&](int t, char* kdst, char* vdst) {
    int key0;
    const int nv = tile_keys(t, key0);
    const int base = nv > 0 ? key0 : 0;
    if (nv == kBK) {   // whole tile valid: scalar tile offset + constant lane offsets
#pragma unroll
      for (int m = 0; m < DPW; ++m) {
        const int u = kNW * m + w;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kdst + 1024 * u), 16,
                                                 dma_off[m], row_offset_bytes(key0, ROWB), 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vdst + 1024 * u), 16,
                                                 dma_off[m], row_offset_bytes(key0, ROWB), 0, 0);
      }
    } else {           // partial tile: rows past Nk re-read row Nk-1 (finite, masked later)
#pragma unroll
      for (int m = 0; m < DPW; ++m) {
        const int u = kNW * m + w;
        const int rr = min(base + dma_row[m], Nk - 1);
        const int off = row_offset_bytes(rr, ROWB) + (dma_off[m] - dma_row[m] * ROWB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kdst + 1024 * u), 16,
                                                 off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vdst + 1024 * u), 16,
                                                 off, 0, 0, 0);
      }
    }
  };

  // per-lane LDS byte offsets of the operand reads (slot-relative)
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
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  // One tile: wait until tile t is in slot (Kl, Vl), start the DMA of tile
  // t + 1 into the other slot (Kn, Vn), then compute.  Called with constant
  // slots (the loop below takes tiles in pairs) so that every LDS access
  // names its variable.
  auto tile_body = [&](int t, const char* Kl, const char* Vl, char* Kn, char* Vn) {
    // Only tile t is outstanding here (tile t + 1 is issued after the
    // barrier), so this wave waits for all its transfers.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                       // all parts landed; the other slot is free
    if (t + 1 < T) fetch_tile(t + 1, Kn, Vn);
    int key0;
    const int nv = tile_keys(t, key0);
    if (nv <= 0) return;

    // ---- S^T = K Q^T : KT sub-tiles of 32 keys ----------------------------------
    f32x16 sacc[KT];
    // the KT accumulation chains interleave, so consecutive MFMAs are independent
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kl + 32 * kt * ROWB + koff[ks]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], sacc[kt], 0, 0, 0);
      }
    schedule_mfma_chain<4, KSTEPS * KT, 1>();   // K reads four MFMAs ahead
    // sacc[kt][r] = S(key 32*kt + (r%4) + 8*(r/4) + 4*h, query n)
    if (nv < kBK) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kt + (r % 4) + 8 * (r / 4) + 4 * h >= nv) sacc[kt][r] = -INFINITY;
    }
    // ---- weights against the reference max ------------------------------------
    // pw[c][e]: bf16 pairs of the weights of keys 16c.. of this tile, in the
    // register order the P*V MFMA consumes; the row sum is taken over exactly
    // these bf16 values.
    bf16x2 pw[NC][4];
    float ls = 0.f;
    auto weights = [&](float m_use) {
      ls = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kt = c / 2, r = 8 * (c % 2) + 2 * e;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], sl2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r + 1], sl2, -m_use));
          pw[c][e] = bf16x2{static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pw[c][e], ones, ls, false);
        }
    };
    const bool first = m_ref == -INFINITY;
    if (!__ballot(first)) weights(m_ref);
    // First tile, or a tile whose weights outgrew the reference: take the
    // exact tile max, move the reference, rescale, recompute.
    const float ls_pair = ls + partner_lane32(ls);
    if (__ballot(first || !(ls_pair <= kMaxRowSum))) {
      float mx = sacc[0][0];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
      mx = fmaxf(mx, partner_lane32(mx));
      const float m_new = fmaxf(m_ref, mx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 when m_ref = -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_ref = m_new;
      weights(m_ref == -INFINITY ? 0.f : m_ref);
    }
    l_run += ls;
    // ---- O^T += V^T P^T -----------------------------------------------------------
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[2 * e] = pw[c][e][0];
        pb[2 * e + 1] = pw[c][e][1];
      }
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
    schedule_mfma_chain<6, NC * DT, 2>();       // V^T reads six MFMAs ahead
  };

  if (T > 0) fetch_tile(0, ldsK0, ldsV0);
  for (int t = 0; t < T; t += 2) {
    tile_body(t, ldsK0, ldsV0, ldsK1, ldsV1);
    if (t + 1 < T) tile_body(t + 1, ldsK1, ldsV1, ldsK0, ldsV0);
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
      lse[bh * Nq + tok] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
#endif
}

template <int B>
sparstar_status launch_b(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH,
                         int64_t Nq, int64_t Nk, int64_t D, const int32_t* kv_count,
                         const int32_t* kv_index, int64_t max_kept, float scale, uint16_t* o,
                         float* lse, hipStream_t s) {
  const int64_t nqb = (Nq + B - 1) / B;
  const int64_t launches = BH * ((nqb + kXcds - 1) / kXcds) * kXcds;
  if (launches > 2147483647LL) {
    set_error("sparstar_block_sparse_attn_fwd: grid too large");
    return SPARSTAR_ERR_INVALID_ARGUMENT;
  }
  const dim3 grid(static_cast<uint32_t>(launches)), block(64 * (B / 32));
  const float sl2 = scale * 1.4426950408889634f;
  if (D == 128)
    attn_fwd_bf16_kernel<128, B><<<grid, block, 0, s>>>(q, k, v, (int)Nq, (int)Nk, (int)nqb, (int)BH,
                                                        kv_count, kv_index, (int)max_kept, sl2, o, lse);
  else
    attn_fwd_bf16_kernel<64, B><<<grid, block, 0, s>>>(q, k, v, (int)Nq, (int)Nk, (int)nqb, (int)BH,
                                                       kv_count, kv_index, (int)max_kept, sl2, o, lse);
  return check_launch("sparstar_block_sparse_attn_fwd");
}

}  // namespace

sparstar_status launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t block,
                                     const int32_t* kv_count, const int32_t* kv_index,
                                     int64_t max_kept, float scale, uint16_t* o, float* lse,
                                     hipStream_t s) {
  if (block == 32)
    return launch_b<32>(q, k, v, BH, Nq, Nk, D, kv_count, kv_index, max_kept, scale, o, lse, s);
  if (block == 64)
    return launch_b<64>(q, k, v, BH, Nq, Nk, D, kv_count, kv_index, max_kept, scale, o, lse, s);
  return launch_b<128>(q, k, v, BH, Nq, Nk, D, kv_count, kv_index, max_kept, scale, o, lse, s);
}

}  // namespace sparstar
