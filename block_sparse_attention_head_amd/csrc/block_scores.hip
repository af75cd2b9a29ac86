// Aggregated block scores, Eq. 2 of SparSTAR (review section "What carries
// the argument"): S_ij = tau * qbar_i . kbar_j, per (batch, head).
//
// The selector ranks these scores, and an exact tie rule only means something
// if the GPU and a float64 reference agree on the order of nearly equal
// scores.  Products of two float32 means are exact in float64, so the dot
// product is accumulated in float64 on the fp64 matrix cores
// (score_tile.hpp) and rounded once to float32.
//
// The kernel is bound by the fp64 matrix cores, so the work is split evenly
// over exactly the wavefronts the GPU holds at once: a work item is 16 q rows
// x 32 k columns (two 16 x 16 tiles, two independent accumulation chains),
// items are numbered strip-major, and each one-wavefront workgroup takes a
// contiguous run of items (reloading its q operands only when the strip
// changes).  Without this, uneven placement of a larger grid leaves some
// SIMDs with twice the matrix work of others.
#include "score_tile.hpp"

namespace sparstar {
namespace {

template <int D>
__global__ __launch_bounds__(64) void block_scores_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nqb, int nkb,
    int strips, int pairs, int64_t items, double tau, float* __restrict__ S) {
  const int64_t per = (items + gridDim.x - 1) / gridDim.x;
  const int64_t it0 = blockIdx.x * per;
  const int64_t it1 = it0 + per < items ? it0 + per : items;
  const int l = threadIdx.x, lr = l % 16, ls = l / 16;
  const int ntk = (nkb + 15) / 16;

  int64_t cur_strip = -1;   // (b*h) * strips + strip whose q operands are loaded
  f32x4 qv[D / 16];
  for (int64_t it = it0; it < it1; ++it) {
    const int64_t hs = it / pairs;
    const int jt = 2 * static_cast<int>(it - hs * pairs);
    const int64_t bh = hs / strips;
    const int i0 = static_cast<int>(hs - bh * strips) * 16;
    if (hs != cur_strip) {
      const int iq = i0 + lr;   // rows past the edge read row 0 and are not stored
      load_operands<D>(qbar + (bh * nqb + (iq < nqb ? iq : 0)) * static_cast<int64_t>(D) + 4 * ls, qv);
      cur_strip = hs;
    }
    const float* kh = kbar + bh * static_cast<int64_t>(nkb) * D;
    auto krow = [&](int t) {
      const int jk = 16 * t + lr;   // columns past the edge read row 0 and are not stored
      return kh + static_cast<int64_t>(jk < nkb ? jk : 0) * D + 4 * ls;
    };
    f32x4 ka[D / 16], kb[D / 16];
    load_operands<D>(krow(jt), ka);
    load_operands<D>(krow(jt + 1 < ntk ? jt + 1 : jt), kb);
    f64x4 a0, a1;
    score_tiles16x2<D>(qv, ka, kb, a0, a1);
    float* Sh = S + bh * static_cast<int64_t>(nqb) * nkb;
    auto store = [&](const f64x4& acc, int t) {
      // acc[r] = S(i0 + ls + 4r, 16 t + lr)
      const int jk = 16 * t + lr;
      if (t < ntk && jk < nkb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + ls + 4 * r;
          if (i < nqb) Sh[static_cast<int64_t>(i) * nkb + jk] = static_cast<float>(tau * acc[r]);
        }
      }
    };
    store(a0, jt);
    store(a1, jt + 1);
  }
}

// Resident one-wavefront workgroups of `kernel` on the current device.
template <typename K>
sparstar_status resident_waves(K kernel, int64_t& waves) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess ||
      cus < 1 || per_cu < 1) {
    set_error("sparstar_block_scores: cannot query the device");
    return SPARSTAR_ERR_HIP;
  }
  waves = static_cast<int64_t>(cus) * per_cu;
  return SPARSTAR_OK;
}

template <int D>
sparstar_status launch_d(const float* qbar, const float* kbar, int64_t BH, int64_t nqb,
                         int64_t nkb, float tau, float* S, hipStream_t s) {
  const int64_t strips = (nqb + 15) / 16;
  const int64_t pairs = ((nkb + 15) / 16 + 1) / 2;
  const int64_t items = BH * strips * pairs;
  int64_t waves = 0;
  const sparstar_status st = resident_waves(block_scores_kernel<D>, waves);
  if (st != SPARSTAR_OK) return st;
  const dim3 grid(static_cast<uint32_t>(items < waves ? items : waves)), block(64);
  block_scores_kernel<D><<<grid, block, 0, s>>>(qbar, kbar, (int)nqb, (int)nkb, (int)strips,
                                                (int)pairs, items, (double)tau, S);
  return check_launch("sparstar_block_scores");
}

}  // namespace

sparstar_status launch_block_scores(const float* qbar, const float* kbar, int64_t BH,
                                    int64_t nqb, int64_t nkb, int64_t D, float tau, float* S,
                                    hipStream_t s) {
  return D == 128 ? launch_d<128>(qbar, kbar, BH, nqb, nkb, tau, S, s)
                  : launch_d<64>(qbar, kbar, BH, nqb, nkb, tau, S, s);
}

}  // namespace sparstar
