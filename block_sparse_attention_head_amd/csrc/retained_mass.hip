// Retained attention mass of a block selection, per query token (SparSTAR
// review, "Core claim": selections are compared by the share of dense
// attention mass they keep).
//
// With LSE_sel the log-sum-exp of a query's logits over the kept keys and
// LSE_dense the same over all keys, the dense softmax probability summed over
// the kept keys is exp(LSE_sel - LSE_dense).  Both come from the attention
// kernel (the second with every block listed), so this kernel is the
// elementwise last step.
#include <cmath>

#include "common.hpp"

namespace sparstar {
namespace {

__global__ __launch_bounds__(256) void retained_mass_kernel(const float* __restrict__ lse_sel,
                                                            const float* __restrict__ lse_dense,
                                                            int64_t n, float* __restrict__ mass) {
  for (int64_t t = blockIdx.x * 256ll + threadIdx.x; t < n; t += static_cast<int64_t>(gridDim.x) * 256) {
    const float a = lse_sel[t], d = lse_dense[t];
    // nothing kept (a = -inf) or no key at all (d = -inf): no mass is retained
    mass[t] = (a == -INFINITY || d == -INFINITY) ? 0.f : expf(a - d);
  }
}

}  // namespace

sparstar_status launch_retained_mass(const float* lse_sel, const float* lse_dense, int64_t n,
                                     float* mass, hipStream_t s) {
  const int64_t blocks = (n + 255) / 256;
  const dim3 grid(static_cast<uint32_t>(blocks < 65536 ? blocks : 65536)), block(256);
  retained_mass_kernel<<<grid, block, 0, s>>>(lse_sel, lse_dense, n, mass);
  return check_launch("sparstar_retained_mass");
}

}  // namespace sparstar
