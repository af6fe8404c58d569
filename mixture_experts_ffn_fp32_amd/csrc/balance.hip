// Bias-based load balancing ("APEX-1 Mathematical Reference - Part 3",
// section 14.3): b_e <- clamp(b_e + alpha * sign(1/E - c_e / (N K)), -1, 1).
// The sign is taken on integers, N K - E c_e, so an exactly balanced expert
// never moves however large N is.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void balance_kernel(int E, int64_t nk, const int32_t *counts,
                                                      float alpha, float *bias) {
  for (int e = threadIdx.x + blockIdx.x * 256; e < E; e += 256 * gridDim.x) {
    const int64_t diff = nk - static_cast<int64_t>(E) * counts[e];
    const float s = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
    float b = bias[e] + alpha * s;  // alpha * s is exact: one rounding
    bias[e] = fminf(1.f, fmaxf(-1.f, b));
  }
}

}  // namespace

hipError_t launch_balance(int E, int64_t nk, const int32_t *counts, float alpha, float *bias,
                          hipStream_t s) {
  balance_kernel<<<(E + 255) / 256, 256, 0, s>>>(E, nk, counts, alpha, bias);
  return hipGetLastError();
}

}  // namespace moe
