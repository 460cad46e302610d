// Adaptive regulariser of SwiAttn, per token (one layer).
//
// SwiAttn report, section 2, adaptive regulariser paragraph: token t of a
// layer carries the loss gamma_t * softplus(R(h_t)), where R(h_t) is the
// router logit and gamma_t = gamma_base / (eps + NLL(t) + alpha *
// ||o_FULL - o_SWA||^2) lowers the pressure towards the window branch for
// hard tokens (high NLL) and for tokens whose two branch outputs differ.
// The distance is the per-token value that prefill's both-branch mode
// writes; the logits are the router's optional output.  With several gate
// groups every group's logit shares the token's gamma.
//
// One pass over the logits (bound: HBM): 16 bytes read or written per
// (token, group) at G = 1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace swi {

constexpr int kRegThreads = 256;

__global__ __launch_bounds__(kRegThreads) void regularizer_kernel(const float* z, const float* nll,
                                                                  const float* diff, float* loss,
                                                                  int64_t n, int G, float gamma_base,
                                                                  float eps, float alpha) {
  const int64_t stride = int64_t(gridDim.x) * kRegThreads;
  for (int64_t i = int64_t(blockIdx.x) * kRegThreads + threadIdx.x; i < n; i += stride) {
    const int64_t t = i / G;
    const float gamma = gamma_base / (eps + nll[t] + alpha * diff[t]);
    const float x = z[i];
    // softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|): no overflow
    // for large x, no cancellation for very negative x
    const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
    loss[i] = gamma * sp;
  }
}

hipError_t launch_regularizer(const float* z, const float* nll, const float* diff, float* loss,
                              int B, int N, int G, float gamma_base, float eps, float alpha,
                              hipStream_t s) {
  const int64_t n = int64_t(B) * N * G;
  const int64_t want = (n + kRegThreads - 1) / kRegThreads;
  const int grid = int(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(regularizer_kernel, dim3(grid), dim3(kRegThreads), 0, s, z, nll, diff, loss, n, G,
                     gamma_base, eps, alpha);
  return hipGetLastError();
}

}  // namespace swi
