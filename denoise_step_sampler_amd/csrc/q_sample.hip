// Closed-form forward corruption x_t ~ q(x_t | x_0) (Technical Report part 2/6 sec. 2.1.1
// eq. (1); DiffusionGemma-Lite, forward process): each position keeps its clean token with
// probability kappa of its canvas, else takes a uniform token.  One thread per position.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

__global__ __launch_bounds__(256) void k_q_sample(const int32_t* __restrict__ x0, int R, int V,
                                                  const float* __restrict__ kappa, uint32_t k0,
                                                  uint32_t k1, int32_t* __restrict__ xt) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int c = r / DG_CANVAS;
  float kp = kappa[c];
  kp = fminf(fmaxf(kp, 0.0f), 1.0f);  // NaN -> 0
  const uint32_t thr = (uint32_t)floorf(kp * 16777216.0f);
  const u32x4 wd = philox4x32_10(u32x4{0u, (uint32_t)r, 0u, kTagQSample}, k0, k1);
  const bool keep = (wd[0] >> 8) < thr;
  xt[r] = keep ? x0[r] : uniform_token(wd[1], (uint32_t)V);
}

}  // namespace

hipError_t q_sample_launch(const int32_t* x0, int n_canvas, int V, const float* kappa,
                           uint32_t k0, uint32_t k1, int32_t* xt, hipStream_t stream) {
  const int R = n_canvas * DG_CANVAS;
  hipLaunchKernelGGL(k_q_sample, dim3((R + 255) / 256), dim3(256), 0, stream, x0, R, V, kappa,
                     k0, k1, xt);
  return hipGetLastError();
}

}  // namespace dg
