// The DiffusionGemma-Lite sampler step (DiffusionGemma-Lite, section 4.2 "The commit rule",
// section 4.4 "Entropy-bounded adaptive stopping") on the vocabulary pass outputs:
//
//   k_lite_conf  conf_r = exp(z_am - lse_r), the probability of the row's argmax token under
//                the (capped) distribution the pass's statistics describe; z_am = S_am / T_c
//                with T_c the statistics temperature (1 for the page's untempered posterior
//                p = softmax(logits); the annealed tau(k) enters only the pass's x0-hat draw)
//                and S_am = h_r . E[am] recomputed as one 2d-byte dot product per row (one
//                wave per row, 16-byte loads, fp32 accumulation), since the pass keeps only the
//                argmax's index.
//   k_lite_step  one workgroup per canvas, one thread per position: the unchanged-or-stronger
//                commit (argmax == prev or conf >= prev_conf), frozen commits, uniform
//                redraw of the rest, the returned canvas, and the entropy-only stop counter
//                on the fp64 mean entropy.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kC = DG_CANVAS;

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void k_lite_conf(LiteArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.R) return;
  const int am = a.argmax_tok[r];
  if (am < 0 || am >= a.V) {
    if (lane == 0) a.conf[r] = __builtin_nanf("");
    return;
  }
  const u16x8* hp = reinterpret_cast<const u16x8*>(a.h + (size_t)r * a.d);
  const u16x8* ep = reinterpret_cast<const u16x8*>(a.E + (size_t)am * a.d);
  float s = 0.0f;
  for (int k = lane; k < a.d / 8; k += 64) {
    const u16x8 x = hp[k], y = ep[k];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      s += __uint_as_float((uint32_t)x[j] << 16) * __uint_as_float((uint32_t)y[j] << 16);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += xor_f(s, m);
  if (lane == 0) {
    const int c = r / kC;
    const float capped = a.softcap > 0.0f ? a.softcap * tanhf(s / a.softcap) : s;
    a.conf[r] = expf(capped / a.temperature[c] - a.lse[r]);
  }
}

__global__ __launch_bounds__(kC) void k_lite_step(LiteArgs a) {
  __shared__ float sH[kC];
  const int c = blockIdx.x;
  const int t = threadIdx.x;
  const int r = c * kC + t;
  const int am = a.argmax_tok[r];
  const float cf = a.conf[r];
  const bool was = a.committed[r] != 0;
  const bool commit = (am == a.prev_argmax[r]) || (cf >= a.prev_conf[r]);
  const bool fresh = commit && !was;
  const int draw = a.gumbel_tok[r];
  int x;
  if (fresh) {
    x = draw;
  } else if (was) {
    x = a.x[r];
  } else {
    const u32x4 wd = philox4x32_10(u32x4{0u, (uint32_t)r, (uint32_t)a.step[c], kTagRenoise},
                                   a.k0, a.k1);
    x = uniform_token(wd[0], (uint32_t)a.V);
  }
  const bool now = was || fresh;
  a.x[r] = x;
  a.committed[r] = now ? 1 : 0;
  if (a.final_tokens) a.final_tokens[r] = now ? x : draw;
  a.prev_argmax[r] = am;
  a.prev_conf[r] = cf;
  sH[t] = a.entropy[r];
  __syncthreads();
  if (t == 0) {
    double sum = 0.0;
    for (int j = 0; j < kC; ++j) sum += (double)sH[j];
    const double mean = sum / kC;
    if (a.mean_entropy) a.mean_entropy[c] = (float)mean;
    if (a.stability_steps > 0) {
      const int cnt = mean < (double)a.threshold ? a.stable_count[c] + 1 : 0;
      a.stable_count[c] = cnt;
      a.converged[c] = cnt >= a.stability_steps ? 1 : 0;
    } else {
      a.converged[c] = 0;
    }
  }
}

}  // namespace

hipError_t lite_step_launch(const LiteArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_lite_conf, dim3((unsigned)((a.R + 3) / 4)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(k_lite_step, dim3((unsigned)(a.R / kC)), dim3(kC), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dg
