// Per-canvas entropy-bounded acceptance, uniform renoising and argmax-stability convergence
// (Technical Report part 2/6 sec. 3.3; DiffusionGemma Explained, "Sampling"; vLLM blog,
// sampler step).  One workgroup of 256 threads per canvas, one thread per position.
//
// The positions are ordered by the 64-bit key (orderable entropy bits << 32 | position)
// with a workgroup bitonic sort in LDS, which makes the order unique and stable by
// position.  Each thread then forms the exclusive prefix of the sorted entropies by a
// left-to-right fp64 sum (the reference order, so the acceptance threshold test sees the
// same prefix value for every rank).
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kC = DG_CANVAS;

__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kC) void k_accept_renoise(AcceptArgs a) {
  __shared__ unsigned long long keys[kC];
  __shared__ double sortedH[kC];
  __shared__ float sH[kC];
  __shared__ int s_diff;
  const int c = blockIdx.x;
  const int t = threadIdx.x;
  const int r = c * kC + t;
  const int am = a.argmax_tok[r];

  if (a.commit != nullptr && a.commit[c] != 0) {
    a.next_tokens[r] = am;
    if (a.accept_mask) a.accept_mask[r] = 1;
    a.prev_argmax[r] = -1;
    if (t == 0) {
      a.stable_count[c] = 0;
      a.converged[c] = 0;
    }
    return;
  }

  const float H = a.entropy[r];
  sH[t] = H;
  keys[t] = ((unsigned long long)orderable(H) << 32) | (unsigned)t;
  if (t == 0) s_diff = 0;
  __syncthreads();

  // bitonic sort, ascending
  for (int k = 2; k <= kC; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int p = t ^ j;
      if (p > t) {
        const unsigned long long x = keys[t], y = keys[p];
        const bool up = (t & k) == 0;
        if ((x > y) == up) {
          keys[t] = y;
          keys[p] = x;
        }
      }
      __syncthreads();
    }
  }
  sortedH[t] = (double)sH[(int)(keys[t] & 0xFFFFFFFFull)];
  __syncthreads();

  // exclusive prefix of rank t, summed left to right in fp64
  double before = 0.0;
  for (int j = 0; j < t; ++j) before += sortedH[j];
  const int pos = (int)(keys[t] & 0xFFFFFFFFull);
  const bool acc = before <= (double)a.budget;
  const int rp = c * kC + pos;
  int nxt;
  if (acc) {
    nxt = a.gumbel_tok[rp];
  } else {
    const u32x4 wd = philox4x32_10(u32x4{0u, (uint32_t)rp, (uint32_t)a.step[c], kTagRenoise},
                                   a.k0, a.k1);
    nxt = uniform_token(wd[0], (uint32_t)a.V);
  }
  a.next_tokens[rp] = nxt;
  if (a.accept_mask) a.accept_mask[rp] = acc ? 1 : 0;

  // argmax stability
  const int prev = a.prev_argmax[r];
  if (prev != am) atomicOr(&s_diff, 1);
  __syncthreads();
  a.prev_argmax[r] = am;
  if (t == 0) {
    double sum = 0.0;
    for (int j = 0; j < kC; ++j) sum += (double)sH[j];
    const double mean = sum / kC;
    const int cnt = (s_diff == 0) ? a.stable_count[c] + 1 : 0;
    a.stable_count[c] = cnt;
    a.converged[c] = (cnt >= a.stability && mean < (double)a.confidence) ? 1 : 0;
    if (a.mean_entropy) a.mean_entropy[c] = (float)mean;
  }
}

}  // namespace

hipError_t accept_renoise_launch(const AcceptArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_accept_renoise, dim3(a.n_canvas), dim3(kC), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dg
