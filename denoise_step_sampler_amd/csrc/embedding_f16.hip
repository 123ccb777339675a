// The embedding as the expectation pass reads it: fp16, row-major, E16[v][k] = E[v][k] for
// v < V and 0 for V <= v < vp (vp = the vocabulary padded to whole 256-entry tiles).
//
// The self-conditioning expectation sum_v p_v E_v ("DiffusionGemma Technical Report" sec. 3.2
// eq. (6)) multiplies probability weights by E on fp16 MFMA: bf16 weights, 8 significant bits,
// leave a relative error of about 1e-3 in the expectation of a flat distribution (the rounding
// errors do not average down against the expectation's own size), against the 2e-3 bar of the
// pass; fp16 weights have 11.  The MFMA takes both operands in one format, so E comes as fp16
// too, in E's own layout (the pass stages 32-row slabs of it and forms B fragments with
// transpose reads).  Every bf16 E with |E| < 65504 converts with one rounding (values below
// 2^-14 become fp16 subnormals, absolute error at most 2^-25); the FP8 embedding's dequantised
// values 2^k value(code) likewise.
//
//   k_e16<false>  from bf16 E [V, d]
//   k_e16<true>   from E4M3 codes [V, d] and row exponents (2^k value(code))
// Elementwise, 8 entries (one 16-byte store) a thread; a grid-stride loop over the vp d / 8
// groups, rows past V written as zeros.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f16x2_bits(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// value(code) 2^k for an E4M3 code (no NaN codes are produced by the quantiser).
__device__ __forceinline__ float e4m3_scaled(uint32_t code, int k) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  const float v = e == 0 ? (float)m * 0x1p-9f
                         : (float)(8u + m) * __builtin_amdgcn_ldexpf(1.0f, (int)e - 10);
  const float w = __builtin_amdgcn_ldexpf(v, k);
  return (code & 0x80u) ? -w : w;
}

template <bool kF8>
__global__ __launch_bounds__(256) void k_e16(const void* src, const int32_t* kexp, int V, int d,
                                             size_t n_groups, uint16_t* E16) {
  const int gpr = d / 8;  // 8-entry groups a row
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_groups;
       i += (size_t)gridDim.x * 256) {
    const int v = (int)(i / (size_t)gpr);
    u32x4 y = {0u, 0u, 0u, 0u};
    if (v < V) {
      if constexpr (kF8) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(src) + 8 * i);
        const int k = kexp[v];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = x[j >> 1] >> (16 * (j & 1));
          y[j] = f16x2_bits(e4m3_scaled(w & 0xFFu, k), e4m3_scaled((w >> 8) & 0xFFu, k));
        }
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + 8 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          y[j] = f16x2_bits(__uint_as_float(x[j] << 16), __uint_as_float(x[j] & 0xFFFF0000u));
      }
    }
    *reinterpret_cast<u32x4*>(E16 + 8 * i) = y;
  }
}

template <bool kF8>
hipError_t launch(const void* src, const int32_t* kexp, int V, int d, uint16_t* E16,
                  hipStream_t stream) {
  const size_t n_groups = (size_t)e16_rows(V) * (size_t)(d / 8);
  const size_t blocks = (n_groups + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL((k_e16<kF8>), dim3(grid), dim3(256), 0, stream, src, kexp, V, d, n_groups,
                     E16);
  return hipGetLastError();
}

}  // namespace

hipError_t e16_launch(const uint16_t* E, int V, int d, uint16_t* E16, hipStream_t stream) {
  return launch<false>(E, nullptr, V, d, E16, stream);
}

hipError_t e16_fp8_launch(const uint8_t* codes, const int32_t* kexp, int V, int d, uint16_t* E16,
                          hipStream_t stream) {
  return launch<true>(codes, kexp, V, d, E16, stream);
}

}  // namespace dg
