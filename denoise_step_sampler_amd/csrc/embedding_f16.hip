// The embedding as the expectation pass reads it: fp16, transposed, E16T[k][v] = E[v][k] for
// v < V and 0 for V <= v < vp (vp = the vocabulary padded to whole 256-entry tiles).
//
// The self-conditioning expectation sum_v p_v E_v ("DiffusionGemma Technical Report" sec. 3.2
// eq. (6)) multiplies probability weights by E on fp16 MFMA: bf16 weights, 8 significant bits,
// leave a relative error of about 1e-3 in the expectation of a flat distribution (the rounding
// errors do not average down against the expectation's own size), against the 2e-3 bar of the
// pass; fp16 weights have 11.  The MFMA takes both operands in one format, so E comes as fp16
// too, transposed so that a B fragment (eight consecutive vocabulary entries of one column) is
// one 16-byte read.  Every bf16 E with |E| < 65504 converts with one rounding (values below
// 2^-14 become fp16 subnormals, absolute error at most 2^-25); the FP8 embedding's dequantised
// values 2^k value(code) likewise.
//
//   k_e16t<false>  from bf16 E [V, d]
//   k_e16t<true>   from E4M3 codes [V, d] and row exponents (2^k value(code))
// One workgroup per 64 x 64 block of (v, k): 16 entries a thread into an LDS tile, then 16
// entries of one transposed row a thread, as two 16-byte stores.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
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
__global__ __launch_bounds__(256) void k_e16t(const void* src, const int32_t* kexp, int V, int d,
                                              int vp, uint16_t* E16T) {
  __shared__ uint16_t tile[64][64 + 2];
  const int v0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  {
    const int r = t >> 2, q = t & 3;  // entries (v0 + r, k0 + 16 q .. + 15)
    const int v = v0 + r;
    uint16_t out[16];
    if (v < V) {
      if constexpr (kF8) {
        const uint8_t* c = static_cast<const uint8_t*>(src) + (size_t)v * d + k0 + 16 * q;
        const u32x4 x = *reinterpret_cast<const u32x4*>(c);
        const int k = kexp[v];
#pragma unroll
        for (int b = 0; b < 16; ++b) out[b] = f16_bits(e4m3_scaled((x[b >> 2] >> (8 * (b & 3))) & 0xFFu, k));
      } else {
        const uint16_t* e = static_cast<const uint16_t*>(src) + (size_t)v * d + k0 + 16 * q;
        const u16x8 a = *reinterpret_cast<const u16x8*>(e);
        const u16x8 b = *reinterpret_cast<const u16x8*>(e + 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          out[i] = f16_bits(__uint_as_float((uint32_t)a[i] << 16));
          out[8 + i] = f16_bits(__uint_as_float((uint32_t)b[i] << 16));
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 16; ++b) out[b] = 0;
    }
#pragma unroll
    for (int b = 0; b < 16; ++b) tile[r][16 * q + b] = out[b];
  }
  __syncthreads();
  {
    const int kk = t >> 2, q = t & 3;  // transposed row k0 + kk, entries v0 + 16 q .. + 15
    u32x4 y0, y1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y0[j] = (uint32_t)tile[16 * q + 2 * j][kk] | ((uint32_t)tile[16 * q + 2 * j + 1][kk] << 16);
      y1[j] = (uint32_t)tile[16 * q + 8 + 2 * j][kk] |
              ((uint32_t)tile[16 * q + 8 + 2 * j + 1][kk] << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(E16T + (size_t)(k0 + kk) * vp + v0 + 16 * q);
    dst[0] = y0;
    dst[1] = y1;
  }
}

}  // namespace

hipError_t e16t_launch(const uint16_t* E, int V, int d, uint16_t* E16T, hipStream_t stream) {
  const int vp = e16t_pitch(V);
  hipLaunchKernelGGL((k_e16t<false>), dim3((unsigned)(vp / 64), (unsigned)(d / 64)), dim3(256),
                     0, stream, static_cast<const void*>(E), nullptr, V, d, vp, E16T);
  return hipGetLastError();
}

hipError_t e16t_fp8_launch(const uint8_t* codes, const int32_t* kexp, int V, int d,
                           uint16_t* E16T, hipStream_t stream) {
  const int vp = e16t_pitch(V);
  hipLaunchKernelGGL((k_e16t<true>), dim3((unsigned)(vp / 64), (unsigned)(d / 64)), dim3(256), 0,
                     stream, static_cast<const void*>(codes), kexp, V, d, vp, E16T);
  return hipGetLastError();
}

}  // namespace dg
