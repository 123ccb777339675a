// FP8 embedding: OCP E4M3 codes with one power-of-two scale 2^k per row (the vLLM blog's FP8
// checkpoint; the pages give no scale scheme).  k is the smallest integer >= -117 with
// max |E_row| <= 448 * 2^k; a code is the E4M3 value nearest to E / 2^k, ties to the even code.
// A power-of-two scale makes every dequantised value 2^k * value(code) an exact bf16 number,
// so the vocabulary pass on the FP8 embedding is the bf16 pass on its dequantised rows.
//
//   k_fp8_quantize    one wave per row: the row's |max|, k from its exponent field, codes
// (The expectation pass's fp16 operand is built from the codes by e16_fp8_launch.)
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kKMin = -117;

// Nearest E4M3 code of x, |x| <= 448, ties to the even code; zero (of either sign) -> 0x00.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = u >> 31, a = u & 0x7FFFFFFFu;
  if (a == 0) return 0;
  const int e = (int)(a >> 23) - 127;
  uint32_t code;
  if (e < -6) {
    // below the smallest normal 2^-6: multiples of 2^-9, rounded half to even by rintf
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    uint32_t r = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    uint32_t ee = (uint32_t)(e + 7);
    if (r == 8) {
      r = 0;
      ++ee;
    }
    code = (ee << 3) | r;
  }
  return code == 0 ? 0 : (code | (s << 7));
}

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void k_fp8_quantize(const uint16_t* E, int V, int d,
                                                      uint8_t* codes, int32_t* kexp) {
  const int lane = threadIdx.x & 63;
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= V) return;
  const u16x8* row = reinterpret_cast<const u16x8*>(E + (size_t)v * d);
  uint32_t amax = 0;  // |bf16| bits: the order of the magnitudes
  for (int j = lane; j < d / 8; j += 64) {
    const u16x8 x = row[j];
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = max(amax, (uint32_t)(x[i] & 0x7FFFu));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, m, 64));
  // smallest k with amax <= 448 2^k = 0.875 2^(9 + k): amax = f 2^ea with f in [0.5, 1)
  int k = kKMin;
  if (amax >= 0x0080u) {  // a normal |max| (below 2^-126 the floor applies)
    int ea;
    const float f = frexpf(__uint_as_float(amax << 16), &ea);
    k = max(f <= 0.875f ? ea - 9 : ea - 8, kKMin);
  }
  if (lane == 0) kexp[v] = k;
  uint8_t* out = codes + (size_t)v * d;
  for (int j = lane; j < d / 8; j += 64) {
    const u16x8 x = row[j];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_code(__builtin_amdgcn_ldexpf(__uint_as_float((uint32_t)x[i] << 16), -k)) << (8 * i);
      hi |= e4m3_code(__builtin_amdgcn_ldexpf(__uint_as_float((uint32_t)x[4 + i] << 16), -k))
            << (8 * i);
    }
    *reinterpret_cast<u32x2*>(out + 8 * j) = u32x2{lo, hi};
  }
}

}  // namespace

hipError_t fp8_quantize_launch(const uint16_t* E, int V, int d, uint8_t* codes, int32_t* kexp,
                               hipStream_t stream) {
  hipLaunchKernelGGL(k_fp8_quantize, dim3((unsigned)((V + 3) / 4)), dim3(256), 0, stream, E, V,
                     d, codes, kexp);
  return hipGetLastError();
}

}  // namespace dg
