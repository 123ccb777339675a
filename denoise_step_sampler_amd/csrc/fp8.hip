// FP8 embedding: OCP E4M3 codes with one power-of-two scale 2^k per row (the vLLM blog's FP8
// checkpoint; the pages give no scale scheme).  k is the smallest integer >= -117 with
// max |E_row| <= 448 * 2^k; a code is the E4M3 value nearest to E / 2^k, ties to the even code.
// A power-of-two scale makes every dequantised value 2^k * value(code) an exact bf16 number,
// so the vocabulary pass on the FP8 embedding is the bf16 pass on its dequantised rows.
//
//   k_fp8_quantize    one wave per row: the row's |max|, k from its exponent field, codes
//   k_fp8_dequantize  16 codes per thread to 16 bf16 (exact), 32-byte stores
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

// 2^k * value(code) as bf16 bits (exact: at most four significant bits, a normal number).
__device__ __forceinline__ uint32_t e4m3_bf16(uint32_t code, int k) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  const float v = e == 0 ? (float)m * 0x1p-9f : (float)(8u + m) * __builtin_amdgcn_ldexpf(1.0f, (int)e - 10);
  const float w = __builtin_amdgcn_ldexpf(v, k);
  return (__float_as_uint(w) >> 16) | ((code & 0x80u) << 8);
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

__global__ __launch_bounds__(256) void k_fp8_dequantize(const uint8_t* codes, const int32_t* kexp,
                                                        int V, int d, uint16_t* E) {
  const size_t n16 = (size_t)V * d / 16;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const int v = (int)((i * 16) / (size_t)d);
  const int k = kexp[v];
  const u32x4 c = reinterpret_cast<const u32x4*>(codes)[i];
  u32x4 o0, o1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = c[q];
    const uint32_t b0 = e4m3_bf16(w & 0xFFu, k), b1 = e4m3_bf16((w >> 8) & 0xFFu, k);
    const uint32_t b2 = e4m3_bf16((w >> 16) & 0xFFu, k), b3 = e4m3_bf16(w >> 24, k);
    const uint32_t p01 = b0 | (b1 << 16), p23 = b2 | (b3 << 16);
    if (q < 2) {
      o0[2 * q] = p01;
      o0[2 * q + 1] = p23;
    } else {
      o1[2 * (q - 2)] = p01;
      o1[2 * (q - 2) + 1] = p23;
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(E) + 2 * i;
  dst[0] = o0;
  dst[1] = o1;
}

// codesT[k][v] = codes[v][k] for a 64 x 64 block of (v, k) per workgroup, through LDS; the
// rows of codesT have pitch vp (a multiple of 256), entries v >= V are written as 0.
__global__ __launch_bounds__(256) void k_fp8_transpose(const uint8_t* codes, int V, int d, int vp,
                                                       uint8_t* codesT) {
  __shared__ uint8_t tile[64][64 + 16];
  const int v0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  const int t = threadIdx.x;
  {
    const int r = t >> 2, q = t & 3;  // row v0 + r, 16 bytes q of its 64
    u32x4 x = u32x4{0, 0, 0, 0};
    if (v0 + r < V) x = *reinterpret_cast<const u32x4*>(codes + (size_t)(v0 + r) * d + k0 + 16 * q);
#pragma unroll
    for (int b = 0; b < 16; ++b) tile[r][16 * q + b] = (uint8_t)(x[b >> 2] >> (8 * (b & 3)));
  }
  __syncthreads();
  {
    const int kk = t >> 2, q = t & 3;  // row k0 + kk of codesT, entries v0 + 16 q .. + 15
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= (uint32_t)tile[16 * q + 4 * j + b][kk] << (8 * b);
      y[j] = w;
    }
    *reinterpret_cast<u32x4*>(codesT + (size_t)(k0 + kk) * vp + v0 + 16 * q) = y;
  }
}

}  // namespace

hipError_t fp8_transpose_launch(const uint8_t* codes, int V, int d, uint8_t* codesT,
                                hipStream_t stream) {
  const int vp = fp8_transposed_pitch(V);
  hipLaunchKernelGGL(k_fp8_transpose, dim3((unsigned)(vp / 64), (unsigned)(d / 64)), dim3(256), 0,
                     stream, codes, V, d, vp, codesT);
  return hipGetLastError();
}

hipError_t fp8_quantize_launch(const uint16_t* E, int V, int d, uint8_t* codes, int32_t* kexp,
                               hipStream_t stream) {
  hipLaunchKernelGGL(k_fp8_quantize, dim3((unsigned)((V + 3) / 4)), dim3(256), 0, stream, E, V,
                     d, codes, kexp);
  return hipGetLastError();
}

hipError_t fp8_dequantize_launch(const uint8_t* codes, const int32_t* kexp, int V, int d,
                                 uint16_t* E, hipStream_t stream) {
  const size_t n16 = (size_t)V * d / 16;
  hipLaunchKernelGGL(k_fp8_dequantize, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream,
                     codes, kexp, V, d, E);
  return hipGetLastError();
}

}  // namespace dg
