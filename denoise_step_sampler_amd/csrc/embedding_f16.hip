// The embedding as the expectation pass reads it: fp16, in the B-fragment order of
// v_mfma_f32_16x16x32_f16.  For the entry block b (entries 32 b .. 32 b + 31, zero past V, the
// vocabulary padded to whole 256-entry tiles) and the column block c (columns 16 c .. 16 c + 15)
// the 1 KB block at byte (b d / 16 + c) * 1024 holds, in its 16 bytes number n + 16 g, column
// 16 c + n of entries 32 b + 8 g .. + 7: one fragment is one lane-contiguous 16-byte read, and
// the blocks one chunk of the pass needs (one entry block, consecutive column blocks) are one
// contiguous run.
//
// The self-conditioning expectation sum_v p_v E_v ("DiffusionGemma Technical Report" sec. 3.2
// eq. (6)) multiplies probability weights by E on fp16 MFMA: bf16 weights, 8 significant bits,
// leave a relative error of about 1e-3 in the expectation of a flat distribution (the rounding
// errors do not average down against the expectation's own size), against the 2e-3 bar of the
// pass; fp16 weights have 11.  The MFMA takes both operands in one format, so E comes as fp16
// too.  Every bf16 E with |E| < 65504 converts with one rounding (values below 2^-14 become fp16
// subnormals, absolute error at most 2^-25); the FP8 embedding's dequantised values
// 2^k value(code) likewise.
//
//   k_e16<false>  from bf16 E [V, d]
//   k_e16<true>   from E4M3 codes [V, d] and row exponents (2^k value(code))
// One 256-thread workgroup per (entry block, 128 columns): the 32 x 128 tile through LDS, read
// and written as 16-byte pieces (8 blocks of 1 KB written contiguously).
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
__global__ __launch_bounds__(256) void k_e16(const void* src, const int32_t* kexp, int V, int d,
                                             uint16_t* E16) {
  __shared__ uint16_t tile[32][128 + 8];  // entries x columns (rows padded against conflicts)
  const int b = blockIdx.x, c0 = blockIdx.y * 8;  // entry block, first column block
  const int t = threadIdx.x;
  // load: 32 rows x 128 columns, 8 entries (16 bytes of fp16) a piece, two pieces a thread
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = t + 256 * p;
    const int r = q >> 4, c8 = (q & 15) * 8;  // row in the block, first column of the piece
    const int v = 32 * b + r;
    uint16_t out[8];
    if (v < V) {
      const size_t off = (size_t)v * d + 16 * c0 + c8;
      if constexpr (kF8) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(src) + off);
        const int k = kexp[v];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = f16_bits(e4m3_scaled((x[i >> 2] >> (8 * (i & 3))) & 0xFFu, k));
      } else {
        const u16x8 x = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(src) + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = f16_bits(__uint_as_float((uint32_t)x[i] << 16));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[r][c8 + i] = out[i];
  }
  __syncthreads();
  // store: block c0 + cb, lane n + 16 g <- column 16 cb + n, entries 8 g .. 8 g + 7
  uint16_t* dst = E16 + ((size_t)b * (d / 16) + c0) * 512;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = t + 256 * p;               // 16-byte piece q of the 8 KB run
    const int cb = q >> 6, l = q & 63, n = l & 15, gq = l >> 4;
    u16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = tile[8 * gq + e][16 * cb + n];
    *reinterpret_cast<u16x8*>(dst + 8 * q) = y;
  }
}

template <bool kF8>
hipError_t launch(const void* src, const int32_t* kexp, int V, int d, uint16_t* E16,
                  hipStream_t stream) {
  const dim3 grid((unsigned)(e16_rows(V) / 32), (unsigned)(d / 128));
  hipLaunchKernelGGL((k_e16<kF8>), grid, dim3(256), 0, stream, src, kexp, V, d, E16);
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
