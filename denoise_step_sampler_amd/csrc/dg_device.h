// Device-side helpers for the gfx950 kernels: vector types, MFMA accumulator layout,
// Philox4x32-10, the noise maps, bf16 packing and wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Stream tags of the Philox counters (fourth counter word).
constexpr uint32_t kTagGumbel = 0x47554D42u;
constexpr uint32_t kTagRenoise = 0x52454E4Fu;
constexpr uint32_t kTagQSample = 0x51534D50u;

// ---------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64-bit
// multiplications by fixed odd constants, the high halves mixed into the other two words
// with the round key; the key advances by the Weyl constants between rounds.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c.z;
    u32x4 n;
    // three-way XORs as one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
    n.x = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96);
    n.y = (uint32_t)p1;
    n.z = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96);
    n.w = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Uniform token in [0, V): floor(x * V / 2^32).
__device__ __forceinline__ int uniform_token(uint32_t x, uint32_t V) {
  return (int)__umulhi(x, V);
}

// Hardware base-2 log / exp (v_log_f32, v_exp_f32).
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Gumbel noise in base-2 units up to a constant: for the 32-bit word x with
// u = ((x >> 9) + 0.5) 2^-23 the Gumbel value is g = -ln(-ln u), and
//   g log2(e) = -log2(-log2 u) - log2(ln 2);
// this returns -log2(-log2 u), i.e. g log2(e) shifted by the constant log2(ln 2), which
// leaves every argmax of z log2(e) + noise unchanged.  Both logarithms are the hardware
// log2 (v_log_f32), whose result is within about 1e-7 relative for every u of this form,
// u near 1 included (measured on gfx950 against fp64), so the large Gumbel values that
// decide the sample keep full relative precision.
__device__ __forceinline__ float gumbel2s_from_word(uint32_t x) {
  // (x >> 9) 2^-23 + 2^-24, exactly: alignbit(0x7F, x, 9) = 0x3F800000 | (x >> 9) is the float
  // 1 + (x >> 9) 2^-23, and subtracting 1 - 2^-24 from a number in [1, 2) is exact (the two are
  // within a factor of two of each other)
  const float u = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, x, 9)) - (1.0f - 0x1p-24f);
  return -hw_log2(-hw_log2(u));
}

// a * b and a - b, each rounded on its own.  The device library's __fmul_rn / __fsub_rn are
// plain operators compiled where contraction is allowed, so a product followed by a
// difference would become one fma (one rounding) whatever pragma surrounds the call; these
// carry no contraction permission, so the pair keeps both roundings.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float sub_rn(float a, float b) {
#pragma clang fp contract(off)
  return a - b;
}

// ---------------------------------------------------------------------------------------
// bf16 packing, round to nearest even (inputs finite).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two floats to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}
// acc + the two bf16 halves of w (one v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(float acc, uint32_t w) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }

// Two floats to packed fp16, round to nearest even (one v_cvt_pk_f16_f32); finite inputs
// below 2^-24 in magnitude round to zero, below 2^-14 to subnormals.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}
// acc + the two fp16 halves of w (one v_dot2c_f32_f16 against (1, 1)).
__device__ __forceinline__ float add_f16x2(float acc, uint32_t w) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
}
// x rounded to fp16 (nearest even) and back: the value an fp16 weight holds.
__device__ __forceinline__ float round_f16(float x) { return (float)(_Float16)x; }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------------------
// MFMA v_mfma_f32_32x32x16_bf16.  Operand fragments: lane l holds 8 consecutive K values of
// row (l % 32) of A (M x K) and of column (l % 32) of B (K x N), K half (l / 32).  The same
// K slots are used for A and B, so the product is the full K = 16 sum.
// Accumulator: lane l, element i holds D[m][n] with n = l % 32 and
// m = 8 (i / 4) + 4 (l / 32) + (i % 4).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ int acc32_m(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// ---------------------------------------------------------------------------------------
// Wave64 reductions.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

// (value, index) pair: larger value wins, ties go to the smaller index.
// Running argmax over entries met in increasing index order: a later entry replaces the
// current one only when strictly larger, which keeps the smallest index among equal values.
__device__ __forceinline__ void argmax_next(float& v, int& i, float v2, int i2) {
  const bool take = v2 > v;
  v = take ? v2 : v;
  i = take ? i2 : i;
}
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  const bool take = (v2 > v) | ((v2 == v) & (i2 < i));  // branch-free: selects, no exec masks
  v = take ? v2 : v;
  i = take ? i2 : i;
}

// Online-softmax partial in base-2 units: max m, l = sum 2^(z-m), a = sum 2^(z-m) (z-m).
__device__ __forceinline__ void lse_merge(float& m, float& l, float& a, float m2, float l2,
                                          float a2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // both empty
  const float d1 = m - M, d2 = m2 - M;
  const float s1 = (m == -INFINITY) ? 0.0f : hw_exp2(d1);
  const float s2 = (m2 == -INFINITY) ? 0.0f : hw_exp2(d2);
  const float t1 = (m == -INFINITY) ? 0.0f : s1 * (a + d1 * l);
  const float t2 = (m2 == -INFINITY) ? 0.0f : s2 * (a2 + d2 * l2);
  l = s1 * l + s2 * l2;
  a = t1 + t2;
  m = M;
}

// ---------------------------------------------------------------------------------------
// LDS access and LDS DMA (global_load_lds_dwordx4: 64 lanes x 16 bytes = one 1 KB copy).
// ---------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ u32x4 lds_read16(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}


// LDS DMA issued as inline assembly: the compiler does not see these copies, so it neither
// waits for them before unrelated LDS reads (it cannot tell the two stages apart for the
// transpose reads) nor counts them; the kernel waits for them explicitly (vm_wait) before the
// barrier that publishes a stage.  base is wave-uniform, off per lane, dst the wave-uniform
// LDS address of the 1 KB destination; the one-cycle nop covers the M0 -> LDS DMA hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_asm(const void* base, uint32_t off, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(dst)
               : "m0");
}
#pragma clang diagnostic pop

// A pointer the caller knows to be the same in every lane, read from the first lane (keeps an
// address the compiler would otherwise hold per lane in scalar registers, as dma_asm needs).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}


}  // namespace dg
