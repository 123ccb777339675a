// Self-conditioning consumer for gfx950: the next decode step's input rows from the
// self-conditioning expectation sc = sum_v p_v E_v and the renoised tokens
// ("DiffusionGemma Explained", Self-conditioning and the decode forward; the conditioning MLP
// of its "MLP and mixture-of-experts block"; RMSNorm as in its "RMSNorm" section; Technical
// Report sec. 3.2 eq. (6), FFW(p_hat_0 E)):
//
//   x1  = bf16(w * cx * sqrt(D) / (||cx|| + eps)),  cx = sc * sqrt(D)      k_ffw_prenorm
//   y   = bf16((x1 W_up^T) * GELU(x1 W_gate^T))                           k_ffw_gemm<true>
//   res = y W_down^T  (fp32)                                              k_ffw_gemm<false>
//   out = bf16(x * sqrt(D) / (||x|| + eps)),  x = E[tok] sqrt(D) + res     k_ffw_out
//
// The two products are bf16 MFMA GEMMs (v_mfma_f32_32x32x16_bf16, fp32 accumulate) on
// 128 x 128 tiles of 256-thread workgroups, two per CU: operands are copied by LDS DMA in
// 64-element K chunks (one 128-byte line per row) into two 32 KB stages, XOR-swizzled so the
// fragment reads are conflict-free; the copy of chunk k + 1 runs under the MFMAs of chunk k.
// The gate and up projections share one tile: its 128 staged weight rows are 64 gate rows
// and the 64 up rows of the same features, so each lane holds the gate and up values of the
// same (row, feature) and the GELU product is formed in registers; only y (bf16) is written.
// Tiles are dealt to the eight XCDs in contiguous runs, so the workgroups of one XCD share
// the activation rows of a tile row through their L2.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kFM = 128;              // activation rows per tile
constexpr int kFN = 128;              // staged weight rows per tile
constexpr int kFK = 64;               // K chunk
constexpr int kFRow = 2 * kFK;        // bytes of one staged row
constexpr int kFBOff = kFM * kFRow;   // stage offset of the weight rows
constexpr int kFStage = (kFM + kFN) * kFRow;
constexpr int kRowsPerCanvas = 256;

// 16-byte slot of K segment q in staged row r is q ^ fswz(r): the sixteen rows one
// ds_read_b128 pass serves fall on distinct banks.
__device__ __forceinline__ int fswz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

struct FfwGemm {
  const uint16_t* A;    // [M, K] activations (x1 or y)
  const uint16_t* B0;   // [N, K] W_gate (gated) or W_down
  const uint16_t* B1;   // [N, K] W_up (gated)
  const uint8_t* commit;  // per canvas of 256 rows, or null
  int M, N, K;
  int n_mt, n_nt;       // tiles along M and N
  uint16_t* y;          // gated: [M, N] bf16
  float* res;           // plain: [M, N] fp32
};

// kGated: N tile of 64 features (64 gate + 64 up staged rows), output y; otherwise N tile of
// 128 output columns, output res.
template <bool kGated>
__global__ __launch_bounds__(256, 2) void k_ffw_gemm(FfwGemm g) {
  __shared__ __attribute__((aligned(1024))) char stg[2][kFStage];
  const int total = g.n_mt * g.n_nt;
  // contiguous runs of tiles per XCD (workgroup b runs on XCD b % 8)
  const int per = (total + 7) >> 3;
  const int q = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (q >= total) return;
  const int mt = q / g.n_nt, nt = q - mt * g.n_nt;
  const int m0 = mt * kFM;
  if (g.commit != nullptr && g.commit[m0 / kRowsPerCanvas]) return;
  constexpr int kNW = kGated ? 64 : 128;  // output columns per tile
  const int n0 = nt * kNW;
  const int M = g.M, N = g.N, K = g.K;
  const int t = threadIdx.x, lane = t & 63, fr = lane & 31, fh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w & 1, wn = w >> 1;
  const int nk = K / kFK;
  const uint32_t pitch = 2u * (uint32_t)K;

  // DMA sources: wave w copies activation rows and weight rows [32 w, 32 w + 32) of the
  // stage, four 8-row copies each; rows past the matrix repeat its last row (never stored).
  const int dlrow = lane >> 3;
  const char* abase;
  const char* bbase;
  uint32_t offA[4], offB[4];
  {
    const int ra0 = min(m0 + 32 * w, M - 1);
    abase = reinterpret_cast<const char*>(g.A) + (size_t)ra0 * pitch;
    const uint16_t* Bm;
    int rb_first;
    if (kGated) {
      Bm = w < 2 ? g.B0 : g.B1;
      rb_first = n0 + 32 * (w & 1);
    } else {
      Bm = g.B0;
      rb_first = n0 + 32 * w;
    }
    const int rb0 = min(rb_first, N - 1);
    bbase = reinterpret_cast<const char*>(Bm) + (size_t)rb0 * pitch;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lr = 8 * j + dlrow;  // row within the wave's 32
      const uint32_t slot = 16u * (uint32_t)((lane & 7) ^ fswz(lr));
      offA[j] = (uint32_t)(min(m0 + 32 * w + lr, M - 1) - ra0) * pitch + slot;
      offB[j] = (uint32_t)(min(rb_first + lr, N - 1) - rb0) * pitch + slot;
    }
  }
  uint32_t sa[2];
  sa[0] = (uint32_t)(uintptr_t)(lds_char*)stg[0];
  sa[1] = (uint32_t)(uintptr_t)(lds_char*)stg[1];
  auto issue = [&](int kc, uint32_t dst) {
    const uint32_t kb = (uint32_t)kc * (uint32_t)kFRow;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma_asm(abase + kb, offA[j], dst + 1024u * (uint32_t)(4 * w + j));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma_asm(bbase + kb, offB[j], dst + (uint32_t)kFBOff + 1024u * (uint32_t)(4 * w + j));
  };

  // fragment offsets (stage-relative) for the four 16-wide K steps of a chunk
  const int sw = fswz(fr);
  int browoff[2];
  if (kGated) {
    browoff[0] = 32 * wn;        // gate rows of this wave's 32 features
    browoff[1] = 64 + 32 * wn;   // the matching up rows
  } else {
    browoff[0] = 64 * wn;
    browoff[1] = 64 * wn + 32;
  }
  uint32_t rdA[4], rdB[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    rdA[ks] = (uint32_t)((64 * wm + fr) * kFRow + 16 * ((2 * ks + fh) ^ sw));
    rdB[ks] = (uint32_t)(kFBOff + (browoff[0] + fr) * kFRow + 16 * ((2 * ks + fh) ^ sw));
  }
  const uint32_t dB1 = (uint32_t)((browoff[1] - browoff[0]) * kFRow);

  f32x16 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{0};

  // fragments in two register sets: the reads of step ks + 1 are issued before the MFMAs of
  // step ks, and the last step of a chunk (its operands in registers) is multiplied after
  // the next barrier, behind the first reads of the next chunk
  u32x4 fa[2][2], fb[2][2];
  auto rd = [&](const lds_char* s, int ks, int q) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) fa[q][mb] = lds_read16(s + rdA[ks] + 32 * kFRow * mb);
    fb[q][0] = lds_read16(s + rdB[ks]);
    fb[q][1] = lds_read16(s + rdB[ks] + dB1);
  };
  auto mm = [&](int q) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[q][mb], fb[q][nb], acc[mb][nb]);
  };
  issue(0, sa[0]);
  for (int kc = 0; kc < nk; ++kc) {
    // chunk kc has landed (this wave's copies, then every wave's at the barrier), and every
    // wave is done reading chunk kc - 1, whose stage takes chunk kc + 1
    vm_wait<0>();
    __syncthreads();
    if (kc + 1 < nk) issue(kc + 1, sa[(kc + 1) & 1]);
    const lds_char* s = (const lds_char*)stg[kc & 1];
    rd(s, 0, 0);
    if (kc > 0) mm(1);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      rd(s, ks + 1, (ks + 1) & 1);
      mm(ks & 1);
    }
  }
  mm(1);

  // epilogue: lane holds column n = fr of each 32-wide block and rows acc32_m(i, lane)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = m0 + 64 * wm + 32 * mb + acc32_m(i, lane);
      if (row >= M) continue;
      if (kGated) {
        const int col = n0 + 32 * wn + fr;
        if (col < N) {
          const float gv = acc[mb][0][i], uv = acc[mb][1][i];
          g.y[(size_t)row * N + col] = (uint16_t)f32_to_bf16_bits(uv * gelu_erf(gv));
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + 64 * wn + 32 * nb + fr;
          if (col < N) g.res[(size_t)row * N + col] = acc[mb][nb][i];
        }
      }
    }
  }
}

// Block-wide sum over 256 threads (four waves).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_f(v, m);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

struct FfwRows {
  const float* sc;        // [R, D] or null
  const int32_t* tokens;  // [R]
  const uint16_t* E;      // [V, D]
  const uint16_t* pre_norm;  // [D]
  const uint8_t* commit;
  int R, V, D;
  float scale;            // sqrt(D)
  float eps;
  uint16_t* x1;           // [R, D]
  const float* res;       // [R, D] or null (first step)
  uint16_t* out;          // [R, D]
};

// x1 = bf16(w cx sqrt(D) / (||cx|| + eps)), cx = sc sqrt(D); one workgroup per row, four
// entries per thread and step (16-byte loads of sc, 8-byte loads of the weight and stores).
__global__ __launch_bounds__(256) void k_ffw_prenorm(FfwRows a) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  if (a.commit != nullptr && a.commit[r / kRowsPerCanvas]) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.sc + (size_t)r * a.D);
  const int n4 = a.D / 4;
  float ss = 0.0f;
  for (int k = threadIdx.x; k < n4; k += 256) {
    const f32x4 x = src[k] * a.scale;
    ss += (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
  }
  const float n = sqrtf(block_sum256(ss, red));
  const float f = a.scale / (n + a.eps);
  const u32x2* wp = reinterpret_cast<const u32x2*>(a.pre_norm);
  u32x2* dst = reinterpret_cast<u32x2*>(a.x1 + (size_t)r * a.D);
  for (int k = threadIdx.x; k < n4; k += 256) {
    const f32x4 x = src[k] * a.scale;
    const u32x2 w = wp[k];
    const uint32_t lo = f32_to_bf16_bits(bf16_lo(w[0]) * (x[0] * f)) |
                        (f32_to_bf16_bits(bf16_hi(w[0]) * (x[1] * f)) << 16);
    const uint32_t hi = f32_to_bf16_bits(bf16_lo(w[1]) * (x[2] * f)) |
                        (f32_to_bf16_bits(bf16_hi(w[1]) * (x[3] * f)) << 16);
    dst[k] = u32x2{lo, hi};
  }
}

// out = bf16(x sqrt(D) / (||x|| + eps)), x = E[tok] sqrt(D) + res; one workgroup per row, four
// entries per thread and step.  A token outside [0, V) gives a row of NaN.
__global__ __launch_bounds__(256) void k_ffw_out(FfwRows a) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  if (a.commit != nullptr && a.commit[r / kRowsPerCanvas]) return;
  const int tok = a.tokens[r];
  const int n4 = a.D / 4;
  u32x2* dst = reinterpret_cast<u32x2*>(a.out + (size_t)r * a.D);
  if (tok < 0 || tok >= a.V) {
    for (int k = threadIdx.x; k < n4; k += 256) dst[k] = u32x2{0x7FC07FC0u, 0x7FC07FC0u};
    return;
  }
  const u32x2* e = reinterpret_cast<const u32x2*>(a.E + (size_t)tok * a.D);
  const f32x4* rs = a.res ? reinterpret_cast<const f32x4*>(a.res + (size_t)r * a.D) : nullptr;
  auto load = [&](int k) {
    const u32x2 w = e[k];
    f32x4 x = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])} * a.scale;
    if (rs) x += rs[k];
    return x;
  };
  float ss = 0.0f;
  for (int k = threadIdx.x; k < n4; k += 256) {
    const f32x4 x = load(k);
    ss += (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
  }
  const float n = sqrtf(block_sum256(ss, red));
  const float f = a.scale / (n + a.eps);
  for (int k = threadIdx.x; k < n4; k += 256) {
    const f32x4 x = load(k) * f;
    dst[k] = u32x2{f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16),
                   f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16)};
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

FfwPlan ffw_plan(int n_canvas, int D, int F) {
  FfwPlan p{};
  p.R = (size_t)n_canvas * kRowsPerCanvas;
  p.off_x1 = 0;
  p.off_y = align256(p.off_x1 + p.R * (size_t)D * 2);
  p.off_res = align256(p.off_y + p.R * (size_t)F * 2);
  p.bytes = align256(p.off_res + p.R * (size_t)D * 4);
  return p;
}

hipError_t ffw_launch(const FfwArgs& a, const FfwPlan& p, void* workspace, hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  FfwRows rows{};
  rows.sc = a.sc;
  rows.tokens = a.tokens;
  rows.E = a.E;
  rows.pre_norm = a.pre_norm;
  rows.commit = a.commit;
  rows.R = (int)p.R;
  rows.V = a.V;
  rows.D = a.D;
  rows.scale = sqrtf((float)a.D);
  rows.eps = a.eps;
  rows.x1 = reinterpret_cast<uint16_t*>(ws + p.off_x1);
  rows.res = nullptr;
  rows.out = a.out;
  if (a.sc != nullptr) {
    uint16_t* y = reinterpret_cast<uint16_t*>(ws + p.off_y);
    float* res = reinterpret_cast<float*>(ws + p.off_res);
    hipLaunchKernelGGL(k_ffw_prenorm, dim3((unsigned)p.R), dim3(256), 0, stream, rows);
    FfwGemm g{};
    g.A = rows.x1;
    g.B0 = a.W_gate;
    g.B1 = a.W_up;
    g.commit = a.commit;
    g.M = (int)p.R;
    g.N = a.F;
    g.K = a.D;
    g.n_mt = (g.M + kFM - 1) / kFM;
    g.n_nt = (a.F + 63) / 64;
    g.y = y;
    unsigned grid = (unsigned)(8 * ((g.n_mt * g.n_nt + 7) / 8));
    hipLaunchKernelGGL(k_ffw_gemm<true>, dim3(grid), dim3(256), 0, stream, g);
    FfwGemm h{};
    h.A = y;
    h.B0 = a.W_down;
    h.commit = a.commit;
    h.M = (int)p.R;
    h.N = a.D;
    h.K = a.F;
    h.n_mt = g.n_mt;
    h.n_nt = (a.D + 127) / 128;
    h.res = res;
    grid = (unsigned)(8 * ((h.n_mt * h.n_nt + 7) / 8));
    hipLaunchKernelGGL(k_ffw_gemm<false>, dim3(grid), dim3(256), 0, stream, h);
    rows.res = res;
  }
  hipLaunchKernelGGL(k_ffw_out, dim3((unsigned)p.R), dim3(256), 0, stream, rows);
  return hipGetLastError();
}

}  // namespace dg
