// Vocabulary pass as two streamed GEMMs for gfx950.
//
// The pass computes, per row r of h and temperature T_c of its canvas c, the logits
// S = h E^T (tied unembedding, "DiffusionGemma Technical Report" sec. 3.2 eq. (5)), the
// tempered softmax p = softmax(S / T_c) with its log-partition and entropy ("DiffusionGemma
// Explained", Sampling), the argmax of S and the Gumbel-max sample argmax(S / T_c + g) (the
// vLLM sampler step), and the self-conditioning expectation sum_v p_v E_v (eq. (6) of the
// report, the argument of FFW).  d = 2816 makes the expectation's accumulator of one
// canvas 256 x 2816 fp32 (2.9 MB): it cannot live beside the logits tile in one CU, so the
// pass runs as two contractions over the same E:
//
//   k_gemm_logits   S^T tile = E_t h_c^T (256 vocabulary x 256 rows of one canvas, bf16
//                   MFMA 32x32x16, fp32 accumulate over all of d) and its epilogue: per row
//                   and 128-entry half tile the integer reference ref = ceil(max z2)
//                   (z2 = S log2(e) / T), the online-softmax partial (sum 2^(z2 - ref),
//                   entropy moment), argmax and Philox Gumbel key; the weights 2^(z2 - ref)
//                   in (0, 1] go to memory as fp16 (one rounding), with the reference beside
//                   them.  The fp32 logits never leave the registers.
//   k_gemm_selfcond acc[256 rows, BN columns] += P~ E over one vocabulary range (fp16 MFMA
//                   16x16x32 on the weights and the fp16 embedding), each half tile's weights
//                   scaled by a power of two to a common unit of the row.
//   k_gemm_rows     per row: merges the statistic partials (max/sum/moment merge of the
//                   chunked logsumexp in "DiffusionGemma-Lite", (value, -index) max for the
//                   tokens), corrects the four largest weights' fp16 rounding exactly and
//                   forms the range weights 2^(U_s - m) / lb of the expectation partials;
//   k_gemm_sc       per row and column: the weighted sum of the expectation partials.
//
// Both GEMMs run 512-thread workgroups (one per CU) on 256 x 256 tiles and stage their
// operands through LDS by LDS DMA (global_load_lds_dwordx4, 1 KB per instruction, issued as
// inline assembly with explicit vmcnt waits): the logits pass in two stages of 64-element K
// chunks (each chunk's copies issued one chunk ahead), the expectation pass in four stages of
// 32-entry chunks (three ahead).  Work is mapped to the eight XCDs so that the CUs of one XCD
// share operands through their L2: the logits pass runs up to eight canvases per XCD over the
// same vocabulary tiles (each E line is read by all of them) while the XCDs of a canvas group
// split the vocabulary; the expectation pass runs the column blocks of one (range, canvas)
// pair on one XCD (the weights are read once from memory, E of the range by every canvas of
// the XCD).
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4v __attribute__((ext_vector_type(4)));

constexpr int kTile = 256;      // vocabulary tile of the logits pass (and rows per canvas)
constexpr int kHalf = 128;      // granularity of the weight references
constexpr int kWG = 256;        // workgroups per round of the logits pass
constexpr int kFacStride = 72;  // floats per row of the combine's weights
constexpr int kRoundMax = 32;   // canvases per round of the logits pass (four per XCD)

// ---------------------------------------------------------------------------------------
// Schedule of the logits pass.  Canvases are taken in `order` (non-commit first) in rounds
// of g = a power of two <= kRoundMax; a round gives each canvas L = 256 / g vocabulary
// lanes, and lane l of a canvas processes tiles l, l + L, l + 2L, ...  Workgroup b runs on
// XCD b % 8 (the dispatcher deals workgroups to the XCDs round-robin), slot b / 8.  Each
// XCD holds c = min(g, 8) canvases with 32 / c lanes each, all walking the same tiles, so an
// E tile crosses into the XCD's L2 once for c canvases and each canvas's h chunk once for
// its 32 / c lanes; the XCDs of one canvas group split the vocabulary, so E is fetched from
// beyond L2 once per group (g / c times in all).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int round_size(int remaining, int gmax) {
  int g = gmax;
  while (g > remaining) g >>= 1;
  return g;
}

struct Lane {
  int k;     // canvas within the round
  int lane;  // vocabulary lane
  int L;     // lanes per canvas
};

__device__ __forceinline__ Lane lane_of(int b, int g) {
  // c = min(g, 8) canvases share each XCD; the g / c groups of canvases each take 8 c / g
  // XCDs, which split the vocabulary among them (XCD xi of a group: tiles = xi mod X).
  const int x = b & 7, s = b >> 3;
  const int c = g < 8 ? g : 8;
  const int G = g / c, X = 8 / G;
  Lane r;
  r.L = kWG / g;
  r.k = (x % G) * c + s % c;
  r.lane = x / G + X * (s / c);
  return r;
}

// Lanes per canvas of the canvas at position pos of the order (same rounds as above).
__device__ __forceinline__ int lanes_at(int pos, int n_canvas, int gmax) {
  int start = 0;
  for (;;) {
    const int g = round_size(n_canvas - start, gmax);
    if (pos < start + g) return kWG / g;
    start += g;
  }
}

// Running statistics of one row over the tiles of a lane (base-2 units): reference m, sum
// l = sum 2^(z2 - m), moment a = sum 2^(z2 - m) (z2 - m), and lb = the same sum over the
// fp16-rounded weights the expectation pass multiplies (its normaliser).
struct RowAcc {
  float m, l, a, lb, amv, gv;
  int ami, gi;
  float tm[4];  // the four largest half-tile maxima of z2 (descending) ...
  int tv[4];    // ... and their vocabulary entries
};
// Keeps the four largest (z2, -v) pairs in descending order (bubble insertion, no branches).
__device__ __forceinline__ void top4_insert(float (&tm)[4], int (&tv)[4], float m, int v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool take = (m > tm[k]) | ((m == tm[k]) & (v < tv[k]));
    const float om = tm[k];
    const int ov = tv[k];
    tm[k] = take ? m : om;
    tv[k] = take ? v : ov;
    m = take ? om : m;
    v = take ? ov : v;
  }
}
__device__ __forceinline__ void row_acc_reset(RowAcc& s) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s.tm[k] = -INFINITY;
    s.tv[k] = 0x7FFFFFFF;
  }
  s.m = -INFINITY;
  s.l = 0.0f;
  s.lb = 0.0f;
  s.a = 0.0f;
  s.amv = -INFINITY;
  s.gv = -INFINITY;
  s.ami = 0x7FFFFFFF;
  s.gi = 0x7FFFFFFF;
}

// Online-softmax merge (base 2) carrying the rounded-weight sum along with the exact one.
__device__ __forceinline__ void lse_merge_b(float& m, float& l, float& a, float& lb, float m2,
                                            float l2, float a2, float lb2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  const float d1 = m - M, d2 = m2 - M;
  const float s1 = (m == -INFINITY) ? 0.0f : hw_exp2(d1);
  const float s2 = (m2 == -INFINITY) ? 0.0f : hw_exp2(d2);
  const float t1 = (m == -INFINITY) ? 0.0f : s1 * (a + d1 * l);
  const float t2 = (m2 == -INFINITY) ? 0.0f : s2 * (a2 + d2 * l2);
  l = s1 * l + s2 * l2;
  lb = s1 * lb + s2 * lb2;
  a = t1 + t2;
  m = M;
}

// ---------------------------------------------------------------------------------------
// Logits pass.
// ---------------------------------------------------------------------------------------
struct GemmK {
  VocabArgs a;
  const int* order;   // [n_canvas] canvases, non-commit first
  const int* pos;     // [n_canvas] position of each canvas in order
  const int* n_nc_p;  // number of non-commit canvases
  uint16_t* P;        // fp16 weights 2^(z2 - ref) in MFMA-fragment order (null: no
                      // expectation, nothing stored): 1 KB blocks
                      // [row / 16][v / 32], entry (row, v) at 8 (row % 16 + 16 ((v % 32) / 8))
                      // + v % 8 of its block; row = 256 pos + i
  int* ref;           // [n_half][R] integer references (base-2 units), row = 256 pos + i
  float* st_m;        // [R][st_stride] statistic partials (slot = 2 lane + half)
  float* st_l;
  float* st_lb;
  float* st_tm;       // [4][R][st_stride] top-4 half-tile maxima (z2) and their entries
  int* st_tv;
  float* st_a;
  float* st_amv;
  int* st_ami;
  float* st_gv;
  int* st_gi;
  float* accp;        // [n_range][R][d] expectation partials, row = 256 pos + i
  float* accM;        // [n_range][R] their references
  float* fac;         // [R][kFacStride]: range weights [0, 64), correction weights [64, 68),
                      // correction entries (int) [68, 72)
  int n_tiles;        // vocabulary tiles of 256
  size_t vpad;        // n_tiles * 256
  int n_range;        // vocabulary ranges of the expectation pass
  int ncb;            // 16-column blocks per wave in the expectation pass
  int n_colblk;       // d / (32 ncb)
  int flat;           // expectation units mapped flat (1) or pair-per-XCD (0)
  int gmax;           // largest round of the logits pass (canvases)
  int st_stride;      // statistic slots per row: 2 x the most lanes any canvas gets
};

// Per-lane epilogue of one row (32-row block of this wave) over the wave's 128 entries: the
// lane holds 64 of them in s0..s3 (entry vt0 + 32 mb + 8 (i / 4) + 4 (lane / 32) + i % 4),
// lane ^ 32 the other 64.  kHeavy: the full epilogue; otherwise only the argmax.
// z2 = S c2 and dz = z2 - ref are rounded separately (no contraction), so that the
// combine can recompute the weight of a half tile's maximum bit for bit.
// pt: this lane's 8-byte group in the weight block of the half tile's first 32 entries.
// The running statistics live in LDS (lds_st: this lane's row; lanes l and l ^ 32 hold the
// same row and compute identical values, lanes < 32 store them), so that the epilogue's
// registers are left to the logits and the noise.
typedef __attribute__((address_space(3))) RowAcc LdsRowAcc;

// Final-logit soft cap (DiffusionGemma Explained, "Logit Softcapping"): z2 = c tanh(S / c) c2
// with c2 = log2(e) / T, evaluated as tanh(S inv_c) cz, cz = c c2 (one rounding of c c2 per
// canvas).  tanhf is the device library's (relative error of a few ulp at every |S / c|,
// saturating to +-1), so the capped logit keeps the accuracy of S near 0.
struct SoftCap {
  float inv_c, cz;
};

__device__ __forceinline__ float soft_cap_z2(float s, const SoftCap& sc) {
#pragma clang fp contract(off)
  return mul_rn(tanhf(mul_rn(s, sc.inv_c)), sc.cz);
}

// kCap: z2 = soft_cap_z2(S) in place of S c2; the argmax stays on S.
// kSep: the Gumbel key takes its own temperature, c2g = log2(e) / T_draw (S c2g, or
// tanh(S / c) c c2g with the cap) in place of z2; the statistics keep c2.
// kStore: the weights are stored at pt (the expectation is asked for).
template <bool kHeavy, bool kCap, bool kSep = false, bool kStore = true>
__device__ __forceinline__ void epi_row(const f32x16& s0, const f32x16& s1, const f32x16& s2,
                                        const f32x16& s3, int vt0, int V, float c2,
                                        const SoftCap& cap, uint32_t row, uint32_t step,
                                        uint32_t k0, uint32_t k1, uint16_t* pt, int* ref_out,
                                        LdsRowAcc* lds_st, float c2g = 0.0f, float czg = 0.0f) {
  // HIP contracts a * b - c into one fma by default, which would round dz once instead of
  // twice and break the bit-for-bit recomputation in the combine (mul_rn / sub_rn keep the
  // two roundings)
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int vb0 = vt0 + 4 * (lane >> 5);
  // the scans keep entry indices relative to the block's first entry, so that each select
  // takes a constant (no per-entry index arithmetic); the empty value maps back to 0x7FFFFFFF
  float amv = -INFINITY;
  int amr = 0x7FFFFFFF - vb0;
  // entries past V exist only in the last tile: a full half tile scans without the checks
  const bool full = vt0 + kHalf <= V;
  auto scan = [&](auto masked, const f32x16& sb, int ro) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int o = ro + 8 * (i >> 2) + (i & 3);
      const float x = (!decltype(masked)::value || vb0 + o < V) ? sb[i] : -INFINITY;
      argmax_next(amv, amr, x, o);  // o increases along the scan
    }
  };
  auto scan_all = [&](auto masked) {
    scan(masked, s0, 0);
    scan(masked, s1, 32);
    scan(masked, s2, 64);
    scan(masked, s3, 96);
  };
  if (full)
    scan_all(std::false_type{});
  else
    scan_all(std::true_type{});
  int ami = amr + vb0;
  argmax_merge(amv, ami, xor_f(amv, 32), xor_i(ami, 32));
  // the half tile's largest z2: rounding is monotone and c2 > 0, so max_v (S_v c2) rounded
  // equals (max_v S_v) c2 rounded.  With the cap: the z2 of S's argmax, which the block loop
  // recomputes bit for bit; tanh is increasing, so another entry can exceed it only by the
  // rounding of tanhf, which leaves its 2^(z2 - ref) within an ulp of 1 (bf16 1.0)
  const float m = !kCap ? mul_rn(amv, c2)
                        : (amv == -INFINITY ? -INFINITY : soft_cap_z2(amv, cap));
  const bool writer = lane < 32;
  {
    float sv = lds_st->amv;
    int si = lds_st->ami;
    argmax_merge(sv, si, amv, ami);
    if (writer) {
      lds_st->amv = sv;
      lds_st->ami = si;
    }
  }
  if (!kHeavy) return;
  // integer reference >= every z2 of the half tile (clamped to +-2^24 so that differences
  // of references stay exact integers)
  const bool empty = (m == -INFINITY);
  const float ref = empty ? 0.0f : fminf(fmaxf(ceilf(m), -16777216.0f), 16777216.0f);
  // the half tile's maximum (its entry is the argmax of S: c2 > 0) joins the row's top four
  if (!empty) {
    float tm[4];
    int tv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tm[k] = lds_st->tm[k];
      tv[k] = lds_st->tv[k];
    }
    top4_insert(tm, tv, m, ami);
    if (writer) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lds_st->tm[k] = tm[k];
        lds_st->tv[k] = tv[k];
      }
    }
  }
  float ls = 0.0f, as = 0.0f, lsb = 0.0f, gv = -INFINITY;
  int gi = 0x7FFFFFFF;
  // kMasked: the block reaches past V (only the last tile); a full block has no checks, so
  // no per-entry branches or selects
  auto block = [&](auto masked, const f32x16& sb, int vbb, uint16_t* pbk) {
    constexpr bool kMasked = decltype(masked)::value;
    int gir = gi - vbb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int vb = vbb + 8 * q;
      const u32x4 wd = philox4x32_10(u32x4{(uint32_t)vb >> 2, row, step, kTagGumbel}, k0, k1);
      float pv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // with kSep and the cap, sb holds tanh(S / c): z2 = t (c c2), the key's t (c c2g)
        const float z2 = kCap ? (kSep ? mul_rn(sb[4 * q + j], cap.cz) : sb[4 * q + j])
                              : mul_rn(sb[4 * q + j], c2);
        const float zk = !kSep ? z2 : kCap ? mul_rn(sb[4 * q + j], czg) : mul_rn(sb[4 * q + j], c2g);
        const float dz = sub_rn(z2, ref);
        const float g2 = gumbel2s_from_word(wd[j]);
        if (kMasked) {
          const bool ok = vb + j < V;
          const float pe = ok ? hw_exp2(dz) : 0.0f;
          ls += pe;
          as = __builtin_fmaf(pe, ok ? dz : 0.0f, as);
          argmax_next(gv, gir, ok ? zk + g2 : -INFINITY, 8 * q + j);
          pv[j] = pe;
        } else {
          const float pe = hw_exp2(dz);
          ls += pe;
          as = __builtin_fmaf(pe, dz, as);
          argmax_next(gv, gir, zk + g2, 8 * q + j);  // entries in increasing order
          pv[j] = pe;
        }
      }
      const uint32_t w01 = pack_f16x2(pv[0], pv[1]), w23 = pack_f16x2(pv[2], pv[3]);
      // the rounded weights' sum normalises the expectation: needed only when it is asked for
      if (kStore) lsb = add_f16x2(add_f16x2(lsb, w01), w23);
      if (kStore) *reinterpret_cast<u32x2*>(pbk + 128 * q) = u32x2{w01, w23};
    }
    gi = gir + vbb;
  };
  // one 32-entry block at a time, in a run-time loop (one copy of the block's code: unrolled,
  // the blocks' Philox streams would compete for the registers that hold the logits)
  auto run = [&](auto masked) {
#pragma unroll 1
    for (int mb = 0; mb < 4; ++mb) {
      f32x16 sb;
      switch (mb) {
        case 0: sb = s0; break;
        case 1: sb = s1; break;
        case 2: sb = s2; break;
        default: sb = s3; break;
      }
      // capped z2 of the whole block first, so that tanhf's temporaries are dead before
      // the noise's are live (with kSep, tanh(S / c) alone: both products are formed below)
      if (kCap) {
#pragma clang fp contract(off)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sb[i] = kSep ? tanhf(mul_rn(sb[i], cap.inv_c)) : soft_cap_z2(sb[i], cap);
      }
      block(masked, sb, vb0 + 32 * mb, pt + 512 * mb);
    }
  };
  if (full)
    run(std::false_type{});
  else
    run(std::true_type{});
  __builtin_amdgcn_sched_barrier(0);
  ls += xor_f(ls, 32);
  as += xor_f(as, 32);
  lsb += xor_f(lsb, 32);
  argmax_merge(gv, gi, xor_f(gv, 32), xor_i(gi, 32));
  if (writer) *ref_out = empty ? INT32_MIN : (int)ref;
  float sm = lds_st->m, sl = lds_st->l, sa = lds_st->a, slb = lds_st->lb;
  float sgv = lds_st->gv;
  int sgi = lds_st->gi;
  lse_merge_b(sm, sl, sa, slb, empty ? -INFINITY : ref, ls, as, lsb);
  argmax_merge(sgv, sgi, gv, gi);
  if (writer) {
    lds_st->m = sm;
    lds_st->l = sl;
    lds_st->a = sa;
    lds_st->lb = slb;
    lds_st->gv = sgv;
    lds_st->gi = sgi;
  }
}

// Round r of the canvas order: canvases [start, start + g).  Rounds of gmax while gmax or
// more remain, then the binary decomposition of the rest.
__device__ __forceinline__ void round_info(int r, int n_canvas, int gmax, int& start, int& gsz) {
  const int full = n_canvas / gmax;
  if (r < full) {
    start = gmax * r;
    gsz = gmax;
    return;
  }
  start = gmax * full;
  int rem = n_canvas - start, k = r - full;
  for (int gg = gmax >> 1; gg >= 1; gg >>= 1) {
    if (rem & gg) {
      if (k == 0) {
        gsz = gg;
        return;
      }
      --k;
      start += gg;
    }
  }
  gsz = 0;
}

// One workgroup per (round, slot): the tiles t = lane, lane + L, ... of one canvas.  K is
// staged in chunks of 64 elements (one 128-byte line per row: 256 E rows + 256 h rows,
// 64 KB a stage) through two stages; whole lines per copy keep the L2 -> LDS stream at its
// best rate, and a chunk's copies are issued a full chunk before it is multiplied.
constexpr int kKC1 = 64;           // K chunk of the logits pass
constexpr int kRow1 = 2 * kKC1;    // bytes of one staged row
constexpr int kNst1 = 2;           // stages

// 16-byte slot of segment s in staged 128-byte row r: XOR swizzle over the eight segments,
// so that the sixteen consecutive rows one ds_read_b128 pass serves fall on distinct banks.
__device__ __forceinline__ int swz1(int r) { return (r >> 1) & 7; }

// Eight E4M3 codes (two words) widened to eight bf16 (exact; v_cvt_scalef32_pk_bf16_fp8 with
// scale 1), in order.
__device__ __forceinline__ u32x4 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
#define DG_CV(w, hi) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, hi))
  return u32x4{DG_CV(w0, false), DG_CV(w0, true), DG_CV(w1, false), DG_CV(w1, true)};
#undef DG_CV
}

// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 x E4M3 (format codes 0): a lane's 32 codes of A
// (row lane % 32) and of B (column lane % 32) as two 16-byte halves each; E8M0 scales sa, sb
// (byte 0 of each) of the lane's A row and B column, 2^(s - 127).
__device__ __forceinline__ f32x16 mfma32x32x64f8(const u32x4& a0, const u32x4& a1,
                                                 const u32x4& b0, const u32x4& b1, f32x16 c,
                                                 int sa, int sb) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// kMode 1 (kF8): E arrives as E4M3 codes with a power-of-two scale per row (g.a.E8,
// g.a.E_exp).  The codes are staged as 64-byte rows; one 16-byte read gives a lane the codes of
// two 16-wide K steps, widened to bf16 in registers; the h fragments use the same permutation
// of K within the chunk (step 2 j + t, lane half f: K = 32 j + 16 f + 8 t + 0..7), and the
// accumulator of entry v is scaled by 2^E_exp[v] before the epilogue (exact).
// kMode 2 (kA8): E and h both as E4M3 codes with power-of-two row scales (h quantised per row
// when the pass runs).  Both are staged like the bf16 operands, 128-byte rows, now 128 K
// elements a chunk; v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 64-wide K steps (lane half f
// holds K = 64 s + 32 f + 0..31 of its row, two 16-byte reads) and applies the two row scales
// as its E8M0 block scales, so the accumulator holds S itself.  The MFMA's own summation of a
// 64-wide step is not exact (measured: within 2^-11.9 of the step's largest product).
template <bool kCap, int kMode, bool kSep = false>
__global__ __launch_bounds__(512, 1) void k_gemm_logits(GemmK g) {
  constexpr bool kF8 = kMode == 1, kA8 = kMode == 2;
  constexpr int kERow = kF8 ? kKC1 : kRow1;    // bytes of one staged E row
  constexpr int kHOff = kTile * kERow;         // 256 E rows, then 256 h rows
  constexpr int kStage = kHOff + kTile * kRow1;
  __shared__ __attribute__((aligned(1024))) char stg[kNst1][kStage];
  const char* Eb = (kF8 || kA8) ? reinterpret_cast<const char*>(g.a.E8)
                                : reinterpret_cast<const char*>(g.a.E);
  const int V = g.a.V, d = g.a.d, n_canvas = g.a.n_canvas;
  const int t = threadIdx.x, lane = t & 63, fr = lane & 31, fh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int vh = w & 1, rq = w >> 1;  // wave tile: vocabulary half vh x rows [64 rq, 64 rq + 64)
  const int T = g.n_tiles;
  const int nk = kA8 ? d / 128 : d / kKC1;  // chunks; even but for kA8 (d % 128 == 0)
  const size_t R = (size_t)n_canvas * kTile;

  int start, gsz;
  round_info(blockIdx.x >> 8, n_canvas, g.gmax, start, gsz);
  const Lane ln = lane_of(blockIdx.x & 255, gsz);
  if (gsz == 0 || ln.lane >= T) return;
  const int c = __builtin_amdgcn_readfirstlane(g.order[start + ln.k]);
  const int p = __builtin_amdgcn_readfirstlane(g.pos[c]);
  const bool heavy = p < *g.n_nc_p;

  // LDS fragment offsets (stage-relative) of this lane for the four 16-wide K steps
  const int sw = swz1(fr);
  uint32_t rdE[4], rdH[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (kA8) {
      // 64-wide step s = ks / 2, its 16-byte half ks % 2: segment 4 s + 2 fh + ks % 2
      const int seg = 4 * (ks >> 1) + 2 * fh + (ks & 1);
      rdE[ks] = (uint32_t)((128 * vh + fr) * kRow1 + 16 * (seg ^ sw));
      rdH[ks] = (uint32_t)(kHOff + (64 * rq + fr) * kRow1 + 16 * (seg ^ sw));
    } else if (kF8) {
      // code rows: 16-byte segment q of row r at q ^ ((r >> 2) & 3); reads j = 0, 1
      rdE[ks] = (uint32_t)((128 * vh + fr) * kERow + 16 * (((2 * (ks & 1) + fh)) ^ ((fr >> 2) & 3)));
      rdH[ks] = (uint32_t)(kHOff + (64 * rq + fr) * kRow1 +
                           16 * ((4 * (ks >> 1) + 2 * fh + (ks & 1)) ^ sw));
    } else {
      rdE[ks] = (uint32_t)((128 * vh + fr) * kRow1 + 16 * ((2 * ks + fh) ^ sw));
      rdH[ks] = (uint32_t)(kHOff + (64 * rq + fr) * kRow1 + 16 * ((2 * ks + fh) ^ sw));
    }
  }
  // DMA: a copy moves 8 staged rows (1 KB); lane -> row 8 j + lane / 8, slot lane % 8,
  // global segment slot ^ swz1(row).  Wave w copies E rows and h rows [32 w, 32 w + 32) of
  // the stage, four copies each.  Sources: a wave-uniform base plus a 32-bit lane offset.
  const int dlrow = lane >> 3;
  const uint32_t pitch = kA8 ? (uint32_t)d : 2u * (uint32_t)d;  // bytes of an h row
  const uint32_t epitch = (kF8 || kA8) ? (uint32_t)d : pitch;
  uint32_t offH[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    offH[j] = (uint32_t)(8 * j + dlrow) * pitch + 16u * (uint32_t)((lane & 7) ^ swz1(8 * j + dlrow));
  const char* hb = (kA8 ? reinterpret_cast<const char*>(g.a.h8)
                        : reinterpret_cast<const char*>(g.a.h)) +
                   ((size_t)c * kTile + 32 * w) * pitch;
  // E rows of the wave's block of tile tt, clamped to V - 1: base row and lane offsets
  // (code rows: two copies of 16 rows, lane -> row 16 j + lane / 4, segment lane % 4)
  auto e_src = [&](int tt, const char*& eb, uint32_t (&oe)[4]) {
    const int r0 = tt * kTile + 32 * w;
    const int rb = min(r0, V - 1);
    eb = Eb + (size_t)rb * epitch;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kF8) {
        const int rv = min(r0 + 16 * (j & 1) + (lane >> 2), V - 1);
        oe[j] = (uint32_t)(rv - rb) * epitch + 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
      } else {
        const int rv = min(r0 + 8 * j + dlrow, V - 1);
        oe[j] = (uint32_t)(rv - rb) * epitch + 16u * (uint32_t)((lane & 7) ^ swz1(8 * j + dlrow));
      }
    }
  };
  // copies of chunk kc into the stage at LDS address dst: the E rows of a tile whose source
  // is (eb, oe), and the canvas's h rows (inline-assembly DMA: the compiler would otherwise
  // wait for every copy in flight before the next read of LDS, the stages it cannot tell
  // apart)
  auto issue_e = [&](int kc, const char* eb, const uint32_t (&oe)[4], uint32_t dst) {
    const uint32_t kb = (uint32_t)kc * (uint32_t)kERow;
    if (kF8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) dma_asm(eb + kb, oe[j], dst + 1024u * (uint32_t)(2 * w + j));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma_asm(eb + kb, oe[j], dst + 1024u * (uint32_t)(4 * w + j));
    }
  };
  auto issue_h = [&](int kc, uint32_t dst) {
    const uint32_t kb = (uint32_t)kc * (uint32_t)kRow1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma_asm(hb + kb, offH[j], dst + (uint32_t)kHOff + 1024u * (uint32_t)(4 * w + j));
  };
  auto issue = [&](int kc, const char* eb, const uint32_t (&oe)[4], uint32_t dst) {
    issue_e(kc, eb, oe, dst);
    issue_h(kc, dst);
  };
  uint32_t sa[kNst1];  // LDS addresses of the stages
#pragma unroll
  for (int q = 0; q < kNst1; ++q) sa[q] = (uint32_t)(uintptr_t)(lds_char*)stg[q];

  f32x16 acc[4][2];
  // running statistics of this wave's 64 rows: [wave][nb][row in block]
  __shared__ RowAcc lds_stats[8][2][32];
  LdsRowAcc* st0p = (LdsRowAcc*)(&lds_stats[w][0][fr]);
  LdsRowAcc* st1p = (LdsRowAcc*)(&lds_stats[w][1][fr]);
  if (lane < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      LdsRowAcc* q = nb ? st1p : st0p;
      q->m = -INFINITY;
      q->l = 0.0f;
      q->a = 0.0f;
      q->lb = 0.0f;
      q->amv = -INFINITY;
      q->gv = -INFINITY;
      q->ami = 0x7FFFFFFF;
      q->gi = 0x7FFFFFFF;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        q->tm[k] = -INFINITY;
        q->tv[k] = 0x7FFFFFFF;
      }
    }
  }

  // compute the chunk in stage sc once every copy has landed; meanwhile copy chunk kn of the
  // tile (eb, oe) into stage sn, which every wave finished reading before the barrier.  The
  // last 16-wide step's MFMAs of each chunk run at the start of the next one, after its
  // first fragment reads are issued (their operands are already in registers), so the read
  // latency behind every barrier is covered by MFMA work.
  u32x4 fa[2][4], fb[2][2];
  auto last_step = [&]() {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[1][mb], fb[1][nb], acc[mb][nb]);
  };
  u32x4 c8[4];  // kF8: the codes of two K steps (E row block mb)
  auto chunk8 = [&](auto deferred, const char* sc, uint32_t sn, int kn, const char* eb,
                    const uint32_t (&oe)[4]) {
    vm_wait<0>();
    __syncthreads();
    const lds_char* s = (const lds_char*)sc;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) c8[mb] = lds_read16(s + rdE[0] + 32 * kERow * mb);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) fb[0][nb] = lds_read16(s + rdH[0] + 32 * kRow1 * nb);
    if (decltype(deferred)::value) last_step();
    issue_e(kn, eb, oe, sn);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) fa[0][mb] = e4m3x8_bf16(c8[mb][0], c8[mb][1]);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int cb = ks & 1;
      if (ks == 1) issue_h(kn, sn);
      if (ks == 1) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) c8[mb] = lds_read16(s + rdE[1] + 32 * kERow * mb);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        fb[cb ^ 1][nb] = lds_read16(s + rdH[ks + 1] + 32 * kRow1 * nb);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[cb][mb], fb[cb][nb], acc[mb][nb]);
      // A of step ks + 1: the other half of the codes in hand (ks even), or the next read's
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        fa[cb ^ 1][mb] = (ks & 1) ? e4m3x8_bf16(c8[mb][0], c8[mb][1])
                                  : e4m3x8_bf16(c8[mb][2], c8[mb][3]);
    }
  };
  // kA8: the two 64-wide steps of the chunk, E rows scaled by 2^(sA - 127), h rows by
  // 2^(sB - 127).  Software-pipelined by E row block: the fragments of block mb + 1 (after the
  // last block: the next step's h fragments and first block) are read before block mb's two
  // MFMAs, so each read has two MFMAs (128 cycles) to land in.
  int sA[4] = {127, 127, 127, 127}, sB[2] = {127, 127};
  auto chunk_a8 = [&](const char* sc, uint32_t sn, int kn, const char* eb,
                      const uint32_t (&oe)[4]) {
    vm_wait<0>();
    __syncthreads();
    const lds_char* s = (const lds_char*)sc;
    u32x4 b8[2][2], a8[2][2];  // h fragments of the step; E fragments, double-buffered
    auto read_b = [&](int st) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) b8[nb][hf] = lds_read16(s + rdH[2 * st + hf] + 32 * kRow1 * nb);
    };
    auto read_a = [&](int st, int mb, int buf) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) a8[buf][hf] = lds_read16(s + rdE[2 * st + hf] + 32 * kRow1 * mb);
    };
    read_b(0);
    read_a(0, 0, 0);
    issue_e(kn, eb, oe, sn);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4 bc[2][2];  // this step's h fragments (the next step's are read during block 3)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bc[nb][0] = b8[nb][0], bc[nb][1] = b8[nb][1];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int cur = (4 * st + mb) & 1;
        if (mb < 3) {
          read_a(st, mb + 1, cur ^ 1);
        } else if (st == 0) {
          read_b(1);
          read_a(1, 0, cur ^ 1);
        }
        if (st == 1 && mb == 0) issue_h(kn, sn);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = mfma32x32x64f8(a8[cur][0], a8[cur][1], bc[nb][0], bc[nb][1], acc[mb][nb],
                                       sA[mb], sB[nb]);
      }
    }
    // order: the first block's reads, then per block the next block's reads before its MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };
  auto chunk = [&](auto deferred, const char* sc, uint32_t sn, int kn, const char* eb,
                   const uint32_t (&oe)[4]) {
    if constexpr (kF8) {
      chunk8(deferred, sc, sn, kn, eb, oe);
      return;
    }
    vm_wait<0>();
    __syncthreads();
    const lds_char* s = (const lds_char*)sc;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) fa[0][mb] = lds_read16(s + rdE[0] + 32 * kRow1 * mb);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) fb[0][nb] = lds_read16(s + rdH[0] + 32 * kRow1 * nb);
    if (decltype(deferred)::value) last_step();
    // the E copies first (they may miss in L2), the h copies (L2-resident) a step later
    issue_e(kn, eb, oe, sn);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int cb = ks & 1;
      if (ks == 1) issue_h(kn, sn);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        fa[cb ^ 1][mb] = lds_read16(s + rdE[ks + 1] + 32 * kRow1 * mb);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        fb[cb ^ 1][nb] = lds_read16(s + rdH[ks + 1] + 32 * kRow1 * nb);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[cb][mb], fb[cb][nb], acc[mb][nb]);
    }
    // order: the first step's reads, the previous chunk's last MFMAs, then per 16-wide step
    // its MFMAs interleaved with the next step's reads
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    if (decltype(deferred)::value) __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };

  const float c2 = kLog2e / g.a.temperature[c];
  SoftCap cap{};
  if (kCap) cap = SoftCap{1.0f / g.a.softcap, g.a.softcap * c2};
  // kSep: the draw's constants (log2(e) / T_draw, and c log2(e) / T_draw with the cap)
  const float c2g = kSep ? kLog2e / g.a.draw_temperature[c] : c2;
  const float czg = kSep && kCap ? g.a.softcap * c2g : 0.0f;
  const uint32_t step = (uint32_t)g.a.step[c];
  const uint32_t k0 = g.a.k0, k1 = g.a.k1;
  const int rloc0 = 64 * rq + fr;  // row (in the canvas) of block 0; block 1 is 32 rows on
  const uint32_t row0 = (uint32_t)(c * kTile + rloc0), row1 = row0 + 32;
  // weight blocks of rows rloc0 (row16 = 16 p + 4 rq + fr / 16) and rloc0 + 32 (row16 + 2);
  // lane group (fr % 16, fh) at element 8 (fr % 16) + 4 fh of a block
  const size_t nvb = g.vpad / 32;
  uint16_t* prow0 = g.P + ((size_t)(16 * p + 4 * rq + (fr >> 4)) * nvb) * 512 + 8 * (fr & 15) + 4 * fh;
  uint16_t* prow1 = prow0 + 2 * nvb * 512;

  const char* eb;
  uint32_t oe[4];
  e_src(ln.lane, eb, oe);
  issue(0, eb, oe, sa[0]);
  if constexpr (kA8) {
    sB[0] = g.a.h_exp[(size_t)c * kTile + 64 * rq + fr] + 127;
    sB[1] = g.a.h_exp[(size_t)c * kTile + 64 * rq + 32 + fr] + 127;
  }
  int cur = 0;  // kA8: the stage holding the tile's first chunk (nk may be odd)
  // bf16 and kF8: nk is even, every tile starts on stage 0, and its last chunk copies the next
  // tile's first chunk (or, after the last tile, repeats this tile's; never read)
  for (int tt = ln.lane; tt < T; tt += ln.L) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{0};
    const char* ebn;
    uint32_t oen[4];
    e_src(tt + ln.L < T ? tt + ln.L : tt, ebn, oen);
    if constexpr (kA8) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        sA[mb] = g.a.E_exp[min(tt * kTile + kHalf * vh + 32 * mb + fr, V - 1)] + 127;
      // chunk kc from stage cur, copying chunk kc + 1 (after the last: the next tile's first)
      // into the other stage
      for (int kc = 0; kc < nk; ++kc) {
        const bool last = kc + 1 == nk;
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = last ? oen[j] : oe[j];
        chunk_a8(cur ? stg[1] : stg[0], cur ? sa[0] : sa[1], last ? 0 : kc + 1,
                 last ? ebn : eb, o);
        cur ^= 1;
      }
    } else {
      // chunk j is computed from stage j % 2 and copies chunk j + 1 into the other stage
      chunk(std::false_type{}, stg[0], sa[1], 1, eb, oe);
      for (int kc = 1; kc < nk - 1; kc += 2) {
        chunk(std::true_type{}, stg[1], sa[0], kc + 1, eb, oe);
        chunk(std::true_type{}, stg[0], sa[1], kc + 2, eb, oe);
      }
      chunk(std::true_type{}, stg[1], sa[0], 0, ebn, oen);
      last_step();
    }
    eb = ebn;
#pragma unroll
    for (int j = 0; j < 4; ++j) oe[j] = oen[j];
    // ---- epilogue of tile tt
    const int vt0 = tt * kTile + kHalf * vh;
    if constexpr (kF8) {
      // S = 2^E_exp[v] (sum h q): the lane's entries vt0 + 32 mb + 8 q + 4 (lane / 32) + 0..3
      const int vl = vt0 + 4 * fh;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int vb = vl + 32 * mb + 8 * q;
          int ke[4];
          if (vt0 + kHalf <= V) {
            const i32x4v k4 = *reinterpret_cast<const i32x4v*>(g.a.E_exp + vb);
#pragma unroll
            for (int j = 0; j < 4; ++j) ke[j] = k4[j];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) ke[j] = g.a.E_exp[min(vb + j, V - 1)];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              acc[mb][nb][4 * q + j] = __builtin_amdgcn_ldexpf(acc[mb][nb][4 * q + j], ke[j]);
        }
    }
    int* rout0 = g.ref + (size_t)(2 * tt + vh) * R + (size_t)p * kTile + rloc0;
    const size_t vblk = (size_t)(vt0 >> 5) * 512;  // first 32-entry block of the half tile
    if (heavy && g.P != nullptr) {
      epi_row<true, kCap, kSep>(acc[0][0], acc[1][0], acc[2][0], acc[3][0], vt0, V, c2, cap, row0,
                                step, k0, k1, prow0 + vblk, rout0, st0p, c2g, czg);
      epi_row<true, kCap, kSep>(acc[0][1], acc[1][1], acc[2][1], acc[3][1], vt0, V, c2, cap, row1,
                                step, k0, k1, prow1 + vblk, rout0 + 32, st1p, c2g, czg);
    } else if (heavy) {  // no expectation: the weights are not stored
      epi_row<true, kCap, kSep, false>(acc[0][0], acc[1][0], acc[2][0], acc[3][0], vt0, V, c2,
                                       cap, row0, step, k0, k1, prow0, rout0, st0p, c2g, czg);
      epi_row<true, kCap, kSep, false>(acc[0][1], acc[1][1], acc[2][1], acc[3][1], vt0, V, c2,
                                       cap, row1, step, k0, k1, prow1, rout0 + 32, st1p, c2g, czg);
    } else {
      epi_row<false, false>(acc[0][0], acc[1][0], acc[2][0], acc[3][0], vt0, V, c2, cap, row0,
                            step, 0, 0, prow0, rout0, st0p);
      epi_row<false, false>(acc[0][1], acc[1][1], acc[2][1], acc[3][1], vt0, V, c2, cap, row1,
                            step, 0, 0, prow1, rout0 + 32, st1p);
    }
  }
  vm_wait<0>();
  // statistic partials of this (canvas, lane, half)
  if (lane < 32) {
    const int slot = 2 * ln.lane + vh;
    const size_t o0 = ((size_t)c * kTile + rloc0) * (size_t)g.st_stride + slot;
    const size_t plane = (size_t)g.st_stride * R;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const size_t o = o0 + (size_t)32 * nb * (size_t)g.st_stride;
      const LdsRowAcc* st = nb ? st1p : st0p;
      g.st_amv[o] = st->amv;
      g.st_ami[o] = st->ami;
      if (heavy) {
        g.st_m[o] = st->m;
        g.st_l[o] = st->l;
        g.st_a[o] = st->a;
        g.st_lb[o] = st->lb;
        g.st_gv[o] = st->gv;
        g.st_gi[o] = st->gi;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          g.st_tm[k * plane + o] = st->tm[k];
          g.st_tv[k * plane + o] = st->tv[k];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Expectation pass.  Units (non-commit position pc, column block j, range s); the pairs
// (s, pc) are numbered range-major, pair q runs on XCD q % 8, and the XCD's units (its pairs
// in order, each with its column blocks) go round-robin to its 32 slots.
// Wave w: rows [64 (w >> 1), +64) x columns [16 NCB (w & 1), +16 NCB) of the unit's BN.
//
// Operands, both fp16 on v_mfma_f32_16x16x32_f16: the weights 2^(z2 - ref) the logits pass
// stored, each relative to the integer reference ref of its row and 128-entry half tile, and
// E16 (the embedding as fp16, rows padded with zeros to whole tiles) in B-fragment order: the
// 1 KB block of entries 32 b .. 32 b + 31 and columns 16 c .. 16 c + 15 at (b d / 16 + c) KB, lane
// n + 16 g's 16 bytes holding column n's entries 8 g .. 8 g + 7, so a chunk's blocks are one
// contiguous run for the copies and a B fragment is one 16-byte read.  Every row's partial is kept in units of 2^U,
// U = M - 15 with M the row's largest half-tile reference over the unit's vocabulary range
// (the prologue reads them all first): a half tile with reference rf enters with its weights
// multiplied by 2^(rf - U) in fp16 (one packed multiply per A register).  For rf >= U that is
// a scale by 2^0 .. 2^15, exact (the weights are at most 1, so at most 2^15 < 65504), and the
// products are those of the stored weights; for rf < U the scaled weights round to fp16's
// subnormal grid (2^-24 in units of 2^U, i.e. 2^-39 of the row's largest weight) and below
// 2^-25 of the unit vanish, which changes the partial by less than 2^14 2^-40 of that largest
// weight.  Each stored weight keeps fp16's precision relative to its own half tile, so a flat
// distribution's expectation loses nothing to the cross-tile scaling; the fp32 accumulator
// holds at most 2^14 terms of at most 2^15 |E|.
// ---------------------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16x16x32h(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

struct Unit {
  int pc, j, s, t0, t1;
  bool valid;
};

// XCD mapping: local unit lu of XCD x is column block lu % n_colblk of pair
// q = x + 8 (lu / n_colblk).  Flat mapping (x = -1): unit lu is column block lu % n_colblk of
// pair lu / n_colblk (used when pinning pairs to XCDs would leave CUs idle).
__device__ __forceinline__ Unit unit_at(int x, int lu, int n_nc, int n_range, int n_colblk, int T) {
  Unit u;
  const int i = lu / n_colblk;
  u.j = lu - i * n_colblk;
  const int q = x < 0 ? i : x + 8 * i;
  u.valid = q < n_nc * n_range;
  const int qq = u.valid ? q : 0;
  u.s = qq / n_nc;
  u.pc = qq - u.s * n_nc;
  u.t0 = (int)(((long long)T * u.s) / n_range);
  u.t1 = (int)(((long long)T * (u.s + 1)) / n_range);
  return u;
}

__device__ __forceinline__ uint32_t lds_u32(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(p);
}

// A unit spans at most kMaxUnitTiles vocabulary tiles (its scale table fits in LDS).
constexpr int kMaxUnitTiles = 64;
constexpr int kUp = 15;     // U = M - kUp: the largest half tile's weights enter times 2^15
// scale-table entry of a half tile whose weights vanish (2^(rf - U) below 2^-24, or past V):
// far enough below fp16's smallest subnormal that 2^kZero rounds to 0
constexpr int kZero = -32;

// 2^k in fp16 for kZero <= k <= kUp: exact for k >= -24 (subnormal below -14), 0 for k <= -26
// (one v_ldexp_f16; the scale table holds no -25)
__device__ __forceinline__ _Float16 f16_pow2(int k) {
  return __builtin_amdgcn_ldexph((_Float16)1.0f, k);
}

// both fp16 halves of a times s (one v_pk_mul_f16, s broadcast by op_sel); the operands are
// taken by value
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, _Float16 s) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) * (f16x2){s, s});
}

template <int NCB>
__global__ __launch_bounds__(512, 1) void k_gemm_selfcond(GemmK g) {
  constexpr int BN = 32 * NCB;            // columns of a unit
  constexpr int kKC2 = 32;                // K chunk (vocabulary entries) per stage
  constexpr int kNst2 = 4;                // stages: copies run three chunks ahead
  constexpr int kPB = kTile * 2 * kKC2;   // weights: 16 fragment blocks of 1 KB (16 KB)
  constexpr int kEB = kKC2 * 2 * BN;      // E: 32 entries x BN columns, 2 NCB blocks of 1 KB
  constexpr int kStage = kPB + kEB;
  constexpr int kNE = kEB / 1024;         // E copies per stage (2 NCB)
  constexpr int kNEw = kNE >= 8 ? kNE / 8 : 1;  // E copies per wave (waves >= kNE repeat one)
  static_assert(kNE % 8 == 0 || kNE < 8, "E copies must divide among the eight waves");
  constexpr int kCpw = 2 + kNEw;          // copies per wave and chunk
  __shared__ __attribute__((aligned(1024))) char stg[kNst2][kStage];
  // scale exponent rf - U of (half tile ht, row): byte 256 ht + 64 rw + 4 (row % 16) + rb for
  // row = 64 rw + 16 rb + row % 16, so that one 32-bit read gives a lane its four A rows
  __shared__ __attribute__((aligned(16))) int8_t shb[2 * kMaxUnitTiles * kTile];
  // the prologue's two partial maxima per row live in stage 1 (no copy has been issued yet)
  int (*sM)[kTile] = reinterpret_cast<int (*)[kTile]>(stg[1]);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int rw = w >> 1, cw = w & 1;
  const int T = g.n_tiles;
  const int n_nc = *g.n_nc_p;
  const size_t R = (size_t)g.a.n_canvas * kTile;
  const Unit u = g.flat ? unit_at(-1, blockIdx.x, n_nc, g.n_range, g.n_colblk, T)
                       : unit_at(blockIdx.x & 7, blockIdx.x >> 3, n_nc, g.n_range, g.n_colblk, T);
  if (!u.valid || u.t1 <= u.t0) return;
  const int nh = 2 * (u.t1 - u.t0);  // half tiles of the unit (<= 2 kMaxUnitTiles)

  // ---- prologue: per row (two threads, alternate half tiles) the largest reference M, then
  // the scale exponents; the partial's unit U = M - kUp (-inf for a range past V)
  {
    const int row = t & (kTile - 1), hh = t >> 8;
    const int* rp = g.ref + (size_t)2 * u.t0 * R + (size_t)u.pc * kTile + row;
    int mx = INT32_MIN;  // INT32_MIN: a half tile past V (zero weights)
#pragma unroll 8
    for (int ht = hh; ht < nh; ht += 2) mx = max(mx, rp[(size_t)ht * R]);
    sM[hh][row] = mx;
    __syncthreads();
    const int M = max(sM[0][row], sM[1][row]);
    const int pos = 64 * (row >> 6) + 4 * (row & 15) + ((row >> 4) & 3);
#pragma unroll 8
    for (int ht = hh; ht < nh; ht += 2) {
      const int rf = rp[(size_t)ht * R];
      // rf <= M; references lie within +-2^24, so the difference does not overflow
      const int k = rf - M + kUp;
      shb[ht * kTile + pos] = (int8_t)(rf == INT32_MIN || k < -24 ? kZero : k);
    }
    if (hh == 0 && u.j == 0)
      g.accM[(size_t)u.s * R + (size_t)u.pc * kTile + row] =
          M == INT32_MIN ? -INFINITY : (float)(M - kUp);
    __syncthreads();  // sM (stage 1) is overwritten by the first copies
  }

  // ---- copies.  Weights: copy j of wave w moves the fragment block of row16 2 w + j for the
  // chunk (LDS 1 KB number 2 w + j).  E: copy m moves fragment block (w + 8 m) % kNE of the
  // unit's 2 NCB column blocks for the chunk (contiguous in E16), to the same 1 KB of the stage.
  const size_t nvb = g.vpad / 32;
  const char* pbase = reinterpret_cast<const char*>(g.P) +
                      (((size_t)u.pc * 16 + 2 * w) * nvb + (size_t)u.t0 * (kTile / 32)) * 1024;
  const uint32_t offP = 16u * (uint32_t)lane;
  const size_t ncb16 = (size_t)g.a.d / 16;              // column blocks of E16
  const int ew = kNE >= 8 ? w : w % kNE;             // this wave's first E copy
  const char* ebase = reinterpret_cast<const char*>(g.a.E16) +
                      (((size_t)u.t0 * (kTile / 32)) * ncb16 + (size_t)u.j * 2 * NCB + ew) * 1024;
  const int nkc = (u.t1 - u.t0) * (kTile / kKC2);  // a multiple of 8
  uint32_t sa[kNst2];  // LDS addresses of the stages
#pragma unroll
  for (int q = 0; q < kNst2; ++q) sa[q] = (uint32_t)(uintptr_t)(lds_char*)stg[q];

  // copies of chunk kc (clamped to the unit's last chunk: the copies issued past the end go
  // to a stage nobody reads again)
  // (the copy sources are wave-uniform; uniform_ptr states it, so that they stay in SGPRs)
  auto issue_p = [&](int kc, uint32_t dst) {
    kc = min(kc, nkc - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma_asm(uniform_ptr(pbase + ((size_t)j * nvb + kc) * 1024), offP,
              dst + 1024u * (uint32_t)(2 * w + j));
  };
  auto issue_e = [&](int kc, uint32_t dst) {
    kc = min(kc, nkc - 1);
    const char* eb = ebase + (size_t)kc * ncb16 * 1024;
#pragma unroll
    for (int m = 0; m < kNEw; ++m)
      dma_asm(uniform_ptr(eb + (size_t)m * 8 * 1024), offP,
              dst + (uint32_t)kPB + 1024u * (uint32_t)(ew + 8 * m));
  };

  const int ar = lane & 15;
  f32x4 acc[4][NCB];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x4{0, 0, 0, 0};
  // one chunk from stage sc once its copies have landed (the two chunks issued after it may
  // still be in flight), its weights scaled by sc2 (per A row of the lane: 64 rw + 16 rb + ar);
  // copies chunk kn into stage sn, which every wave finished reading before the barrier
  auto chunk = [&](const char* sc, uint32_t sn, int kn, const _Float16 (&sc2)[4]) {
    vm_wait<2 * kCpw>();
    __syncthreads();
    // the E copies at once (E may miss in L2), the weight copies halfway through the chunk
    issue_e(kn, sn);
    const lds_char* sp = (const lds_char*)sc;
    const lds_char* se = (const lds_char*)(sc + kPB) + NCB * cw * 1024 + 16 * lane;
    u32x4 fa[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const u32x4 x = lds_read16(sp + (4 * rw + rb) * 1024 + 16 * lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) fa[rb][q] = mul_f16x2(x[q], sc2[rb]);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (cb == NCB / 2) issue_p(kn, sn);
      const u32x4 fb = lds_read16(se + 1024 * cb);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb][cb] = mfma16x16x32h(fa[rb], fb, acc[rb][cb]);
    }
  };

#pragma unroll
  for (int q = 0; q < kNst2 - 1; ++q) {
    issue_e(q, sa[q]);
    issue_p(q, sa[q]);
  }
  const lds_char* shp = (const lds_char*)shb + 64 * rw + 4 * ar;
  for (int kc = 0; kc < nkc; kc += kNst2) {  // one half tile (four chunks) per iteration
    const uint32_t shw = lds_u32(shp + (kc >> 2) * kTile);
    _Float16 sc2[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) sc2[rb] = f16_pow2((int)(int8_t)(uint8_t)(shw >> (8 * rb)));
    chunk(stg[0], sa[3], kc + 3, sc2);
    chunk(stg[1], sa[0], kc + 4, sc2);
    chunk(stg[2], sa[1], kc + 5, sc2);
    chunk(stg[3], sa[2], kc + 6, sc2);
  }
  vm_wait<0>();
  // expectation partial of this unit, in units of 2^U of its rows (U = M - kUp)
  float* out = g.accp + ((size_t)u.s * R + (size_t)u.pc * kTile) * g.a.d + (size_t)u.j * BN +
               16 * NCB * cw + (lane & 15);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * rw + 16 * rb + 4 * (lane >> 4) + i;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) out[(size_t)row * g.a.d + 16 * cb] = acc[rb][cb][i];
    }
}

// ---------------------------------------------------------------------------------------
// Canvas order: non-commit canvases first, each part in index order; position of each
// canvas; number of non-commit canvases.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm_init(const uint8_t* commit, int n, int* order,
                                                   int* pos, int* n_nc) {
  __shared__ int cnt[256];
  __shared__ int total;
  const int t = threadIdx.x;
  const int per = (n + 255) / 256;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int k = 0;
  for (int c = lo; c < hi; ++c) k += (commit == nullptr || commit[c] == 0) ? 1 : 0;
  cnt[t] = k;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = cnt[i];
      cnt[i] = run;
      run += v;
    }
    total = run;
    *n_nc = run;
  }
  __syncthreads();
  int a = cnt[t];
  int bb = total + (lo - cnt[t]);
  for (int c = lo; c < hi; ++c) {
    const int p = (commit == nullptr || commit[c] == 0) ? a++ : bb++;
    order[p] = c;
    pos[c] = p;
  }
}

// ---------------------------------------------------------------------------------------
// Combine, in two kernels.  k_gemm_rows: one wave per row merges the statistic partials of
// the row's lanes (and their top-4 half-tile maxima), writes lse / entropy / argmax / Gumbel
// token, and the weights of the expectation sum: fac[s] = 2^(U_s - m) / lb' for the range
// partials (U_s: the partial's reference) and coef[k] / lb' for the four exact corrections.
// k_gemm_sc: one thread per (row, column) forms sum_s fac[s] acc_s + sum_k coef[k] E[v_k].
//
// Expectation normaliser and top-4 correction.  The expectation pass multiplies fp16 weights
// w~ = fp16(2^(z2 - ref)); dividing by the sum of the same rounded weights (lb) cancels a
// common rounding, and the four largest half-tile maxima of the row, whose rounding would
// otherwise dominate the error of a peaked row, are restored exactly: their residual w - w~
// (w recomputed here bit for bit as the logits pass computed it) is added, scaled, to
// numerator and lb.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm_rows(GemmK g) {
  const int n_canvas = g.a.n_canvas;
  const size_t R = (size_t)n_canvas * kTile;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if ((size_t)r >= R) return;
  const int c = r / kTile, i = r - c * kTile;
  const int p = g.pos[c];
  const bool heavy = p < *g.n_nc_p;
  const int L = lanes_at(p, n_canvas, g.gmax);
  const int n_slot = 2 * min(L, g.n_tiles);
  const size_t plane = (size_t)g.st_stride * R;
  float m = -INFINITY, l = 0.0f, a = 0.0f, lb = 0.0f, amv = -INFINITY, gv = -INFINITY;
  int ami = 0x7FFFFFFF, gi = 0x7FFFFFFF;
  float tm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  int tv[4] = {0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF};
  // up to four slots per lane at a time, their loads issued together (a single canvas has
  // 512 slots a row)
  for (int s0 = lane; s0 < n_slot; s0 += 256) {
    float vm[4], vl[4], va[4], vlb[4], vamv[4], vgv[4], vtm[4][4];
    int vami[4], vgi[4], vtv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = min(s0 + 64 * u, n_slot - 1);
      const size_t o = (size_t)r * (size_t)g.st_stride + s;  // a row's slots are contiguous
      vamv[u] = g.st_amv[o];
      vami[u] = g.st_ami[o];
      if (heavy) {
        vm[u] = g.st_m[o];
        vl[u] = g.st_l[o];
        va[u] = g.st_a[o];
        vlb[u] = g.st_lb[o];
        vgv[u] = g.st_gv[o];
        vgi[u] = g.st_gi[o];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          vtm[u][k] = g.st_tm[k * plane + o];
          vtv[u][k] = g.st_tv[k * plane + o];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0 + 64 * u >= n_slot) break;
      argmax_merge(amv, ami, vamv[u], vami[u]);
      if (heavy) {
        lse_merge_b(m, l, a, lb, vm[u], vl[u], va[u], vlb[u]);
        argmax_merge(gv, gi, vgv[u], vgi[u]);
#pragma unroll
        for (int k = 0; k < 4; ++k) top4_insert(tm, tv, vtm[u][k], vtv[u][k]);
      }
    }
  }
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) {
    argmax_merge(amv, ami, xor_f(amv, msk), xor_i(ami, msk));
    if (heavy) {
      const float m2 = xor_f(m, msk), l2 = xor_f(l, msk), a2 = xor_f(a, msk);
      const float lb2 = xor_f(lb, msk);
      lse_merge_b(m, l, a, lb, m2, l2, a2, lb2);
      argmax_merge(gv, gi, xor_f(gv, msk), xor_i(gi, msk));
      float om[4];
      int ov[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        om[k] = xor_f(tm[k], msk);
        ov[k] = xor_i(tv[k], msk);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) top4_insert(tm, tv, om[k], ov[k]);
    }
  }
  if (lane == 0) g.a.argmax_tok[r] = ami;
  if (!heavy) return;
  float cf[4];
  float lbc = lb;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    cf[k] = 0.0f;
    if (tm[k] != -INFINITY) {
      const float ref = fminf(fmaxf(ceilf(tm[k]), -16777216.0f), 16777216.0f);
      const float w = hw_exp2(sub_rn(tm[k], ref));
      const float wr = round_f16(w);
      cf[k] = (w - wr) * hw_exp2(ref - m);
    }
    lbc += cf[k];
  }
  const float linv = 1.0f / lbc;
  if (lane == 0) {
    const float lg = hw_log2(l);
    if (g.a.lse) g.a.lse[r] = kLn2 * (m + lg);
    g.a.entropy[r] = fmaxf(0.0f, kLn2 * (lg - a / l));
    g.a.gumbel_tok[r] = gi;
  }
  if (g.a.selfcond == nullptr) return;
  const size_t rp = (size_t)p * kTile + i;  // row among the non-commit rows
  float* fr = g.fac + rp * kFacStride;
  for (int s = lane; s < g.n_range; s += 64) {
    const float base = g.accM[(size_t)s * R + rp];
    fr[s] = base == -INFINITY ? 0.0f : hw_exp2(base - m) * linv;
  }
  if (lane < 4) {
    const float cfl = lane == 0 ? cf[0] : lane == 1 ? cf[1] : lane == 2 ? cf[2] : cf[3];
    const int tvl = lane == 0 ? tv[0] : lane == 1 ? tv[1] : lane == 2 ? tv[2] : tv[3];
    fr[64 + lane] = cfl * linv;
    reinterpret_cast<int*>(fr)[68 + lane] = cfl != 0.0f ? tvl : 0;
  }
}

__global__ __launch_bounds__(256) void k_gemm_sc(GemmK g) {
  const int n_canvas = g.a.n_canvas;
  const size_t R = (size_t)n_canvas * kTile;
  const int d = g.a.d;
  const int n_cb = (d + 255) / 256;
  const int r = blockIdx.x / n_cb;
  const int col = (blockIdx.x - r * n_cb) * 256 + threadIdx.x;
  const int c = r / kTile, i = r - c * kTile;
  const int p = g.pos[c];
  if (p >= *g.n_nc_p || col >= d) return;
  const size_t rp = (size_t)p * kTile + i;
  const float* fr = g.fac + rp * kFacStride;
  const float* src = g.accp + rp * d + col;
  const size_t stride = R * d;
  float acc = 0.0f;
  const int nr = g.n_range;
  int s = 0;
  for (; s + 8 <= nr; s += 8) {
    float x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = src[(size_t)(s + q) * stride];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += fr[s + q] * x[q];
  }
  for (; s < nr; ++s) acc += fr[s] * src[(size_t)s * stride];
  const int* vi = reinterpret_cast<const int*>(fr) + 68;
  if (g.a.E8 != nullptr) {
    // E from the FP8 codes: 2^E_exp[v] value(code), exact
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t code = g.a.E8[(size_t)vi[k] * d + col];
      const float ev = __builtin_amdgcn_ldexpf(
          bf16_lo(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                                   code, 1.0f, false))),
          g.a.E_exp[vi[k]]);
      acc += fr[64 + k] * ev;
    }
  } else {
    const uint16_t* E = g.a.E;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc += fr[64 + k] * __uint_as_float((uint32_t)E[(size_t)vi[k] * d + col] << 16);
  }
  g.a.selfcond[(size_t)r * d + col] = acc;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static size_t al256g(size_t x) { return (x + 255) & ~(size_t)255; }

static const int kNcbChoices[3] = {8, 4, 2};

bool gemm_supported(int d) { return d % 128 == 0; }

// Column blocking and vocabulary ranges of the expectation pass, from a cost model of the
// persistent schedule: rounds of the busiest XCD x unit time (scaled by the MFMA-to-byte
// intensity of the unit's tile), plus the HBM time of writing and reading the partials.
static void pick_selfcond_tiling(int n_canvas, int n_tiles, int d, int* ncb_out, int* nr_out,
                                 int* flat_out) {
  double best = 1e300;
  int bn = 2, br = 1, bf = 0;
  for (int qi = 0; qi < 3; ++qi) {
    const int ncb = kNcbChoices[qi];
    if (d % (32 * ncb) != 0) continue;
    const int n_col = d / (32 * ncb);
    const double inten = 2.0 * 256 * 32 * ncb * 64 / (32768.0 + 64.0 * 64 * ncb);
    const double eff = inten >= 140.0 ? 1.0 : inten / 140.0;
    const int rmax = n_tiles < 64 ? n_tiles : 64;
    const int rmin = (n_tiles + kMaxUnitTiles - 1) / kMaxUnitTiles;  // shifts fit in LDS
    for (int nr = rmin; nr <= rmax; ++nr) {
      const int tiles = (n_tiles + nr - 1) / nr;
      const double unit = (double)tiles * 256.0 * 256.0 * 32.0 * ncb * 2.0 / (9.77e12 * 0.5 * eff);
      const double part = (double)n_canvas * 256.0 * d * 4.0 * nr * 2.0 / 5.0e12;
      for (int flat = 0; flat < 2; ++flat) {
        int rounds;
        if (flat) {
          rounds = (n_canvas * nr * n_col + 255) / 256;
        } else {
          const int pairs_x = (n_canvas * nr + 7) / 8;
          rounds = (pairs_x * n_col + 31) / 32;
        }
        // the flat mapping gives up the L2 sharing of weights and E across a pair's units
        const double cost = rounds * unit * (flat ? 1.05 : 1.0) + part;
        if (cost < best * 0.999) {
          best = cost;
          bn = ncb;
          br = nr;
          bf = flat;
        }
      }
    }
  }
  *ncb_out = bn;
  *nr_out = br;
  *flat_out = bf;
}

GemmPlan gemm_plan(int n_canvas, int V, int d) {
  GemmPlan p{};
  p.R = (size_t)n_canvas * kTile;
  p.n_tiles = (V + kTile - 1) / kTile;
  p.vpad = (size_t)p.n_tiles * kTile;
  pick_selfcond_tiling(n_canvas, p.n_tiles, d, &p.ncb, &p.n_range, &p.flat);
  p.n_colblk = d / (32 * p.ncb);
  p.gmax = kRoundMax;
  {
    // the smallest round: kRoundMax while whole rounds remain, else the lowest set bit of the
    // remainder; its canvases get the most lanes, 256 / size (used up to the tile count)
    const int rem = n_canvas % p.gmax;
    const int gmin = rem ? (rem & -rem) : p.gmax;
    p.st_stride = 2 * min(kWG / gmin, p.n_tiles);
  }
  p.n_rounds = n_canvas / p.gmax + __builtin_popcount((unsigned)(n_canvas % p.gmax));
  p.n_units_xcd = ((n_canvas * p.n_range + 7) / 8) * p.n_colblk;
  p.n_units = n_canvas * p.n_range * p.n_colblk;
  size_t off = 0;
  p.off_small = off;
  off += al256g((size_t)(2 * n_canvas + 64) * 4);
  p.off_P = off;
  off += al256g(p.R * p.vpad * 2);
  p.off_ref = off;
  off += al256g((size_t)2 * p.n_tiles * p.R * 4);
  p.off_st = off;
  off += 16 * al256g((size_t)p.st_stride * p.R * 4);  // 8 statistics + 4 x (top z2, entry)
  p.off_accp = off;
  off += al256g((size_t)p.n_range * p.R * d * 4);
  p.off_accM = off;
  off += al256g((size_t)p.n_range * p.R * 4);
  p.off_fac = off;
  off += al256g(p.R * kFacStride * 4);
  p.bytes = off;
  return p;
}

hipError_t gemm_launch(const VocabArgs& a, const GemmPlan& p, void* workspace,
                       hipStream_t stream) {
  char* b = static_cast<char*>(workspace);
  GemmK g{};
  g.a = a;
  int* small = reinterpret_cast<int*>(b + p.off_small);
  int* order = small;
  int* pos = small + a.n_canvas;
  int* n_nc = small + 2 * a.n_canvas;
  g.order = order;
  g.pos = pos;
  g.n_nc_p = n_nc;
  // the weights are stored only when the expectation is asked for
  g.P = a.selfcond != nullptr ? reinterpret_cast<uint16_t*>(b + p.off_P) : nullptr;
  g.ref = reinterpret_cast<int*>(b + p.off_ref);
  const size_t st = al256g((size_t)p.st_stride * p.R * 4);
  g.st_m = reinterpret_cast<float*>(b + p.off_st + 0 * st);
  g.st_l = reinterpret_cast<float*>(b + p.off_st + 1 * st);
  g.st_a = reinterpret_cast<float*>(b + p.off_st + 2 * st);
  g.st_amv = reinterpret_cast<float*>(b + p.off_st + 3 * st);
  g.st_ami = reinterpret_cast<int*>(b + p.off_st + 4 * st);
  g.st_gv = reinterpret_cast<float*>(b + p.off_st + 5 * st);
  g.st_gi = reinterpret_cast<int*>(b + p.off_st + 6 * st);
  g.st_lb = reinterpret_cast<float*>(b + p.off_st + 7 * st);
  g.st_tm = reinterpret_cast<float*>(b + p.off_st + 8 * st);   // 4 planes of st bytes
  g.st_tv = reinterpret_cast<int*>(b + p.off_st + 12 * st);
  g.accp = reinterpret_cast<float*>(b + p.off_accp);
  g.accM = reinterpret_cast<float*>(b + p.off_accM);
  g.fac = reinterpret_cast<float*>(b + p.off_fac);
  g.n_tiles = p.n_tiles;
  g.vpad = p.vpad;
  g.n_range = p.n_range;
  g.ncb = p.ncb;
  g.n_colblk = p.n_colblk;
  g.flat = p.flat;
  g.gmax = p.gmax;
  g.st_stride = p.st_stride;
  hipLaunchKernelGGL(k_gemm_init, dim3(1), dim3(256), 0, stream, a.commit, a.n_canvas, order,
                     pos, n_nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid1((unsigned)(kWG * p.n_rounds));
  const bool cap = a.softcap != 0.0f, sep = a.draw_temperature != nullptr;
  if (a.E8 != nullptr && a.h8 != nullptr) {
    if (cap)
      hipLaunchKernelGGL((k_gemm_logits<true, 2>), grid1, dim3(512), 0, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_logits<false, 2>), grid1, dim3(512), 0, stream, g);
  } else if (a.E8 != nullptr) {
    if (cap)
      hipLaunchKernelGGL((k_gemm_logits<true, 1>), grid1, dim3(512), 0, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_logits<false, 1>), grid1, dim3(512), 0, stream, g);
  } else if (sep) {
    if (cap)
      hipLaunchKernelGGL((k_gemm_logits<true, 0, true>), grid1, dim3(512), 0, stream, g);
    else
      hipLaunchKernelGGL((k_gemm_logits<false, 0, true>), grid1, dim3(512), 0, stream, g);
  } else if (cap) {
    hipLaunchKernelGGL((k_gemm_logits<true, 0>), grid1, dim3(512), 0, stream, g);
  } else {
    hipLaunchKernelGGL((k_gemm_logits<false, 0>), grid1, dim3(512), 0, stream, g);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.selfcond != nullptr) {
    const dim3 grid((unsigned)(p.flat ? p.n_units : 8 * p.n_units_xcd));
    switch (p.ncb) {
      case 8: hipLaunchKernelGGL((k_gemm_selfcond<8>), grid, dim3(512), 0, stream, g); break;
      case 4: hipLaunchKernelGGL((k_gemm_selfcond<4>), grid, dim3(512), 0, stream, g); break;
      default: hipLaunchKernelGGL((k_gemm_selfcond<2>), grid, dim3(512), 0, stream, g); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_gemm_rows, dim3((unsigned)((p.R + 3) / 4)), dim3(256), 0, stream, g);
  e = hipGetLastError();
  if (e != hipSuccess || a.selfcond == nullptr) return e;
  hipLaunchKernelGGL(k_gemm_sc, dim3((unsigned)(((a.d + 255) / 256) * p.R)), dim3(256), 0, stream,
                     g);
  return hipGetLastError();
}

}  // namespace dg
