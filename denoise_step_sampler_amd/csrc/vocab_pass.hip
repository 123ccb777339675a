// The fused vocabulary pass (tied-unembedding logits, tempered softmax statistics, argmax,
// Gumbel-max sample and self-conditioning expectation) for gfx950.
//
// Decomposition (this file):
//   k_vp_tile      one workgroup per (canvas, 128-token vocabulary tile): S^T = E_t h^T on
//                  bf16 MFMA with fp32 accumulation over d, then the epilogue keeps, per
//                  position, the tile's online-softmax partial (max, sum, entropy moment),
//                  argmax and Gumbel-max candidate, and the tile's unnormalised
//                  probabilities 2^(z - m_tile) for the expectation.
//   k_vp_rows      merges the tile partials of each position (max/sum/moment merge of the
//                  chunked logsumexp, lexicographic (value, -index) merge for the tokens).
//   k_vp_selfcond  one workgroup per (canvas, 128-wide slice of d, vocabulary split):
//                  acc[rows, slice] += P_t E_t[:, slice] on bf16 MFMA, E tiles transposed
//                  through LDS, probabilities rescaled to the row maximum before rounding.
//   k_vp_sc        sums the vocabulary-split partials and divides by the softmax sum.
#include "dg_device.h"
#include "dg_internal.h"

namespace dg {

namespace {

constexpr int kThreads = 256;
constexpr int kBV = 128;   // vocabulary tile of the logits kernel
constexpr int kKC = 64;    // d chunk staged per LDS buffer
constexpr int kLdsPitch = kKC + 8;  // bf16 elements per staged row (144 B: conflict-free frags)

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Epilogue helpers of k_vp_tile.  A lane holds one row r and, in four 32x32 accumulator
// blocks, the logits of vocabulary entries v0 + 32 mb + acc32_m(i, lane).
__device__ __forceinline__ void blk_argmax_max(const f32x16& s, int vb0, int V, float c2,
                                               float& bv, int& bi, float& m) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int v = vb0 + 8 * (i >> 2) + (i & 3);
    if (v < V) {
      argmax_merge(bv, bi, s[i], v);
      m = fmaxf(m, s[i] * c2);
    }
  }
}

// Softmax partial, Gumbel candidate and (optionally) unnormalised probabilities of one block.
__device__ __forceinline__ void blk_softmax_gumbel(const f32x16& s, int vb0, int V, float c2,
                                                   float m, uint32_t r, uint32_t step,
                                                   uint32_t k0, uint32_t k1, float* prow,
                                                   float& ls, float& as, float& gv, int& gi) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int vb = vb0 + 8 * q;
    const u32x4 wd = philox4x32_10(u32x4{(uint32_t)vb >> 2, r, step, kTagGumbel}, k0, k1);
    float pv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = vb + j;
      const float z2 = s[4 * q + j] * c2;
      float p = 0.0f;
      if (v < V) {
        const float dz = z2 - m;
        p = hw_exp2(dz);
        ls += p;
        as += p * dz;
        argmax_merge(gv, gi, z2 + gumbel2s_from_word(wd[j]), v);
      }
      pv[j] = p;
    }
    if (prow != nullptr) *reinterpret_cast<f32x4*>(prow + vb) = f32x4{pv[0], pv[1], pv[2], pv[3]};
  }
}

__device__ __forceinline__ void tile_row_epilogue(const f32x16& s0, const f32x16& s1,
                                                  const f32x16& s2, const f32x16& s3,
                                                  const VocabArgs& a, const VocabWs& ws, int tile,
                                                  int r, int v0, int lane, float c2,
                                                  uint32_t step, bool is_commit, size_t R) {
  const int vb0 = v0 + 4 * (lane >> 5);
  float bv = -INFINITY, m = -INFINITY;
  int bi = 0x7FFFFFFF;
  blk_argmax_max(s0, vb0, a.V, c2, bv, bi, m);
  blk_argmax_max(s1, vb0 + 32, a.V, c2, bv, bi, m);
  blk_argmax_max(s2, vb0 + 64, a.V, c2, bv, bi, m);
  blk_argmax_max(s3, vb0 + 96, a.V, c2, bv, bi, m);
  argmax_merge(bv, bi, xor_f(bv, 32), xor_i(bi, 32));
  const size_t so = (size_t)tile * R + r;
  if (lane < 32) {
    ws.t_amv[so] = bv;
    ws.t_ami[so] = bi;
  }
  if (is_commit) return;
  m = fmaxf(m, xor_f(m, 32));
  float ls = 0.0f, as = 0.0f, gv = -INFINITY;
  int gi = 0x7FFFFFFF;
  float* prow = ws.prob != nullptr ? ws.prob + (size_t)r * ws.vpad : nullptr;
  blk_softmax_gumbel(s0, vb0, a.V, c2, m, r, step, a.k0, a.k1, prow, ls, as, gv, gi);
  blk_softmax_gumbel(s1, vb0 + 32, a.V, c2, m, r, step, a.k0, a.k1, prow, ls, as, gv, gi);
  blk_softmax_gumbel(s2, vb0 + 64, a.V, c2, m, r, step, a.k0, a.k1, prow, ls, as, gv, gi);
  blk_softmax_gumbel(s3, vb0 + 96, a.V, c2, m, r, step, a.k0, a.k1, prow, ls, as, gv, gi);
  ls += xor_f(ls, 32);
  as += xor_f(as, 32);
  argmax_merge(gv, gi, xor_f(gv, 32), xor_i(gi, 32));
  if (lane < 32) {
    ws.t_m[so] = m;
    ws.t_l[so] = ls;
    ws.t_a[so] = as;
    ws.t_gv[so] = gv;
    ws.t_gi[so] = gi;
  }
}

// ---------------------------------------------------------------------------------------
// k_vp_tile: logits tile + epilogue.
// grid (n_tiles, n_canvas), block 256 = 4 waves; wave w owns rows [64w, 64w + 64) of the
// canvas and all 128 vocabulary entries of the tile:
//   acc[mb][nb]: 32x32 block of S^T, vocabulary block mb (0..3), row block nb (0..1).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 1) void k_vp_tile(VocabArgs a, VocabWs ws) {
  __shared__ __attribute__((aligned(16))) uint16_t sE[2][kBV][kLdsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sH[2][DG_CANVAS][kLdsPitch];

  const int tile = blockIdx.x;
  const int c = blockIdx.y;
  const int v0 = tile * kBV;
  const int row0 = c * DG_CANVAS;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int d = a.d;
  const bool is_commit = a.commit != nullptr && a.commit[c] != 0;

  // --- staging (registers -> LDS), 16-byte segments
  u32x4 rE[4], rH[8];
  auto load_chunk = [&](int kc) {
    const int k0 = kc * kKC;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = t + kThreads * q;
      const int row = idx >> 3, seg = idx & 7;
      const int v = v0 + row;
      rE[q] = (v < a.V) ? ld16(a.E + (size_t)v * d + k0 + seg * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = t + kThreads * q;
      const int row = idx >> 3, seg = idx & 7;
      rH[q] = ld16(a.h + (size_t)(row0 + row) * d + k0 + seg * 8);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = t + kThreads * q;
      *reinterpret_cast<u32x4*>(&sE[buf][idx >> 3][(idx & 7) * 8]) = rE[q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = t + kThreads * q;
      *reinterpret_cast<u32x4*>(&sH[buf][idx >> 3][(idx & 7) * 8]) = rH[q];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{0};

  const int nk = d / kKC;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  const int fr = lane & 31;          // fragment row / column
  const int fk = (lane >> 5) * 8;    // fragment K half
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) load_chunk(kc + 1);
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      u32x4 fa[4], fb[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        fa[mb] = *reinterpret_cast<const u32x4*>(&sE[buf][32 * mb + fr][16 * ks + fk]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        fb[nb] = *reinterpret_cast<const u32x4*>(&sH[buf][64 * w + 32 * nb + fr][16 * ks + fk]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (kc + 1 < nk) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // --- epilogue: lane holds, for each row block nb, row (64w + 32nb + lane%32) and 64 of the
  // tile's vocabulary entries; lane ^ 32 holds the other 64.
  const float c2 = kLog2e / a.temperature[c];
  const uint32_t step = (uint32_t)a.step[c];
  const size_t R = (size_t)a.n_canvas * DG_CANVAS;
  const int r0 = row0 + 64 * w + fr;
  tile_row_epilogue(acc[0][0], acc[1][0], acc[2][0], acc[3][0], a, ws, tile, r0, v0, lane, c2,
                    step, is_commit, R);
  tile_row_epilogue(acc[0][1], acc[1][1], acc[2][1], acc[3][1], a, ws, tile, r0 + 32, v0, lane,
                    c2, step, is_commit, R);
}

// ---------------------------------------------------------------------------------------
// k_vp_rows: merge the tile partials of each row.  grid R/64, block 256: lane -> row,
// wave -> every 4th tile, then the 4 wave partials merge through LDS.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_vp_rows(VocabArgs a, VocabWs ws) {
  __shared__ float sm[4][64], sl[4][64], sa[4][64], samv[4][64], sgv[4][64];
  __shared__ int sami[4][64], sgi[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.x * 64 + lane;
  const size_t R = (size_t)a.n_canvas * DG_CANVAS;
  const int c = r / DG_CANVAS;
  const bool is_commit = a.commit != nullptr && a.commit[c] != 0;
  float m = -INFINITY, l = 0.0f, ac = 0.0f, amv = -INFINITY, gv = -INFINITY;
  int ami = 0x7FFFFFFF, gi = 0x7FFFFFFF;
  for (int tl = w; tl < ws.n_tiles; tl += 4) {
    const size_t so = (size_t)tl * R + r;
    argmax_merge(amv, ami, ws.t_amv[so], ws.t_ami[so]);
    if (!is_commit) {
      lse_merge(m, l, ac, ws.t_m[so], ws.t_l[so], ws.t_a[so]);
      argmax_merge(gv, gi, ws.t_gv[so], ws.t_gi[so]);
    }
  }
  sm[w][lane] = m; sl[w][lane] = l; sa[w][lane] = ac; samv[w][lane] = amv; sgv[w][lane] = gv;
  sami[w][lane] = ami; sgi[w][lane] = gi;
  __syncthreads();
  if (w != 0) return;
  for (int q = 1; q < 4; ++q) {
    argmax_merge(amv, ami, samv[q][lane], sami[q][lane]);
    if (!is_commit) {
      lse_merge(m, l, ac, sm[q][lane], sl[q][lane], sa[q][lane]);
      argmax_merge(gv, gi, sgv[q][lane], sgi[q][lane]);
    }
  }
  a.argmax_tok[r] = ami;
  if (is_commit) return;
  const float lg = hw_log2(l);
  if (a.lse) a.lse[r] = kLn2 * (m + lg);
  a.entropy[r] = fmaxf(0.0f, kLn2 * (lg - ac / l));
  a.gumbel_tok[r] = gi;
  ws.row_m[r] = m;
  ws.row_linv[r] = 1.0f / l;
}

// ---------------------------------------------------------------------------------------
// k_vp_selfcond: acc[256 rows, DS] += P E over a vocabulary split.
// grid (d / DS, n_split, n_canvas), block 256; wave w owns rows [64w, 64w+64) x DS columns:
//   acc[rb][cb]: rows 32rb.., columns 32cb..;  A = probabilities (rows x vocab),
//   B = E (vocab x columns) read from a transposed, swizzled LDS copy.
// E tile staging: thread (vb, db) loads the 8x8 block E[8vb.., 8db..], transposes it in
// registers and stores 8 rows of the transposed tile.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int et_slot(int x, int vc) { return vc ^ ((x & 7) ^ ((x >> 3) & 15)); }

template <int NCB>
__global__ __launch_bounds__(kThreads, 1) void k_vp_selfcond(VocabArgs a, VocabWs ws) {
  constexpr int DS = 32 * NCB;
  __shared__ __attribute__((aligned(16))) uint16_t sEt[2][DS][kBV];
  const int ds = blockIdx.x, split = blockIdx.y, c = blockIdx.z;
  if (a.commit != nullptr && a.commit[c] != 0) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int d = a.d;
  const int col0 = ds * DS;
  const int row0 = c * DG_CANVAS;
  const int tb = (int)(((long long)ws.n_tiles * split) / ws.n_split);
  const int te = (int)(((long long)ws.n_tiles * (split + 1)) / ws.n_split);

  // staging role: vocabulary block vb (16 of 8 rows), column block db (DS/8 of 8 columns)
  constexpr int kBlocks = (kBV / 8) * (DS / 8);
  const int vb = t / (DS / 8), db = t % (DS / 8);
  const bool stager = t < kBlocks;
  u32x4 rin[8];
  auto load_tile = [&](int tile) {
    if (!stager) return;
    const int vbase = tile * kBV + 8 * vb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = vbase + i;
      rin[i] = (v < a.V) ? ld16(a.E + (size_t)v * d + col0 + 8 * db) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    if (!stager) return;
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // column j of the block -> row (8db + j) of the transpose
      const int q = j >> 1;
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = rin[2 * p][q], hi = rin[2 * p + 1][q];
        o[p] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      const int x = 8 * db + j;
      *reinterpret_cast<u32x4*>(&sEt[buf][x][8 * et_slot(x, vb)]) = o;
    }
  };

  f32x16 acc[2][NCB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x16{0};

  float rowM[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) rowM[rb] = ws.row_m[row0 + 64 * w + 32 * rb + fr];

  if (tb < te) {
    load_tile(tb);
    store_tile(0);
  }
  __syncthreads();
  const size_t R = (size_t)a.n_canvas * DG_CANVAS;
  for (int tile = tb; tile < te; ++tile) {
    const int buf = (tile - tb) & 1;
    if (tile + 1 < te) load_tile(tile + 1);
    float scl[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = row0 + 64 * w + 32 * rb + fr;
      scl[rb] = hw_exp2(ws.t_m[(size_t)tile * R + r] - rowM[rb]);
    }
#pragma unroll
    for (int ks = 0; ks < kBV / 16; ++ks) {
      u32x4 fa[2], fb[NCB];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = row0 + 64 * w + 32 * rb + fr;
        const float* pp = ws.prob + (size_t)r * ws.vpad + tile * kBV + 16 * ks + 8 * fh;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(pp);
        const f32x4 p1 = *reinterpret_cast<const f32x4*>(pp + 4);
        const float s = scl[rb];
        fa[rb] = u32x4{pack_bf16x2(p0[0] * s, p0[1] * s), pack_bf16x2(p0[2] * s, p0[3] * s),
                       pack_bf16x2(p1[0] * s, p1[1] * s), pack_bf16x2(p1[2] * s, p1[3] * s)};
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int x = 32 * cb + fr;
        fb[cb] = *reinterpret_cast<const u32x4*>(&sEt[buf][x][8 * et_slot(x, 2 * ks + fh)]);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = mfma32x32x16(fa[rb], fb[cb], acc[rb][cb]);
    }
    if (tile + 1 < te) store_tile(buf ^ 1);
    __syncthreads();
  }

  // write the split partial: acc[rb][cb] lane l element i -> row 64w + 32rb + acc32_m(i, l),
  // column 32cb + l%32
  float* out = ws.accp + (size_t)split * R * d;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = row0 + 64 * w + 32 * rb + acc32_m(i, lane);
        out[(size_t)r * d + col0 + 32 * cb + fr] = acc[rb][cb][i];
      }
}

// k_vp_sc: selfcond[r, :] = row_linv[r] * sum_split accp[split][r][:], non-commit rows.
__global__ __launch_bounds__(kThreads) void k_vp_sc(VocabArgs a, VocabWs ws) {
  const size_t R = (size_t)a.n_canvas * DG_CANVAS;
  const size_t n4 = R * a.d / 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const size_t e = i * 4;
    const int r = (int)(e / a.d);
    const int c = r / DG_CANVAS;
    if (a.commit != nullptr && a.commit[c] != 0) continue;
    f32x4 s = *reinterpret_cast<const f32x4*>(ws.accp + e);
    for (int sp = 1; sp < ws.n_split; ++sp) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(ws.accp + (size_t)sp * R * a.d + e);
      s += q;
    }
    const float li = ws.row_linv[r];
    *reinterpret_cast<f32x4*>(a.selfcond + e) = s * li;
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

VocabPlan vocab_plan(int n_canvas, int V, int d) {
  VocabPlan p{};
  p.R = (size_t)n_canvas * DG_CANVAS;
  p.n_tiles = (V + kBV - 1) / kBV;
  p.vpad = (size_t)p.n_tiles * kBV;
  p.ds = (d % 128 == 0) ? 128 : 64;
  const int slices = d / p.ds;
  long long want = (1024 + (long long)n_canvas * slices - 1) / ((long long)n_canvas * slices);
  if (want < 1) want = 1;
  if (want > p.n_tiles) want = p.n_tiles;
  if (want > 64) want = 64;
  p.n_split = (int)want;
  size_t off = 0;
  const size_t ts = align256((size_t)p.n_tiles * p.R * 4);
  p.off_tstat = off;
  off += 7 * ts;
  p.off_prob = off;
  off += align256(p.R * p.vpad * 4);
  p.off_row = off;
  off += 2 * align256(p.R * 4);
  p.off_accp = off;
  off += align256((size_t)p.n_split * p.R * d * 4);
  p.bytes = off;
  return p;
}

static VocabWs make_ws(const VocabPlan& p, void* base, bool want_sc) {
  char* b = static_cast<char*>(base);
  const size_t ts = align256((size_t)p.n_tiles * p.R * 4);
  VocabWs w{};
  w.t_m = reinterpret_cast<float*>(b + p.off_tstat + 0 * ts);
  w.t_l = reinterpret_cast<float*>(b + p.off_tstat + 1 * ts);
  w.t_a = reinterpret_cast<float*>(b + p.off_tstat + 2 * ts);
  w.t_amv = reinterpret_cast<float*>(b + p.off_tstat + 3 * ts);
  w.t_ami = reinterpret_cast<int*>(b + p.off_tstat + 4 * ts);
  w.t_gv = reinterpret_cast<float*>(b + p.off_tstat + 5 * ts);
  w.t_gi = reinterpret_cast<int*>(b + p.off_tstat + 6 * ts);
  w.prob = want_sc ? reinterpret_cast<float*>(b + p.off_prob) : nullptr;
  w.row_m = reinterpret_cast<float*>(b + p.off_row);
  w.row_linv = reinterpret_cast<float*>(b + p.off_row + align256(p.R * 4));
  w.accp = reinterpret_cast<float*>(b + p.off_accp);
  w.n_tiles = p.n_tiles;
  w.vpad = p.vpad;
  w.n_split = p.n_split;
  return w;
}

hipError_t vocab_pass_launch(const VocabArgs& a, const VocabPlan& p, void* workspace,
                             hipStream_t stream) {
  const bool want_sc = a.selfcond != nullptr;
  VocabWs ws = make_ws(p, workspace, want_sc);
  hipLaunchKernelGGL(k_vp_tile, dim3(p.n_tiles, a.n_canvas), dim3(kThreads), 0, stream, a, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_vp_rows, dim3((unsigned)(p.R / 64)), dim3(kThreads), 0, stream, a, ws);
  e = hipGetLastError();
  if (e != hipSuccess || !want_sc) return e;
  const dim3 g(a.d / p.ds, p.n_split, a.n_canvas);
  if (p.ds == 128)
    hipLaunchKernelGGL(k_vp_selfcond<4>, g, dim3(kThreads), 0, stream, a, ws);
  else
    hipLaunchKernelGGL(k_vp_selfcond<2>, g, dim3(kThreads), 0, stream, a, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t n4 = p.R * a.d / 4;
  unsigned blocks = (unsigned)((n4 + kThreads - 1) / kThreads);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_vp_sc, dim3(blocks), dim3(kThreads), 0, stream, a, ws);
  return hipGetLastError();
}

}  // namespace dg
