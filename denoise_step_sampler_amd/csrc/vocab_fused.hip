// Fused vocabulary pass for gfx950: one persistent cooperative kernel, no [R, V] buffer.
//
// Why cooperative: the self-conditioning expectation acc[256, d] += P_t E_t needs, for one
// canvas, 256 x d fp32 accumulators (2.9 MB at d = 2816), far more than one CU holds, while
// the logits S_t = E_t h^T need all of d for every vocabulary tile.  So the accumulator is
// split by columns over a group of 16 workgroups sharing one XCD (one L2), and each member
// produces the probability tile of one vocabulary tile per round for the whole group:
//
//   round r, member g:   A: S^T tile t = tb + 16 r + g  (128 vocab x 256 rows, all of d,
//                           bf16 MFMA 32x32x16) -> epilogue (softmax partial, entropy moment,
//                           argmax, Philox Gumbel-max) -> bf16 probabilities 2^(z2 - ref)
//                           into the group's L2 ring, in MFMA-fragment order
//                        B: acc[256, d/16 slice g] += P_t E_t[:, slice] for the 16 tiles of
//                           the previous round (bf16 MFMA 16x16x32)
//
// Staging: global_load_lds_dwordx4 moves E and h chunks straight into LDS (no staging
// registers).  The logits operands sit in XOR-swizzled 128-byte rows (conflict-free
// ds_read_b128); the E slice of the expectation sits row-major and is read with the LDS
// transpose read ds_read_b64_tr_b16, which delivers vocabulary-contiguous operand fragments
// from d-contiguous rows.
//
// Probability reference: the A step writes 2^(z2 - ref) with ref = max(M, m_tile), M the
// group's running row maximum known to this workgroup (B step, same job) and m_tile the tile
// maximum, both in base-2 units, so every stored value is <= 1 and the tile holding the row
// maximum stores its largest probability as exactly 1.  The B step rescales a tile only when
// its ref differs from the group maximum after the round (rare once the maximum has settled);
// the accumulators are rescaled in fp32 when the maximum grows.

// Roles: each workgroup has 8 waves; waves 0-3 run the A step (logits + epilogue), waves 4-7
// the B step, so the epilogue's VALU work and the B MFMAs issue side by side on every SIMD.
// Within a role, waves synchronise through an LDS counter (never the workgroup barrier).
//
// Synchronisation across the group: two monotonically increasing counters per group, waves
// that published a round (A) and waves that consumed one (B); A of round q waits until every B
// wave finished round q - 2 (two ring slots), B of round q waits until every A wave published
// round q.  Group members are formed from the hardware XCC id so that all ring traffic stays
// in one L2; the data is written with plain stores, completed (s_waitcnt) before the counter
// increment, and read after an L1 invalidate.  Every wait is bounded; on time-out the kernel
// raises an error flag, every wave leaves, and the combine kernel poisons the outputs (token
// -1, NaN statistics).
//
// Jobs: (canvas, vocabulary range) pairs, non-commit canvases first, dealt round-robin to
// groups.  Commit canvases need only the argmax: no probabilities, no exchange.
#include <stdlib.h>
#include <string.h>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kG = 16;          // workgroups per group (one d slice each)
constexpr int kThreads = 256;   // 4 waves
constexpr int kBV = 128;        // vocabulary tile
constexpr int kKC = 64;         // d chunk of the logits contraction (128 bytes per row)
constexpr int kStageA = (kBV + DG_CANVAS) * 128;  // one A stage: 48 KB
constexpr int kSmem = 2 * kStageA;                 // 96 KB
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kTileElems = kBV * DG_CANVAS;        // bf16 probability tile: 64 KB

struct Fused {
  VocabArgs a;
  unsigned* sync;     // [0, 8) per-XCC slot counters, [8] error flag, [16 + gid] produced,
                      // [16 + n_groups + gid] consumed
  uint16_t* ring;     // [n_groups][2][kG][kBV * 256]
  float* ring_ref;    // [n_groups][2][kG][256]
  float* st_m;        // [S_v][kG][R] partial statistics
  float* st_l;
  float* st_a;
  float* st_amv;
  int* st_ami;
  float* st_gv;
  int* st_gi;
  float* accp;        // [S_v][R][d]
  float* accM;        // [S_v][R]
  int n_tiles;
  int s_v;
  int n_groups;
  int per_xcd;
};

__device__ __forceinline__ unsigned poll(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void g2l16(const void* g, lds_char* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}

// ---------------------------------------------------------------------------------------
// A step: S^T tile (128 vocab x 256 rows) over all of d.  Wave w owns rows [64w, 64w + 64):
// acc[mb][nb] is the 32x32 block (vocabulary block mb, row block nb).  LDS stage: E chunk
// [128 rows][8 x 16 B] then h chunk [256 rows][8 x 16 B]; chunk s of row r sits at slot
// s ^ (r & 7).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void stage_a(const uint16_t* E, const uint16_t* h, int V, int d,
                                        int v0, int row0, int k0, lds_char* st) {
  // Instruction q of wave w covers rows 32w + 8q + lane/8 (E) and 64w + 8q + lane/8 (h);
  // the swizzled chunk index depends on lane only, so every address is a per-lane offset plus
  // a wave-uniform stride.
  const int lane = threadIdx.x & 63, w = (threadIdx.x >> 6) & 3;
  const int lr = lane >> 3;
  const int seg = (lane & 7) ^ (lr & 7);
  const uint16_t* eb = E + k0 + 8 * seg;
  const uint16_t* hb = h + (size_t)(row0 + 64 * w + lr) * d + k0 + 8 * seg;
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // E: 1024 chunks, 16 instructions
    int v = v0 + 32 * w + 8 * q + lr;
    v = v < V ? v : V - 1;
    g2l16(eb + (size_t)v * d, st + 1024 * (4 * w + q));
  }
#pragma unroll
  for (int q = 0; q < 8; ++q)  // h: 2048 chunks, 32 instructions
    g2l16(hb + (size_t)(8 * q) * d, st + kBV * 128 + 1024 * (8 * w + q));
}

// Tile maximum (base-2 units) and argmax of one row: 64 logits in this lane, 64 in lane ^ 32.
// kMasked: the tile reaches past V.
template <bool kMasked>
__device__ __forceinline__ void blk_max(const f32x16& s, int vb, int V, float c2, float& m,
                                        float& amv, int& ami) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int v = vb + 8 * (i >> 2) + (i & 3);
    const float x = (!kMasked || v < V) ? s[i] : -INFINITY;
    argmax_merge(amv, ami, x, v);
    m = fmaxf(m, x * c2);
  }
}
template <bool kMasked>
__device__ __forceinline__ void tile_row_max(const f32x16& s0, const f32x16& s1,
                                             const f32x16& s2, const f32x16& s3, int vb0, int V,
                                             float c2, float& m, float& amv, int& ami) {
  m = -INFINITY;
  amv = -INFINITY;
  ami = 0x7FFFFFFF;
  blk_max<kMasked>(s0, vb0, V, c2, m, amv, ami);
  blk_max<kMasked>(s1, vb0 + 32, V, c2, m, amv, ami);
  blk_max<kMasked>(s2, vb0 + 64, V, c2, m, amv, ami);
  blk_max<kMasked>(s3, vb0 + 96, V, c2, m, amv, ami);
  m = fmaxf(m, xor_f(m, 32));
  argmax_merge(amv, ami, xor_f(amv, 32), xor_i(ami, 32));
}
__device__ __forceinline__ void tile_max_both(const f32x16 (&acc)[4][2], bool full, int vb0,
                                              int V, float c2, float (&m)[2], float (&amv)[2],
                                              int (&ami)[2]) {
  if (full) {
    tile_row_max<false>(acc[0][0], acc[1][0], acc[2][0], acc[3][0], vb0, V, c2, m[0], amv[0],
                        ami[0]);
    tile_row_max<false>(acc[0][1], acc[1][1], acc[2][1], acc[3][1], vb0, V, c2, m[1], amv[1],
                        ami[1]);
  } else {
    tile_row_max<true>(acc[0][0], acc[1][0], acc[2][0], acc[3][0], vb0, V, c2, m[0], amv[0],
                       ami[0]);
    tile_row_max<true>(acc[0][1], acc[1][1], acc[2][1], acc[3][1], vb0, V, c2, m[1], amv[1],
                       ami[1]);
  }
}

// Per-lane epilogue state of the two rows (nb = 0, 1) a lane owns in the A step.
struct EpiState {
  float mt0, mt1, ref0, ref1, ls0, ls1, as0, as1, gv0, gv1;
  int gi0, gi1;
};

// One "piece" of the epilogue = one 32x32 accumulator block (mb = piece % 4, nb = piece / 4):
// 16 logits of one row in this lane.  Its four parts (q = 0..3) each draw one Philox block
// and write one 8-byte group of the bf16 probability fragment.  The piece is selected at run
// time and copied out of the accumulator, so one copy of the code serves all eight.
struct Piece {
  f32x16 s;
  int vb0;       // vocabulary of element 0 of part 0 in this lane
  uint32_t row;  // global row
  float m, sref;
  char* dst;     // ring bytes of part 0 in this lane; part q at + 256 q
  float ls, as, gv;
  int gi;
};

__device__ __forceinline__ void piece_begin(Piece& p, int piece, const f32x16 (&acc)[4][2],
                                            const EpiState& e, int vt0, int row0,
                                            char* ring_tile) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, fr = lane & 31;
  const int mb = piece & 3, nb = piece >> 2;
  switch (piece) {
    case 0: p.s = acc[0][0]; break;
    case 1: p.s = acc[1][0]; break;
    case 2: p.s = acc[2][0]; break;
    case 3: p.s = acc[3][0]; break;
    case 4: p.s = acc[0][1]; break;
    case 5: p.s = acc[1][1]; break;
    case 6: p.s = acc[2][1]; break;
    default: p.s = acc[3][1]; break;
  }
  p.vb0 = vt0 + 32 * mb + 4 * (lane >> 5);
  p.row = (uint32_t)(row0 + 64 * w + 32 * nb + fr);
  p.m = nb ? e.mt1 : e.mt0;
  p.sref = hw_exp2(p.m - (nb ? e.ref1 : e.ref0));  // <= 1
  const int rbg = 4 * w + 2 * nb + (fr >> 4);
  p.dst = ring_tile + ((rbg * 4 + mb) * 64 + (lane & 15)) * 16 + 8 * (lane >> 5);
  p.ls = 0.0f;
  p.as = 0.0f;
  p.gv = -INFINITY;
  p.gi = 0x7FFFFFFF;
}

template <bool kMasked>
__device__ __forceinline__ void piece_part(Piece& p, int q, int V, float c2, uint32_t step,
                                           uint32_t k0, uint32_t k1) {
  const int vb = p.vb0 + 8 * q;
  const u32x4 wd = philox4x32_10(u32x4{(uint32_t)vb >> 2, p.row, step, kTagGumbel}, k0, k1);
  float pv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float z2 = p.s[4 * q + j] * c2;
    const float dz = z2 - p.m;
    float pe = hw_exp2(dz);
    const float y = z2 + gumbel2_from_word(wd[j]);
    const bool ok = !kMasked || vb + j < V;
    pe = ok ? pe : 0.0f;
    p.ls += pe;
    p.as += ok ? pe * dz : 0.0f;
    argmax_merge(p.gv, p.gi, ok ? y : -INFINITY, vb + j);
    pv[j] = pe * p.sref;
  }
  const u32x2 pk{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
  *reinterpret_cast<u32x2*>(p.dst + 256 * q) = pk;
}

__device__ __forceinline__ void piece_end(const Piece& p, int piece, EpiState& e) {
  if (piece >= 4) {
    e.ls1 += p.ls;
    e.as1 += p.as;
    argmax_merge(e.gv1, e.gi1, p.gv, p.gi);
  } else {
    e.ls0 += p.ls;
    e.as0 += p.as;
    argmax_merge(e.gv0, e.gi0, p.gv, p.gi);
  }
}

// Whole pieces, not interleaved (first round of a job, tiles that reach past V).
__device__ __forceinline__ void epi_pieces(int first, const f32x16 (&acc)[4][2], EpiState& e,
                                           bool full, int vt0, int V, float c2, int row0,
                                           uint32_t step, uint32_t k0, uint32_t k1,
                                           char* ring_tile) {
#pragma unroll 1
  for (int piece = first; piece < 8; ++piece) {
    Piece p;
    piece_begin(p, piece, acc, e, vt0, row0, ring_tile);
    if (full) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        piece_part<false>(p, q, V, c2, step, k0, k1);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        piece_part<true>(p, q, V, c2, step, k0, k1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    piece_end(p, piece, e);
  }
}

// ---------------------------------------------------------------------------------------
// B step helpers.  E slice of one tile in LDS, row-major [128 vocab][DS columns].
// ---------------------------------------------------------------------------------------
// B operand of v_mfma_f32_16x16x32_bf16 for columns [16 cb, 16 cb + 16) and vocabulary
// [32 ks, 32 ks + 32): lane (g = lane / 16, i = lane % 16) needs E[32 ks + 8 g + 0..7][16 cb + i].
// Two transpose reads: lane j of a 16-lane group addresses row 32 ks + 8 g + 4 half + j / 4,
// columns 16 cb + 4 (j % 4) .. + 3; lane i then holds rows + 0..3 of column 16 cb + i.
template <int NCB>
__device__ __forceinline__ u32x4 et_frag(const lds_char* et, int cb, int ks) {
  constexpr int pitch = 32 * NCB;  // bytes per row
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int row = 32 * ks + 8 * g + (j >> 2);
  const int col = 16 * cb + 4 * (j & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(const_cast<lds_char*>(et) + row * pitch + 2 * col));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(const_cast<lds_char*>(et) + (row + 4) * pitch + 2 * col));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Multiply 8 bf16 by an exact power of two (the re-rounding is exact).
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float s) {
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(bf16_lo(v[k]) * s, bf16_hi(v[k]) * s);
  return o;
}

struct RowStats {
  float m, l, a, amv, gv;
  int ami, gi;
};
__device__ __forceinline__ void stats_reset(RowStats& s) {
  s.m = -INFINITY;
  s.l = 0.0f;
  s.a = 0.0f;
  s.amv = -INFINITY;
  s.gv = -INFINITY;
  s.ami = 0x7FFFFFFF;
  s.gi = 0x7FFFFFFF;
}

// ---------------------------------------------------------------------------------------
// Role barriers: the four A waves (and the four B waves) of a workgroup synchronise through
// an LDS counter, so that one role never waits for the other.  Bounded like the group waits.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ bool role_sync(int* ctr, int& gen, unsigned* err) {
  gen += 4;
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  unsigned it = 0;
  while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < gen) {
    if (++it > kSpinLimit) {
      atomicOr(err, 4u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Bounded wait of one wave until *p >= target.
__device__ __forceinline__ bool wave_wait(unsigned* p, unsigned target, unsigned* err) {
  unsigned it = 0;
  while (poll(p) < target) {
    if (poll(err) != 0u) return false;
    if (++it > kSpinLimit) {
      atomicOr(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

__device__ __forceinline__ void wave_signal(unsigned* p) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0) atomicAdd(p, 1u);
}

// Logits tile with the A role's own barrier.
__device__ __forceinline__ bool logits_tile_a(const uint16_t* E, const uint16_t* h, int V, int d,
                                              int v0, int row0, lds_char* smem,
                                              f32x16 (&acc)[4][2], int* bar, int& gen,
                                              unsigned* err) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{0};
  const int nk = d / kKC;
  const int fr = lane & 31, fh = lane >> 5;
  stage_a(E, h, V, d, v0, row0, 0, smem);
  if (!role_sync(bar, gen, err)) return false;
  for (int kc = 0; kc < nk; ++kc) {
    lds_char* cur = smem + (kc & 1) * kStageA;
    if (kc + 1 < nk) stage_a(E, h, V, d, v0, row0, (kc + 1) * kKC, smem + ((kc + 1) & 1) * kStageA);
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      u32x4 fa[4], fb[2];
      const int seg = 2 * ks + fh;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = 32 * mb + fr;
        fa[mb] = lds_read16(cur + row * 128 + 16 * (seg ^ (row & 7)));
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = 64 * w + 32 * nb + fr;
        fb[nb] = lds_read16(cur + kBV * 128 + row * 128 + 16 * (seg ^ (row & 7)));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[mb], fb[nb], acc[mb][nb]);
    }
    if (!role_sync(bar, gen, err)) return false;
  }
  return true;
}

// E slice of half a tile (64 vocabulary rows x DS columns, row-major) for the B role.  Each
// 64-lane instruction loads whole rows (kRpi rows of kRowChunks 16-byte chunks), so a lane's
// source offset is the same in every instruction up to a wave-uniform stride.
template <int NCB>
__device__ __forceinline__ void stage_b_half(const uint16_t* E, int V, int d, int v0, int col0,
                                             lds_char* st) {
  constexpr int DS = 16 * NCB;
  constexpr int kRowChunks = DS / 8;
  constexpr int kRpi = 64 / kRowChunks;               // rows per instruction
  constexpr int kInstr = (64 + kRpi - 1) / kRpi;      // instructions per half tile
  const int lane = threadIdx.x & 63, bw = (threadIdx.x >> 6) - 4;
  const int lr = lane / kRowChunks, cc = lane % kRowChunks;
  const bool active = lr < kRpi;
  const uint16_t* src = E + col0 + 8 * cc;
#pragma unroll
  for (int k = 0; k < (kInstr + 3) / 4; ++k) {
    const int i = bw + 4 * k;
    if (i < kInstr) {
      int v = v0 + i * kRpi + lr;
      v = v < V ? v : V - 1;
      if (active && i * kRpi + lr < 64) g2l16(src + (size_t)v * d, st + i * kRpi * (2 * DS));
    }
  }
}

struct SharedState {
  float sM[DG_CANVAS];        // group running row maximum (base 2, integer), this job
  float sMold[DG_CANVAS];
  int sMjob;                  // job the maxima belong to
  int sMask[2];               // per round parity: tiles whose probabilities need scaling
  int sRescale[2];            // per round parity: some row maximum grew
  int barA, barB;
  int sInfo[4];
};

// ---------------------------------------------------------------------------------------
// The kernel: 512 threads, waves 0-3 = A role, waves 4-7 = B role.
// ---------------------------------------------------------------------------------------
template <int NCB>
__global__ __launch_bounds__(512, 1) void k_vp_fused(Fused f) {
  constexpr int DS = 16 * NCB;
  constexpr int kStageB = 64 * DS * 2;  // half tile of the E slice
  __shared__ __attribute__((aligned(16))) char smem_a[kSmem];
  __shared__ __attribute__((aligned(16))) char smem_b[2 * kStageB];
  __shared__ SharedState ss;

  const uint16_t* E = f.a.E;
  const uint16_t* h = f.a.h;
  const int V = f.a.V, d = f.a.d, n_canvas = f.a.n_canvas;
  const uint8_t* commit = f.a.commit;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, fr = lane & 31;
  const size_t R = (size_t)n_canvas * DG_CANVAS;
  unsigned* err = f.sync + 8;
  const int n_tiles = f.n_tiles, s_v = f.s_v, n_groups = f.n_groups;

  // ---- group formation from the XCC id
  if (t == 0) {
    const int xcc = (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15);
    int ok = xcc < 8;
    unsigned slot = 0;
    if (ok) slot = atomicAdd(&f.sync[xcc], 1u);
    ok = ok && slot < (unsigned)f.per_xcd;
    const int gid = xcc * (f.per_xcd / kG) + (int)slot / kG;
    if (!ok || gid >= n_groups) {
      ok = 0;
      atomicOr(err, 2u);
    }
    int n_nc = n_canvas;
    if (commit != nullptr) {
      n_nc = 0;
      for (int c = 0; c < n_canvas; ++c) n_nc += commit[c] == 0;
    }
    ss.sInfo[0] = ok;
    ss.sInfo[1] = gid;
    ss.sInfo[2] = (int)(slot % kG);
    ss.sInfo[3] = n_nc;
    ss.barA = 0;
    ss.barB = 0;
    ss.sMjob = -1;
    ss.sMask[0] = ss.sMask[1] = 0;
    ss.sRescale[0] = ss.sRescale[1] = 0;
  }
  __syncthreads();  // the only whole-workgroup barrier
  if (!ss.sInfo[0]) return;
  const int gid = ss.sInfo[1], member = ss.sInfo[2], n_nc = ss.sInfo[3];
  unsigned* produced = f.sync + 16 + gid;
  unsigned* consumed = f.sync + 16 + n_groups + gid;
  uint16_t* ring = f.ring + (size_t)gid * 2 * kG * kTileElems;
  float* ring_ref = f.ring_ref + (size_t)gid * 2 * kG * DG_CANVAS;
  const int col0 = member * DS;
  const int n_jobs = n_canvas * s_v;
  const bool role_a = w < 4;
  int gen = 0;       // this wave's role-barrier generation
  unsigned rr = 0;   // heavy rounds of this group so far (identical in every wave)

  if (role_a) {
    for (int job = gid; job < n_jobs; job += n_groups) {
    int c = 0, vr;
    {
      const int heavy = n_nc * s_v;
      const bool want_nc = job < heavy;
      const int idx = want_nc ? job / s_v : (job - heavy) / s_v;
      vr = want_nc ? job % s_v : (job - heavy) % s_v;
      int seen = 0;
      for (int cc = 0; cc < n_canvas; ++cc) {
        const bool nc = commit == nullptr || commit[cc] == 0;
        if (nc == want_nc) {
          if (seen == idx) {
            c = cc;
            break;
          }
          ++seen;
        }
      }
    }
    const bool is_commit = commit != nullptr && commit[c] != 0;
    const int tb = (int)(((long long)n_tiles * vr) / s_v);
    const int te = (int)(((long long)n_tiles * (vr + 1)) / s_v);
    const int nr = (te - tb + kG - 1) / kG;
    const int row0 = c * DG_CANVAS;


      // ================================ A role ================================
      const float c2 = kLog2e / f.a.temperature[c];
      const uint32_t step = (uint32_t)f.a.step[c];
      const uint32_t k0 = f.a.k0, k1 = f.a.k1;
      RowStats st0, st1;
      stats_reset(st0);
      stats_reset(st1);
      f32x16 acc[4][2];
      for (int r = 0; r < nr; ++r) {
        const int tile = tb + r * kG + member;
        const bool a_valid = tile < te;
        const int vt0 = tile * kBV;
        const bool full = vt0 + kBV <= V;
        if (is_commit) {
          if (!a_valid) break;
          if (!logits_tile_a(E, h, V, d, vt0, row0, (lds_char*)smem_a, acc, &ss.barA, gen, err))
            return;
          float m[2], amv[2];
          int ami[2];
          tile_max_both(acc, full, vt0 + 4 * (lane >> 5), V, c2, m, amv, ami);
          argmax_merge(st0.amv, st0.ami, amv[0], ami[0]);
          argmax_merge(st1.amv, st1.ami, amv[1], ami[1]);
          continue;
        }
        // ring slot reuse: every B wave of the group has finished round rr - 2
        if (rr >= 2 && !wave_wait(consumed, 64u * (rr - 1), err)) return;
        if (a_valid) {
          if (!logits_tile_a(E, h, V, d, vt0, row0, (lds_char*)smem_a, acc, &ss.barA, gen, err))
            return;
          float mt[2], tamv[2];
          int tami[2];
          tile_max_both(acc, full, vt0 + 4 * (lane >> 5), V, c2, mt, tamv, tami);
          EpiState e;
          e.ls0 = e.ls1 = e.as0 = e.as1 = 0.0f;
          e.gv0 = e.gv1 = -INFINITY;
          e.gi0 = e.gi1 = 0x7FFFFFFF;
          e.mt0 = mt[0];
          e.mt1 = mt[1];
          // reference: this job's group maximum known so far (B role), else the tile max
          const bool mine = __hip_atomic_load(&ss.sMjob, __ATOMIC_ACQUIRE,
                                              __HIP_MEMORY_SCOPE_WORKGROUP) == job;
          const float M0 = mine ? ss.sM[64 * w + fr] : -INFINITY;
          const float M1 = mine ? ss.sM[64 * w + 32 + fr] : -INFINITY;
          e.ref0 = fmaxf(M0, mt[0]);
          e.ref1 = fmaxf(M1, mt[1]);
          char* ring_out =
              reinterpret_cast<char*>(ring + ((size_t)(rr & 1) * kG + member) * kTileElems);
          epi_pieces(0, acc, e, full, vt0, V, c2, row0, step, k0, k1, ring_out);
          e.ls0 += xor_f(e.ls0, 32);
          e.as0 += xor_f(e.as0, 32);
          argmax_merge(e.gv0, e.gi0, xor_f(e.gv0, 32), xor_i(e.gi0, 32));
          e.ls1 += xor_f(e.ls1, 32);
          e.as1 += xor_f(e.as1, 32);
          argmax_merge(e.gv1, e.gi1, xor_f(e.gv1, 32), xor_i(e.gi1, 32));
          float* rout = ring_ref + ((size_t)(rr & 1) * kG + member) * DG_CANVAS;
          if (lane < 32) {
            rout[64 * w + fr] = e.ref0;
            rout[64 * w + 32 + fr] = e.ref1;
          }
          lse_merge(st0.m, st0.l, st0.a, mt[0], e.ls0, e.as0);
          argmax_merge(st0.amv, st0.ami, tamv[0], tami[0]);
          argmax_merge(st0.gv, st0.gi, e.gv0, e.gi0);
          lse_merge(st1.m, st1.l, st1.a, mt[1], e.ls1, e.as1);
          argmax_merge(st1.amv, st1.ami, tamv[1], tami[1]);
          argmax_merge(st1.gv, st1.gi, e.gv1, e.gi1);
        }
        wave_signal(produced);
        ++rr;
      }
      if (lane < 32) {
        const size_t o0 = ((size_t)vr * kG + member) * R + row0 + 64 * w + fr;
        const size_t o1 = o0 + 32;
        f.st_amv[o0] = st0.amv;
        f.st_ami[o0] = st0.ami;
        f.st_m[o0] = st0.m;
        f.st_l[o0] = st0.l;
        f.st_a[o0] = st0.a;
        f.st_gv[o0] = st0.gv;
        f.st_gi[o0] = st0.gi;
        f.st_amv[o1] = st1.amv;
        f.st_ami[o1] = st1.ami;
        f.st_m[o1] = st1.m;
        f.st_l[o1] = st1.l;
        f.st_a[o1] = st1.a;
        f.st_gv[o1] = st1.gv;
        f.st_gi[o1] = st1.gi;
      }
    }
  } else {
    for (int job = gid; job < n_jobs; job += n_groups) {
    int c = 0, vr;
    {
      const int heavy = n_nc * s_v;
      const bool want_nc = job < heavy;
      const int idx = want_nc ? job / s_v : (job - heavy) / s_v;
      vr = want_nc ? job % s_v : (job - heavy) % s_v;
      int seen = 0;
      for (int cc = 0; cc < n_canvas; ++cc) {
        const bool nc = commit == nullptr || commit[cc] == 0;
        if (nc == want_nc) {
          if (seen == idx) {
            c = cc;
            break;
          }
          ++seen;
        }
      }
    }
    const bool is_commit = commit != nullptr && commit[c] != 0;
    const int tb = (int)(((long long)n_tiles * vr) / s_v);
    const int te = (int)(((long long)n_tiles * (vr + 1)) / s_v);
    const int nr = (te - tb + kG - 1) / kG;
    const int row0 = c * DG_CANVAS;

      if (is_commit) continue;

      // ================================ B role ================================
      const int bw = w - 4;
      const int tbt = t - 256;  // 0..255: the row this thread maintains
      // start of the job: reset the maxima (after the previous job's last use of them)
      if (!role_sync(&ss.barB, gen, err)) return;
      ss.sM[tbt] = -INFINITY;
      if (!role_sync(&ss.barB, gen, err)) return;
      if (tbt == 0) __hip_atomic_store(&ss.sMjob, job, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      f32x4 bacc[4][NCB];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) bacc[rb][cb] = f32x4{0, 0, 0, 0};
      for (int r = 0; r < nr; ++r) {
        if (!wave_wait(produced, 64u * (rr + 1), err)) return;
        asm volatile("buffer_inv sc0" ::: "memory");
        const uint16_t* ring_in = ring + (size_t)(rr & 1) * kG * kTileElems;
        const float* ref_in = ring_ref + (size_t)(rr & 1) * kG * DG_CANVAS;
        const int ptb = tb + r * kG;
        const int n_in = (te - ptb) < kG ? (te - ptb) : kG;
        const int par = rr & 1;
        // new running maxima and per-tile exponents (thread: row tbt)
        {
          const float mo = ss.sM[tbt];
          float mn = mo;
          for (int g = 0; g < n_in; ++g) mn = fmaxf(mn, ref_in[g * DG_CANVAS + tbt]);
          int mask = 0;
          for (int g = 0; g < n_in; ++g)
            if (ref_in[g * DG_CANVAS + tbt] != mn) mask |= 1 << g;
          ss.sMold[tbt] = mo;
          ss.sM[tbt] = mn;
          if (mask) atomicOr(&ss.sMask[par], mask);
          if (mn != mo && mo != -INFINITY) atomicOr(&ss.sRescale[par], 1);
        }
        if (!role_sync(&ss.barB, gen, err)) return;
        const int mask = ss.sMask[par];
        const int rescale = ss.sRescale[par];
        if (tbt == 0) {  // the other parity is next used two role barriers from now
          ss.sMask[par ^ 1] = 0;
          ss.sRescale[par ^ 1] = 0;
        }
        if (rescale) {
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = 64 * bw + 16 * rb + 4 * (lane >> 4) + i;
              const float mo = ss.sMold[row];
              const float sc = (mo == -INFINITY) ? 0.0f : hw_exp2(mo - ss.sM[row]);
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) bacc[rb][cb][i] *= sc;
            }
        }
        // stages: (tile g, half) pairs, E half tiles double-buffered
        const int n_st = 2 * n_in;
        stage_b_half<NCB>(E, V, d, ptb * kBV, col0, (lds_char*)smem_b);
        if (!role_sync(&ss.barB, gen, err)) return;
        for (int k = 0; k < n_st; ++k) {
          const int g = k >> 1, half = k & 1;
          const lds_char* et = (lds_char*)smem_b + (k & 1) * kStageB;
          const char* ptile = reinterpret_cast<const char*>(ring_in + (size_t)g * kTileElems);
          if (k + 1 < n_st)
            stage_b_half<NCB>(E, V, d, (ptb + ((k + 1) >> 1)) * kBV + 64 * ((k + 1) & 1), col0,
                              (lds_char*)smem_b + ((k + 1) & 1) * kStageB);
          const bool scaled = (mask >> g) & 1;
#pragma unroll
          for (int kl = 0; kl < 2; ++kl) {
            u32x4 fa[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
              fa[rb] = *reinterpret_cast<const u32x4*>(
                  ptile + (((4 * bw + rb) * 4 + 2 * half + kl) * 64 + lane) * 16);
            if (scaled) {
#pragma unroll
              for (int rb = 0; rb < 4; ++rb) {
                const int row = 64 * bw + 16 * rb + (lane & 15);
                const float rf = ref_in[g * DG_CANVAS + row];
                fa[rb] = scale_bf16x8(fa[rb], rf == -INFINITY ? 0.0f : hw_exp2(rf - ss.sM[row]));
              }
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              const u32x4 fb = et_frag<NCB>(et, cb, kl);
#pragma unroll
              for (int rb = 0; rb < 4; ++rb) bacc[rb][cb] = mfma16x16x32(fa[rb], fb, bacc[rb][cb]);
            }
          }
          if (!role_sync(&ss.barB, gen, err)) return;
        }
        wave_signal(consumed);
        ++rr;
      }
      // expectation partial of this (range, slice) and the final maxima
      float* out = f.accp + (size_t)vr * R * d;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 64 * bw + 16 * rb + 4 * (lane >> 4) + i;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            out[(size_t)(row0 + row) * d + col0 + 16 * cb + (lane & 15)] = bacc[rb][cb][i];
        }
      if (member == 0) f.accM[(size_t)vr * R + row0 + tbt] = ss.sM[tbt];
    }
  }
}

__global__ void k_vp_fused_init(unsigned* sync, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) sync[i] = 0u;
}

// Merge the partials of each row; sc = sum_range 2^(accM - m) accp / l.
__global__ __launch_bounds__(256) void k_vp_fused_combine(Fused f) {
  const size_t R = (size_t)f.a.n_canvas * DG_CANVAS;
  const int d = f.a.d;
  const int r = blockIdx.x;
  const int c = r / DG_CANVAS;
  const bool is_commit = f.a.commit != nullptr && f.a.commit[c] != 0;
  __shared__ float sm, sl, sbase[64];
  __shared__ int sbad;
  if (threadIdx.x == 0) {
    const bool bad = f.sync[8] != 0u;
    float m = -INFINITY, l = 0.0f, ac = 0.0f, amv = -INFINITY, gv = -INFINITY;
    int ami = 0x7FFFFFFF, gi = 0x7FFFFFFF;
    for (int p = 0; p < f.s_v * kG; ++p) {
      const size_t o = (size_t)p * R + r;
      argmax_merge(amv, ami, f.st_amv[o], f.st_ami[o]);
      if (!is_commit) {
        lse_merge(m, l, ac, f.st_m[o], f.st_l[o], f.st_a[o]);
        argmax_merge(gv, gi, f.st_gv[o], f.st_gi[o]);
      }
    }
    const int b = bad || ami == 0x7FFFFFFF;
    sbad = b;
    f.a.argmax_tok[r] = b ? -1 : ami;
    if (!is_commit) {
      const float lg = hw_log2(l);
      if (f.a.lse) f.a.lse[r] = b ? NAN : kLn2 * (m + lg);
      f.a.entropy[r] = b ? NAN : fmaxf(0.0f, kLn2 * (lg - ac / l));
      f.a.gumbel_tok[r] = b ? -1 : gi;
      sm = m;
      sl = l;
      for (int v = 0; v < f.s_v && v < 64; ++v) sbase[v] = f.accM[(size_t)v * R + r];
    }
  }
  __syncthreads();
  if (is_commit || f.a.selfcond == nullptr) return;
  const float linv = 1.0f / sl;
  const float m = sm;
  const bool b = sbad != 0;
  for (int k = threadIdx.x; k < d; k += blockDim.x) {
    float s = 0.0f;
    for (int v = 0; v < f.s_v; ++v) {
      const float base = sbase[v];
      if (base == -INFINITY) continue;
      s += hw_exp2(base - m) * f.accp[((size_t)v * R + r) * d + k];
    }
    f.a.selfcond[(size_t)r * d + k] = b ? NAN : s * linv;
  }
}

// Cooperative launch guarantees that the whole grid is resident.  DG_COOPERATIVE=0 uses an
// ordinary launch instead (one workgroup per CU still fits; waits stay bounded either way),
// for tools that do not follow cooperative dispatches.
template <int NCB>
hipError_t launch_fused(const Fused& f, int n_wg, hipStream_t stream) {
  const char* e = getenv("DG_COOPERATIVE");
  if (e != nullptr && strcmp(e, "0") == 0) {
    hipLaunchKernelGGL(k_vp_fused<NCB>, dim3(n_wg), dim3(512), 0, stream, f);
    return hipGetLastError();
  }
  void* args[] = {const_cast<Fused*>(&f)};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_vp_fused<NCB>), dim3(n_wg),
                                    dim3(512), args, 0, stream);
}

}  // namespace

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

bool fused_supported(int d) {
  if (d % (16 * kG) != 0) return false;
  const int ncb = d / (16 * kG);
  return ncb == 1 || ncb == 2 || ncb == 4 || ncb == 8 || ncb == 11;
}

FusedPlan fused_plan(int n_canvas, int V, int d, int n_wg) {
  FusedPlan p{};
  p.n_wg = n_wg;
  p.per_xcd = n_wg / 8;
  p.n_groups = 8 * (p.per_xcd / kG);
  p.R = (size_t)n_canvas * DG_CANVAS;
  p.n_tiles = (V + kBV - 1) / kBV;
  int sv = (p.n_groups + n_canvas - 1) / n_canvas;
  if (sv < 2) sv = 2;
  if (sv > p.n_tiles) sv = p.n_tiles;
  if (sv > 64) sv = 64;
  p.s_v = sv;
  size_t off = 0;
  p.off_sync = off;
  off += al256((16 + 2 * (size_t)p.n_groups) * 4);
  p.off_ring = off;
  off += al256((size_t)p.n_groups * 2 * kG * kTileElems * 2);
  p.off_ring_ref = off;
  off += al256((size_t)p.n_groups * 2 * kG * DG_CANVAS * 4);
  p.off_st = off;
  off += 7 * al256((size_t)p.s_v * kG * p.R * 4);
  p.off_accp = off;
  off += al256((size_t)p.s_v * p.R * d * 4);
  p.off_accM = off;
  off += al256((size_t)p.s_v * p.R * 4);
  p.bytes = off;
  return p;
}

hipError_t fused_launch(const VocabArgs& a, const FusedPlan& p, void* workspace,
                        hipStream_t stream) {
  char* b = static_cast<char*>(workspace);
  Fused f{};
  f.a = a;
  f.sync = reinterpret_cast<unsigned*>(b + p.off_sync);
  f.ring = reinterpret_cast<uint16_t*>(b + p.off_ring);
  f.ring_ref = reinterpret_cast<float*>(b + p.off_ring_ref);
  const size_t st = al256((size_t)p.s_v * kG * p.R * 4);
  f.st_m = reinterpret_cast<float*>(b + p.off_st + 0 * st);
  f.st_l = reinterpret_cast<float*>(b + p.off_st + 1 * st);
  f.st_a = reinterpret_cast<float*>(b + p.off_st + 2 * st);
  f.st_amv = reinterpret_cast<float*>(b + p.off_st + 3 * st);
  f.st_ami = reinterpret_cast<int*>(b + p.off_st + 4 * st);
  f.st_gv = reinterpret_cast<float*>(b + p.off_st + 5 * st);
  f.st_gi = reinterpret_cast<int*>(b + p.off_st + 6 * st);
  f.accp = reinterpret_cast<float*>(b + p.off_accp);
  f.accM = reinterpret_cast<float*>(b + p.off_accM);
  f.n_tiles = p.n_tiles;
  f.s_v = p.s_v;
  f.n_groups = p.n_groups;
  f.per_xcd = p.per_xcd;
  hipLaunchKernelGGL(k_vp_fused_init, dim3(1), dim3(256), 0, stream, f.sync, 16 + 2 * p.n_groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.d / (16 * kG)) {
    case 1: e = launch_fused<1>(f, p.n_wg, stream); break;
    case 2: e = launch_fused<2>(f, p.n_wg, stream); break;
    case 4: e = launch_fused<4>(f, p.n_wg, stream); break;
    case 8: e = launch_fused<8>(f, p.n_wg, stream); break;
    case 11: e = launch_fused<11>(f, p.n_wg, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_vp_fused_combine, dim3((unsigned)p.R), dim3(256), 0, stream, f);
  return hipGetLastError();
}

}  // namespace dg
