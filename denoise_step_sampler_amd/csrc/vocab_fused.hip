// Fused vocabulary pass for gfx950: one persistent cooperative kernel, no [R, V] buffer.
//
// Why cooperative: the self-conditioning expectation acc[256, d] += P_t E_t needs, for one
// canvas, 256 x d fp32 accumulators (2.9 MB at d = 2816), far more than one CU holds, while
// the logits S_t = E_t h^T need all of d for every vocabulary tile.  So the accumulator is
// split by columns over a half-group of 16 workgroups sharing one XCD (one L2), and each
// member produces the probability tile of one vocabulary tile per round for its half:
//
//   round r, member g:   A: S^T tile t = tb + 16 r + g  (128 vocab x 256 rows, all of d,
//                           bf16 MFMA 32x32x16) -> epilogue (softmax partial, entropy moment,
//                           argmax, Philox Gumbel-max) -> bf16 probabilities 2^(z2 - ref)
//                           into the group's L2 ring, in MFMA-fragment order
//                        B: acc[256, d/16 slice g] += P_t E_t[:, slice] for the 16 tiles of
//                           the previous round (bf16 MFMA 16x16x32)
//
// Staging: every operand moves global -> LDS by LDS DMA (global_load_lds_dwordx4), through
// three-stage rings, one per role.  The copies are issued in inline assembly and awaited with
// counted s_waitcnt vmcnt(N): the compiler cannot tell the stages apart and would otherwise
// hold every LDS read back until all copies in flight (the next stages too) had landed.  Both
// roles issue their copies in the order they consume them, so an in-order wait never stalls
// on a later stage.  The logits operands sit in XOR-swizzled 64-byte rows (conflict-free
// ds_read_b128); the E slice of the expectation sits row-major and is read with the LDS
// transpose read ds_read_b64_tr_b16, which delivers vocabulary-contiguous operand fragments
// from d-contiguous rows; the probability fragments are copied whole (1 KB per wave and row
// block) and read back contiguously.
//
// Probability reference: the A step writes 2^(z2 - ref) with ref = max(M, m_tile), M the
// group's running row maximum known to this workgroup (B step, same job) and m_tile the tile
// maximum, both in base-2 units, so every stored value is <= 1 and the tile holding the row
// maximum stores its largest probability as exactly 1.  The B step rescales a tile only when
// its ref differs from the group maximum after the round (rare once the maximum has settled);
// the accumulators are rescaled in fp32 when the maximum grows.
//
// Roles: each workgroup has 8 waves; waves 0-3 run the A step (logits + epilogue), waves 4-7
// the B step, so the epilogue's VALU work and the B MFMAs issue side by side on every SIMD.
// Within a role, waves synchronise through an LDS counter (never the workgroup barrier).
//
// Synchronisation across the group: per round parity, a counter of waves that published a
// round (A) and one of waves that consumed one (B), over both halves.  A of round q waits until
// every B wave finished round q - 2 (two ring slots), B of round q waits until every A wave
// published round q.  Keeping the parities apart makes each count exact: no wave can reach round q + 2
// of the same parity before the round q it would be confused with has been consumed.  Group
// members are formed from the hardware XCC id so that all ring traffic stays in one L2; the
// data is written with plain stores, completed (s_waitcnt) before the counter increment, and
// read after an L1 invalidate.  Every wait is bounded; on time-out the kernel raises an error
// flag, every wave leaves, and the combine kernel poisons the outputs (token -1, NaN
// statistics).
//
// Groups and halves: a group is the 32 workgroups of one XCD, in two halves of 16.  The halves
// run two jobs side by side (two canvases over the same vocabulary range), in one round count,
// so every E line one half streams is read by the other half from L2 within the same round:
// the E stream from beyond L2 is paid once per two canvases.  With fewer than 32 workgroups per
// XCD a group is one half.
//
// Jobs: (canvas, vocabulary range) pairs, non-commit canvases first, range-major, taken two
// at a time by the groups.  Commit canvases need only the argmax: no probabilities, no
// exchange.
#include <stdlib.h>
#include <string.h>

#include "dg_device.h"
#include "dg_internal.h"

namespace dg {
namespace {

typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kG = 16;          // workgroups per half-group (one d slice each)
constexpr int kBV = 128;        // vocabulary tile
constexpr int kKC = 32;         // d chunk of the logits contraction: 64 bytes per row
constexpr int kRowA = 2 * kKC;  // bytes of one staged row
constexpr int kStageA = (kBV + DG_CANVAS) * kRowA;  // one A stage: E chunk + h chunk, 24 KB
constexpr int kNStage = 3;                           // stages per role ring
constexpr int kSmemA = kNStage * kStageA;            // 72 KB
constexpr int kBQ = 32;         // vocabulary rows per B stage (a quarter tile)
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kTileElems = kBV * DG_CANVAS;          // bf16 probability tile: 64 KB

// B stage: E slice [32 rows][32 NCB bytes] (NCB KB), the probability fragments of the four
// B waves (4 row blocks x 1 KB each), and the references of the stage's tile (256 floats).
template <int NCB>
constexpr int b_stage_bytes() {
  return NCB * 1024 + 16 * 1024 + 1024;
}

struct Fused {
  VocabArgs a;
  unsigned* sync;     // [0, 8) per-XCC slot counters, [8] error flag, [9] non-commit
                      // canvases, [16 + 4 gid + p] produced and [16 + 4 gid + 2 + p] consumed
                      // counters of round parity p
  const int* order;   // [n_canvas] non-commit canvases first, each part in index order
  uint16_t* ring;     // [n_groups][2][halves * kG][kBV * 256]
  float* ring_ref;    // [n_groups][2][halves * kG][256]
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
  int halves;         // halves per group (1 or 2)
};

// Polls read one wave-uniform word; readfirstlane tells the compiler so, which keeps the
// control flow after every wait scalar (and the loop state out of vector registers).
__device__ __forceinline__ unsigned poll(const unsigned* p) {
  return __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ u32x4 lds_read16(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) {
  return (uint32_t)(uintptr_t)p;
}

// ---------------------------------------------------------------------------------------
// LDS DMA.  One instruction: lane l copies the 16 bytes at base + off (off per lane, base
// wave-uniform) to LDS byte address dst + 16 l (dst wave-uniform, through M0).  Every stream,
// E included, uses the ordinary cached form: an E line is read by several workgroups of the
// same XCD (the two halves, and the B role after the A role), and the non-temporal form was
// measured to lose those L2 hits.  M0 is free between instructions on gfx9 and later (LDS
// instructions no longer read it); the one-cycle nop covers the M0 -> LDS DMA hazard.
// ---------------------------------------------------------------------------------------
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(dst)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are outstanding.  Operations
// complete in issue order, so this waits for everything but the N most recent.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// ---------------------------------------------------------------------------------------
// Role barriers: the four A waves (and the four B waves) of a workgroup synchronise through
// an LDS counter, so that one role never waits for the other.  A wave arrives after its own
// copies into the stage it is about to read have landed (vm_wait before the call) and after
// its reads of the stage being refilled were issued; LDS executes a wave's operations in
// order, so those reads are done before the arrival is counted.  Bounded like the group
// waits: on time-out the flag `bad` is raised, later barriers stop waiting, and the caller
// leaves at its next check (the loops keep one exit, which keeps the accumulators in place).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void role_bar(int* ctr, int& gen, unsigned* err, bool& bad) {
  gen += 4;
  asm volatile("" ::: "memory");
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  unsigned it = 0;
  while (!bad && __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                     ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < gen) {
    if (++it > kSpinLimit) {
      atomicOr(err, 4u);
      bad = true;
    }
  }
  asm volatile("" ::: "memory");
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

// Publish: every store of this wave completes before the counter moves.
__device__ __forceinline__ void wave_signal(unsigned* p) {
  vm_wait<0>();
  if ((threadIdx.x & 63) == 0) atomicAdd(p, 1u);
}

// ---------------------------------------------------------------------------------------
// Jobs.
// ---------------------------------------------------------------------------------------
struct Sched {
  const int* order;
  int s_v, n_nc, n_tiles, n_jobs, n_heavy, n_groups;
  int halves, half, sub;  // halves per group; this workgroup's half and member within it
  int n_hpairs, n_pairs;  // job pairs of the group schedule: non-commit ones first
};

struct Job {
  int c, vr, tb, te, nr;
  bool commit;
};

// Jobs are numbered range-major within each part (non-commit, then commit), so that the two
// groups of one XCD, which take consecutive jobs, stream the same vocabulary tiles for two
// canvases at the same time and share every E line through their L2.
__device__ __forceinline__ Job job_at(const Sched& s, int job) {
  Job J;
  const bool nc = job < s.n_heavy;
  const int k = nc ? job : job - s.n_heavy;
  const int n_part = nc ? s.n_nc : s.n_jobs / s.s_v - s.n_nc;
  J.vr = k / n_part;
  const int idx = k - J.vr * n_part;
  J.c = __builtin_amdgcn_readfirstlane(s.order[nc ? idx : s.n_nc + idx]);  // wave-uniform
  J.commit = !nc;
  J.tb = (int)(((long long)s.n_tiles * J.vr) / s.s_v);
  J.te = (int)(((long long)s.n_tiles * (J.vr + 1)) / s.s_v);
  J.nr = (J.te - J.tb + kG - 1) / kG;
  return J;
}

// Job of half `half` in pair p (the halves of a group run the two jobs of a pair side by
// side), or -1 when the pair has no job for that half.
__device__ __forceinline__ int pair_job(const Sched& s, int p, int half) {
  if (p < s.n_hpairs) {
    const int j = s.halves * p + half;
    return j < s.n_heavy ? j : -1;
  }
  const int j = s.n_heavy + s.halves * (p - s.n_hpairs) + half;
  return j < s.n_jobs ? j : -1;
}

// Rounds of a non-commit pair: the longer of its jobs (the halves share one round count; the
// shorter job's half runs empty rounds).
__device__ __forceinline__ int pair_rounds(const Sched& s, int p) {
  int nr = 0;
  for (int hh = 0; hh < s.halves; ++hh) {
    const int j = pair_job(s, p, hh);
    if (j >= 0) nr = max(nr, job_at(s, j).nr);
  }
  return nr;
}

__device__ __forceinline__ Job half_job(const Sched& s, int p, int& job) {
  job = pair_job(s, p, s.half);
  if (job >= 0) return job_at(s, job);
  Job J;
  J.c = 0;
  J.vr = 0;
  J.tb = 0;
  J.te = 0;
  J.nr = 0;
  J.commit = p >= s.n_hpairs;
  return J;
}

// The A role's next logits tile after round r of pair p: this half's next round of the same
// job, else the first tile of this half in a later pair of the group.
__device__ __forceinline__ bool next_tile(const Sched& s, int p, int tb, int te, int row0,
                                          int r, int& v0n, int& row0n) {
  const int t = tb + kG * (r + 1) + s.sub;
  if (t < te) {
    v0n = t * kBV;
    row0n = row0;
    return true;
  }
  for (int p2 = p + s.n_groups; p2 < s.n_pairs; p2 += s.n_groups) {
    const int j = pair_job(s, p2, s.half);
    if (j < 0) continue;
    const Job J = job_at(s, j);
    if (J.tb + s.sub < J.te) {
      v0n = (J.tb + s.sub) * kBV;
      row0n = J.c * DG_CANVAS;
      return true;
    }
  }
  return false;
}

// ---------------------------------------------------------------------------------------
// A step: S^T tile (128 vocab x 256 rows) over all of d, in 32-wide chunks.  Wave w owns
// rows [64w, 64w + 64): acc[mb][nb] is the 32x32 block (vocabulary block mb, row block nb).
// LDS stage: E chunk [128 rows][4 x 16 B] then h chunk [256 rows][4 x 16 B]; 16-byte segment
// s of row r sits at slot s ^ ((r >> 2) & 3), so that the sixteen consecutive rows one
// ds_read_b128 cycle serves (256 bytes) hit sixteen distinct 16-byte bank groups.
// ---------------------------------------------------------------------------------------
struct ALanes {
  uint32_t rdE0, rdE1;  // LDS read offsets of this lane's E fragment rows, k steps 0 and 1
  uint32_t rdH0, rdH1;  // same for the h rows of this wave
  uint32_t offH;        // DMA: per-lane source offset (bytes) of an h copy
  uint32_t seg16;       // DMA: swizzled 16-byte segment of this lane
  int dlrow;            // DMA: row of this lane within a 16-row copy
};

__device__ __forceinline__ ALanes a_lanes(int w, int d) {
  ALanes k;
  const int lane = threadIdx.x & 63, fr = lane & 31, fh = lane >> 5;
  const int swz = (fr >> 2) & 3;
  k.rdE0 = fr * kRowA + 16 * ((0 + fh) ^ swz);
  k.rdE1 = fr * kRowA + 16 * ((2 + fh) ^ swz);
  k.rdH0 = kBV * kRowA + (64 * w + fr) * kRowA + 16 * ((0 + fh) ^ swz);
  k.rdH1 = kBV * kRowA + (64 * w + fr) * kRowA + 16 * ((2 + fh) ^ swz);
  k.dlrow = lane >> 2;
  k.seg16 = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  k.offH = (uint32_t)k.dlrow * (2u * (uint32_t)d) + k.seg16;
  return k;
}

// Copies of chunk kc of tile (v0, row0) into the stage at LDS address dst: wave w moves E
// rows [32w, 32w + 32) (clamped to V - 1 past the vocabulary) and its own h rows.
// Six DMA instructions per wave.
__device__ __forceinline__ void a_issue(const uint16_t* E, const uint16_t* h, int V, int d,
                                        int v0, int row0, int kc, uint32_t dst, int w,
                                        const ALanes& k) {
  const uint32_t pitch = 2u * (uint32_t)d;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rb = v0 + 32 * w + 16 * j;
    const int br = min(rb, V - 1);
    const int rv = min(rb + k.dlrow, V - 1);
    dma16(E + (size_t)br * d + kc * kKC, (uint32_t)(rv - br) * pitch + k.seg16,
             dst + 1024u * (uint32_t)(2 * w + j));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    dma16(h + (size_t)(row0 + 64 * w + 16 * j) * d + kc * kKC, k.offH,
          dst + (uint32_t)(kBV * kRowA) + 1024u * (uint32_t)(4 * w + j));
}
constexpr int kADma = 6;

__device__ __forceinline__ void a_compute(const lds_char* st, const ALanes& k,
                                          f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const lds_char* pe = st + (ks ? k.rdE1 : k.rdE0);
    const lds_char* ph = st + (ks ? k.rdH1 : k.rdH0);
    u32x4 fa[4], fb[2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) fa[mb] = lds_read16(pe + 32 * kRowA * mb);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) fb[nb] = lds_read16(ph + 32 * kRowA * nb);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32x32x16(fa[mb], fb[nb], acc[mb][nb]);
  }
}

__device__ __forceinline__ int stage_add2(int s) { return s == 0 ? 2 : s - 1; }
__device__ __forceinline__ int stage_add1(int s) { return s == kNStage - 1 ? 0 : s + 1; }

// The A role's copy stream runs across tiles: the last two chunks of a tile issue the first
// two chunks of the next one (pre = they are in flight), so a tile starts without a bubble.
struct APipe {
  int st;    // stage of the next chunk to compute
  bool pre;  // chunks 0 and 1 of the next tile are in flight (after the first tile: always)
};

__device__ __forceinline__ bool a_logits(const uint16_t* E, const uint16_t* h, int V, int d,
                                         int v0, int row0, bool has_next, int v0n, int row0n,
                                         APipe& p, lds_char* smem, int w, const ALanes& k,
                                         f32x16 (&acc)[4][2], int* bar, int& gen,
                                         unsigned* err) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{0};
  const int nk = d / kKC;
  const uint32_t base = lds_addr(smem);
  int s = p.st;
  bool bad = false;
  if (!p.pre) {
    a_issue(E, h, V, d, v0, row0, 0, base + s * kStageA, w, k);
    a_issue(E, h, V, d, v0, row0, 1, base + stage_add1(s) * kStageA, w, k);
  }
  // Chunk kc: its copies have landed (chunk kc + 1 may still be in flight) and every wave is
  // past chunk kc - 1, whose stage receives chunk kc + 2 of the stream.  Past the end of the
  // tile that is the next tile, or, when there is none, the first chunks of this one again:
  // the body stays free of branches (which keeps the accumulators in place) and every
  // iteration has the same number of copies in flight.
  const int vx = has_next ? v0n : v0;
  const int rx = has_next ? row0n : row0;
  for (int kc = 0; kc < nk; ++kc) {
    vm_wait<kADma>();
    role_bar(bar, gen, err, bad);
    const bool in = kc + 2 < nk;
    a_issue(E, h, V, d, in ? v0 : vx, in ? row0 : rx, in ? kc + 2 : kc + 2 - nk,
            base + stage_add2(s) * kStageA, w, k);
    a_compute(smem + s * kStageA, k, acc);
    s = stage_add1(s);
  }
  p.st = s;
  p.pre = true;
  if (bad) vm_wait<0>();
  return !bad;
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
    const float y = z2 + gumbel2s_from_word(wd[j]);
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

__device__ __forceinline__ void epi_pieces(const f32x16 (&acc)[4][2], EpiState& e, bool full,
                                           int vt0, int V, float c2, int row0, uint32_t step,
                                           uint32_t k0, uint32_t k1, char* ring_tile) {
#pragma unroll 1
  for (int piece = 0; piece < 8; ++piece) {
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
// B step.  A stage holds one 32-row quarter of a tile: the E slice row-major [32][DS] and
// the probability fragments of the four B waves.
// ---------------------------------------------------------------------------------------
// B operand of v_mfma_f32_16x16x32_bf16 for columns [16 cb, 16 cb + 16) and the stage's 32
// vocabulary rows: lane (g = lane / 16, i = lane % 16) needs E[8 g + 0..7][16 cb + i].  Two
// transpose reads: lane j of a 16-lane group addresses row 8 g + 4 half + j / 4, columns
// 16 cb + 4 (j % 4) .. + 3; lane i then holds rows + 0..3 of column 16 cb + i.
template <int NCB>
__device__ __forceinline__ u32x4 et_frag(const lds_char* et, int cb) {
  constexpr int pitch = 32 * NCB;  // bytes per row
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, j = lane & 15;
  const int row = 8 * g + (j >> 2);
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

// Multiply 8 bf16 by a power of two (the re-rounding is exact for normal results).
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

// Position of the B role in its stream of stages: (non-commit pair, round, stage of the
// round).  A round of this half has 4 stages per tile it holds, none in the empty rounds at the
// end of the shorter job of a pair (or all rounds of a pair without a job for this half).
struct BCur {
  int p, job, r, s, nst, ptb, tb, te, nr, c, vr;
  unsigned q;  // group round counter; ring slot and counter parity = q & 1
  bool valid;
};

__device__ __forceinline__ void b_round_set(BCur& u) {
  const int n_in = (u.job >= 0 && u.ptb < u.te) ? min(kG, u.te - u.ptb) : 0;
  u.nst = 4 * n_in;
}

__device__ __forceinline__ void b_load_pair(BCur& u, const Sched& sc) {
  u.valid = u.p < sc.n_hpairs;
  if (!u.valid) return;
  const Job J = half_job(sc, u.p, u.job);
  u.nr = pair_rounds(sc, u.p);
  u.c = J.c;
  u.vr = J.vr;
  u.tb = J.tb;
  u.te = J.te;
  u.r = 0;
  u.s = 0;
  u.ptb = J.tb;
  b_round_set(u);
}

__device__ __forceinline__ void b_next_round(BCur& u, const Sched& sc) {
  u.s = 0;
  ++u.q;
  if (++u.r < u.nr) {
    u.ptb += kG;
    b_round_set(u);
    return;
  }
  u.p += sc.n_groups;
  b_load_pair(u, sc);
}

__device__ __forceinline__ void b_advance(BCur& u, const Sched& sc) {
  if (++u.s < u.nst) return;
  b_next_round(u, sc);
}

// Copies of one B stage: E rows [v0, v0 + 32) x columns [col0, col0 + 16 NCB) as NCB 1-KB
// instructions (chunk c = 64 i + lane is row c / (2 NCB), 16-byte column chunk c % (2 NCB)),
// dealt round-robin to the four B waves; this wave's four probability fragments; and, by the
// last wave (which has the fewest E copies), the 256 references of the tile.
template <int NCB>
__device__ __forceinline__ void b_issue(const uint16_t* E, const uint16_t* ring,
                                        const float* ring_ref, int V, int d, int col0,
                                        int slot_tiles, int hoff, const BCur& u, uint32_t dst,
                                        int bw) {
  const int lane = threadIdx.x & 63;
  const int g = u.s >> 2, kq = u.s & 3;
  const int v0 = (u.ptb + g) * kBV + kBQ * kq;
  const int br = min(v0, V - 1);
  const uint16_t* eb = E + (size_t)br * d + col0;
#pragma unroll
  for (int j = 0; j < (NCB + 3) / 4; ++j) {
    const int i = bw + 4 * j;
    if (i < NCB) {
      const int c = 64 * i + lane;
      const int row = c / (2 * NCB), cc = c - row * (2 * NCB);
      const int rv = min(v0 + row, V - 1);
      dma16(eb, (uint32_t)(rv - br) * (2u * (uint32_t)d) + 16u * (uint32_t)cc,
               dst + 1024u * (uint32_t)i);
    }
  }
  const uint16_t* pb = ring + ((size_t)(u.q & 1) * slot_tiles + hoff + g) * kTileElems;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    dma16(pb + ((4 * bw + rb) * 4 + kq) * 512, 16u * (uint32_t)lane,
          dst + (uint32_t)(NCB * 1024 + 4096 * bw + 1024 * rb));
  if (bw == 3)
    dma16(ring_ref + ((size_t)(u.q & 1) * slot_tiles + hoff + g) * DG_CANVAS, 16u * (uint32_t)lane,
          dst + (uint32_t)(NCB * 1024 + 16384));
}

// One B stage.  A tile whose reference differs from the row maximum after the round (for
// some row) has its fragments scaled by 2^(ref - M) per row, from the stage's copy of the
// references.
template <int NCB>
__device__ __forceinline__ void b_compute(const lds_char* st, int bw, bool scaled,
                                          const float* Mn, f32x4 (&bacc)[4][NCB]) {
  const int lane = threadIdx.x & 63;
  u32x4 fa[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    fa[rb] = lds_read16(st + NCB * 1024 + 4096 * bw + 1024 * rb + 16 * lane);
  if (scaled) {
    const __attribute__((address_space(3))) float* refg =
        reinterpret_cast<const __attribute__((address_space(3))) float*>(st + NCB * 1024 +
                                                                          16384);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = 64 * bw + 16 * rb + (lane & 15);
      const float rf = refg[row];
      fa[rb] = scale_bf16x8(fa[rb], rf == -INFINITY ? 0.0f : hw_exp2(rf - Mn[row]));
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const u32x4 fb = et_frag<NCB>(st, cb);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) bacc[rb][cb] = mfma16x16x32(fa[rb], fb, bacc[rb][cb]);
  }
}

// vm_wait with a wave-uniform count n in [4, 7]: a uniform branch to the immediate form.
__device__ __forceinline__ void vm_wait_n(int n) {
  if (n >= 7) {
    vm_wait<7>();
  } else if (n == 6) {
    vm_wait<6>();
  } else if (n == 5) {
    vm_wait<5>();
  } else {
    vm_wait<4>();
  }
}

struct SharedState {
  float sM[DG_CANVAS];        // group running row maximum (base 2) of job sMjob, for the A role
  float sMn[2][DG_CANVAS];    // per round parity: row maximum after the round
  int sMjob;                  // job the maxima in sM belong to (-1: none)
  int sMask[2];               // per round parity: tiles whose probabilities need scaling
  int sResc[2];               // per round parity: some row maximum grew
  int barA, barB;
  int sInfo[4];
};

// ---------------------------------------------------------------------------------------
// The kernel: 512 threads, waves 0-3 = A role, waves 4-7 = B role.
// ---------------------------------------------------------------------------------------
template <int NCB>
__global__ __launch_bounds__(512, 1) void k_vp_fused(Fused f) {
  constexpr int DS = 16 * NCB;
  constexpr int kStageB = b_stage_bytes<NCB>();
  __shared__ __attribute__((aligned(1024))) char smem_a[kSmemA];
  __shared__ __attribute__((aligned(1024))) char smem_b[kNStage * kStageB];
  __shared__ SharedState ss;

  const uint16_t* E = f.a.E;
  const uint16_t* h = f.a.h;
  const int V = f.a.V, d = f.a.d, n_canvas = f.a.n_canvas;
  const int t = threadIdx.x, lane = t & 63, fr = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const size_t R = (size_t)n_canvas * DG_CANVAS;
  unsigned* err = f.sync + 8;
  const int n_tiles = f.n_tiles, s_v = f.s_v, n_groups = f.n_groups;

  // ---- group formation from the XCC id
  if (t == 0) {
    const int xcc = (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15);
    int ok = xcc < 8;
    unsigned slot = 0;
    if (ok) slot = atomicAdd(&f.sync[xcc], 1u);
    const int gs = kG * f.halves;
    ok = ok && slot < (unsigned)((f.per_xcd / gs) * gs);
    const int gid = xcc * (f.per_xcd / gs) + (int)slot / gs;
    if (!ok || gid >= n_groups) {
      ok = 0;
      atomicOr(err, 2u);
    }
    ss.sInfo[0] = ok;
    ss.sInfo[1] = gid;
    ss.sInfo[2] = (int)(slot % gs);
    ss.sInfo[3] = (int)f.sync[9];
    ss.barA = 0;
    ss.barB = 0;
    ss.sMjob = -1;
    ss.sMask[0] = ss.sMask[1] = 0;
    ss.sResc[0] = ss.sResc[1] = 0;
  }
  __syncthreads();  // the only whole-workgroup barrier
  if (!ss.sInfo[0]) return;
  const int gid = __builtin_amdgcn_readfirstlane(ss.sInfo[1]);
  const int member = __builtin_amdgcn_readfirstlane(ss.sInfo[2]);
  const int halves = f.halves;
  const int slot_tiles = kG * halves;  // tiles per ring slot
  Sched sc;
  sc.order = f.order;
  sc.s_v = s_v;
  sc.n_nc = __builtin_amdgcn_readfirstlane(ss.sInfo[3]);
  sc.n_tiles = n_tiles;
  sc.n_jobs = n_canvas * s_v;
  sc.n_heavy = sc.n_nc * s_v;
  sc.n_groups = n_groups;
  sc.halves = halves;
  sc.half = member / kG;
  sc.sub = member % kG;
  sc.n_hpairs = (sc.n_heavy + halves - 1) / halves;
  sc.n_pairs = sc.n_hpairs + (sc.n_jobs - sc.n_heavy + halves - 1) / halves;
  const int sub = sc.sub, hoff = sc.half * kG;
  const unsigned per_round = 64u * (unsigned)halves;  // counter increments per round
  unsigned* produced = f.sync + 16 + 4 * gid;
  unsigned* consumed = produced + 2;
  uint16_t* ring = f.ring + (size_t)gid * 2 * slot_tiles * kTileElems;
  float* ring_ref = f.ring_ref + (size_t)gid * 2 * slot_tiles * DG_CANVAS;
  int gen = 0;  // this wave's role-barrier generation

  if (w < 4) {
    // ================================ A role ================================
    const float* temperature = f.a.temperature;
    const int32_t* steps = f.a.step;
    const uint32_t k0 = f.a.k0, k1 = f.a.k1;
    float* st_m = f.st_m;
    float* st_l = f.st_l;
    float* st_a = f.st_a;
    float* st_amv = f.st_amv;
    int* st_ami = f.st_ami;
    float* st_gv = f.st_gv;
    int* st_gi = f.st_gi;
    const ALanes k = a_lanes(w, d);
    APipe pipe{0, false};
    unsigned rr = 0;  // heavy rounds of this group so far
    f32x16 acc[4][2];
    for (int pr = gid; pr < sc.n_pairs; pr += n_groups) {
      int job;
      const Job J = half_job(sc, pr, job);
      const bool heavy = pr < sc.n_hpairs;
      const int nr = heavy ? pair_rounds(sc, pr) : J.nr;
      const int row0 = J.c * DG_CANVAS;
      const float c2 = kLog2e / temperature[J.c];
      const uint32_t step = (uint32_t)steps[J.c];
      RowStats st0, st1;
      stats_reset(st0);
      stats_reset(st1);
      for (int r = 0; r < nr; ++r) {
        const int tile = J.tb + r * kG + sub;
        const bool valid = tile < J.te;
        const int vt0 = tile * kBV;
        const bool full = vt0 + kBV <= V;
        if (!heavy) {
          if (!valid) break;
          int v0n = 0, row0n = 0;
          const bool hn = next_tile(sc, pr, J.tb, J.te, row0, r, v0n, row0n);
          if (!a_logits(E, h, V, d, vt0, row0, hn, v0n, row0n, pipe, (lds_char*)smem_a, w, k,
                        acc, &ss.barA, gen, err))
            return;
          float m[2], amv[2];
          int ami[2];
          tile_max_both(acc, full, vt0 + 4 * (lane >> 5), V, c2, m, amv, ami);
          argmax_merge(st0.amv, st0.ami, amv[0], ami[0]);
          argmax_merge(st1.amv, st1.ami, amv[1], ami[1]);
          continue;
        }
        const unsigned par = rr & 1;
        // ring slot par is free once every B wave of the group has consumed round rr - 2
        if (rr >= 2 && !wave_wait(consumed + par, per_round * (rr >> 1), err)) {
          vm_wait<0>();
          return;
        }
        if (valid) {
          int v0n = 0, row0n = 0;
          const bool hn = next_tile(sc, pr, J.tb, J.te, row0, r, v0n, row0n);
          if (!a_logits(E, h, V, d, vt0, row0, hn, v0n, row0n, pipe, (lds_char*)smem_a, w, k,
                        acc, &ss.barA, gen, err))
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
          char* ring_out = reinterpret_cast<char*>(
              ring + ((size_t)par * slot_tiles + hoff + sub) * kTileElems);
          epi_pieces(acc, e, full, vt0, V, c2, row0, step, k0, k1, ring_out);
          e.ls0 += xor_f(e.ls0, 32);
          e.as0 += xor_f(e.as0, 32);
          argmax_merge(e.gv0, e.gi0, xor_f(e.gv0, 32), xor_i(e.gi0, 32));
          e.ls1 += xor_f(e.ls1, 32);
          e.as1 += xor_f(e.as1, 32);
          argmax_merge(e.gv1, e.gi1, xor_f(e.gv1, 32), xor_i(e.gi1, 32));
          float* rout = ring_ref + ((size_t)par * slot_tiles + hoff + sub) * DG_CANVAS;
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
        wave_signal(produced + par);
        ++rr;
      }
      if (job >= 0 && lane < 32) {
        const size_t o0 = ((size_t)J.vr * kG + sub) * R + row0 + 64 * w + fr;
        const size_t o1 = o0 + 32;
        st_amv[o0] = st0.amv;
        st_ami[o0] = st0.ami;
        st_m[o0] = st0.m;
        st_l[o0] = st0.l;
        st_a[o0] = st0.a;
        st_gv[o0] = st0.gv;
        st_gi[o0] = st0.gi;
        st_amv[o1] = st1.amv;
        st_ami[o1] = st1.ami;
        st_m[o1] = st1.m;
        st_l[o1] = st1.l;
        st_a[o1] = st1.a;
        st_gv[o1] = st1.gv;
        st_gi[o1] = st1.gi;
      }
    }
    vm_wait<0>();
    return;
  }

  // ================================ B role ================================
  const int bw = w - 4;
  const int tbt = t - 256;  // 0..255: the row this thread maintains
  const int col0 = sub * DS;
  const int nB = (NCB - bw + 3) / 4 + 4 + (bw == 3);  // copies per stage of this wave
  float* accp = f.accp;
  float* accM = f.accM;
  const uint32_t bbase = lds_addr((lds_char*)smem_b);
  BCur cu;
  cu.p = gid;
  cu.q = 0;
  b_load_pair(cu, sc);
  if (!cu.valid) return;
  BCur iu = cu;
  int s_issue = 0, s_comp = 0;
  int inflight = 0;  // stages issued and not yet computed
  f32x4 bacc[4][NCB];
  int mask = 0;
  bool bad = false;

  // Start of a round (at issue time, two stages before it is computed): wait for its data,
  // then fold its tile references into the row maxima of this thread's row.
  auto round_prep = [&](const BCur& u) -> bool {
    const unsigned par = u.q & 1;
    if (!wave_wait(produced + par, per_round * ((u.q >> 1) + 1), err)) return false;
    asm volatile("buffer_inv sc0" ::: "memory");
    const float* ref = ring_ref + ((size_t)par * slot_tiles + hoff) * DG_CANVAS + tbt;
    const int n_in = u.nst >> 2;
    float rv[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) rv[g] = g < n_in ? ref[g * DG_CANVAS] : -INFINITY;
    const float mo = (u.r == 0) ? -INFINITY : ss.sMn[par ^ 1][tbt];
    float mn = mo;
#pragma unroll
    for (int g = 0; g < kG; ++g) mn = fmaxf(mn, rv[g]);
    int m = 0;
#pragma unroll
    for (int g = 0; g < kG; ++g) m |= (g < n_in && rv[g] != mn) ? (1 << g) : 0;
    ss.sMn[par][tbt] = mn;
    if (m) atomicOr(&ss.sMask[par], m);
    if (mo != -INFINITY && mn != mo) atomicOr(&ss.sResc[par], 1);
    return true;
  };
  // Issue the next stage of the stream (empty rounds carry none).
  auto issue_next = [&]() -> bool {
    while (iu.valid && iu.nst == 0) b_next_round(iu, sc);
    if (!iu.valid) return true;
    if (iu.s == 0 && !round_prep(iu)) return false;
    b_issue<NCB>(E, ring, ring_ref, V, d, col0, slot_tiles, hoff, iu,
                 bbase + s_issue * kStageB, bw);
    s_issue = stage_add1(s_issue);
    ++inflight;
    b_advance(iu, sc);
    return true;
  };

  // Empty rounds of this half: nothing to read, but the counts stay exact (a round is counted
  // as consumed only once it has been published).  Run where the compute cursor enters them,
  // outside the stage body, which keeps the accumulators on one path.
  auto skip_empty = [&]() -> bool {
    while (cu.valid && cu.nst == 0) {
      const unsigned par = cu.q & 1;
      if (!wave_wait(produced + par, per_round * ((cu.q >> 1) + 1), err)) return false;
      if (lane == 0) atomicAdd(consumed + par, 1u);
      b_next_round(cu, sc);
    }
    return true;
  };

#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) bacc[rb][cb] = f32x4{0, 0, 0, 0};
  bool ok = issue_next() && issue_next() && skip_empty();
  while (ok && cu.valid) {
    const unsigned par = cu.q & 1;
    // this wave's copies of the stage have landed (the next stage may still be in flight)
    if (inflight >= 2)
      vm_wait_n(nB);
    else
      vm_wait<0>();
    role_bar(&ss.barB, gen, err, bad);
    if (bad || !issue_next()) break;
    if (cu.s == 0) {
      if (cu.r == 0) {
        // new job: publish the maxima under the new job id (the accumulators start at zero)
        if (tbt == 0) __hip_atomic_store(&ss.sMjob, -1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        role_bar(&ss.barB, gen, err, bad);
        ss.sM[tbt] = ss.sMn[par][tbt];
        role_bar(&ss.barB, gen, err, bad);
        if (tbt == 0)
          __hip_atomic_store(&ss.sMjob, cu.job, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        ss.sM[tbt] = ss.sMn[par][tbt];
      }
      mask = ss.sMask[par];
      if (cu.r != 0 && ss.sResc[par]) {
        // the previous round of this job left its maxima in the other parity
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 64 * bw + 16 * rb + 4 * (lane >> 4) + i;
            const float sf = hw_exp2(ss.sMn[par ^ 1][row] - ss.sMn[par][row]);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) bacc[rb][cb][i] *= sf;
          }
      }
    } else if (cu.s == 1 && tbt == 0) {
      // every B wave read this round's flags at stage 0; the next writer is two rounds ahead
      ss.sMask[par] = 0;
      ss.sResc[par] = 0;
    }
    const int g = cu.s >> 2;
    b_compute<NCB>((lds_char*)smem_b + s_comp * kStageB, bw, (mask >> g) & 1, ss.sMn[par],
                   bacc);
    --inflight;
    if (cu.s == cu.nst - 1) {
      // this wave's reads of the round's ring slot are complete
      if (lane == 0) atomicAdd(consumed + par, 1u);
      if (cu.r == cu.nr - 1 || cu.ptb + kG >= cu.te) {
        // last round of the job: expectation partial of this (range, slice), final maxima
        float* out = accp + (size_t)cu.vr * R * d;
        const int row0 = cu.c * DG_CANVAS;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 64 * bw + 16 * rb + 4 * (lane >> 4) + i;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              out[(size_t)(row0 + row) * d + col0 + 16 * cb + (lane & 15)] = bacc[rb][cb][i];
          }
        if (sub == 0) accM[(size_t)cu.vr * R + row0 + tbt] = ss.sMn[par][tbt];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) bacc[rb][cb] = f32x4{0, 0, 0, 0};
      }
    }
    s_comp = stage_add1(s_comp);
    b_advance(cu, sc);
    ok = skip_empty();
  }
  vm_wait<0>();
}

// Zero the counters; order the canvases (non-commit first, each part ascending) and count
// the non-commit ones.
__global__ __launch_bounds__(256) void k_vp_fused_init(unsigned* sync, int n_sync, int* order,
                                                       const uint8_t* commit, int n) {
  __shared__ int cnt[256];
  __shared__ int total;
  const int t = threadIdx.x;
  for (int i = t; i < n_sync; i += 256) sync[i] = 0u;
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
    sync[9] = (unsigned)run;
  }
  __syncthreads();
  int a = cnt[t];                   // non-commit canvases before lo
  int b = total + (lo - cnt[t]);    // commit canvases before lo, after all non-commit ones
  for (int c = lo; c < hi; ++c) {
    if (commit == nullptr || commit[c] == 0)
      order[a++] = c;
    else
      order[b++] = c;
  }
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
  p.halves = p.per_xcd >= 2 * kG ? 2 : 1;
  p.n_groups = 8 * (p.per_xcd / (kG * p.halves));
  p.R = (size_t)n_canvas * DG_CANVAS;
  p.n_tiles = (V + kBV - 1) / kBV;
  int sv = (p.n_groups * p.halves + n_canvas - 1) / n_canvas;
  if (sv < 2) sv = 2;
  if (sv > p.n_tiles) sv = p.n_tiles;
  if (sv > 64) sv = 64;
  p.s_v = sv;
  size_t off = 0;
  p.off_sync = off;
  off += al256((16 + 4 * (size_t)p.n_groups) * 4);
  p.off_order = off;
  off += al256((size_t)n_canvas * 4);
  p.off_ring = off;
  off += al256((size_t)p.n_groups * 2 * kG * p.halves * kTileElems * 2);
  p.off_ring_ref = off;
  off += al256((size_t)p.n_groups * 2 * kG * p.halves * DG_CANVAS * 4);
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
  f.order = reinterpret_cast<const int*>(b + p.off_order);
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
  f.halves = p.halves;
  hipLaunchKernelGGL(k_vp_fused_init, dim3(1), dim3(256), 0, stream, f.sync,
                     16 + 4 * p.n_groups, reinterpret_cast<int*>(b + p.off_order), a.commit,
                     a.n_canvas);
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
