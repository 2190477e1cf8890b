// gemm.h -- bf16 GEMM core for gfx950: C[m, n] = sum_k A[m, k] * B[n, k],
// fp32 accumulation in MFMA (v_mfma_f32_32x32x16_bf16).  Both operands are
// K-contiguous ("out x in" weights), so every copy and every LDS fragment
// read is 16 bytes per lane.
//
// Block tile 256 x 256 over 8 waves in a 2 x 4 grid, each wave 128 x 64 =
// 4 x 2 MFMA tiles (128 fp32 accumulators per lane, two waves per SIMD, one
// block per CU).  Global -> LDS moves use the gfx950 direct path
// (global_load_lds_dwordx4: no register staging).  The copy engine writes
// each wave's 64 x 16 B contiguously, so lane l of a copy slot fetches the
// chunk that belongs at position 64 * (slot's wave position) + l.  Two main
// loops (MOE_GEMM_CFG):
//
//   1: K tiles of 64 in a 2-stage ring (2 x 64 KB).  Per K tile every wave
//      waits for its copies (vmcnt), barrier, issues the copy of the next
//      tile into the other stage, and runs 4 k-steps of MFMAs, reading the
//      fragments of k-step kk + 1 while those of kk run.
//
//   2 (default): ping-pong.  The waves of rows 0..127 (group 0, waves 0-3,
//      one per SIMD) and of rows 128..255 (group 1, waves 4-7) alternate
//      roles every phase: one group runs the 16 MFMAs of one K tile (32
//      wide) from registers while the other group reads its fragments of
//      the next tile from LDS and issues copies.  Each SIMD then always has
//      one wave with MFMAs ready, and a barrier falls while the other wave's
//      last MFMA is still in the pipe.  K tiles sit in a 5-stage ring
//      (5 x 32 KB = 160 KB), issued 4 tiles ahead, so about 7 phases of MFMA
//      time cover each copy's latency.
//
// A stage row is GBK * 2 bytes = GCPR chunks of 16 B; chunk c of row r is
// stored at c ^ g_swz(r), so that the ds_read_b128 of a fragment (32
// consecutive rows, two adjacent chunks) runs at the full LDS rate
// (measured on gfx950: about 240 of 256 B/clk/CU for both row widths).
#pragma once
#include "common.h"

namespace moe {

#ifndef MOE_GEMM_CFG
#define MOE_GEMM_CFG 2
#endif
#if MOE_GEMM_CFG == 1
constexpr int GBK = 64, GNST = 2;
constexpr bool GPP = false;
#else
constexpr int GBK = 32, GNST = 5;
constexpr bool GPP = true;
#endif
constexpr int GBM = 256, GBN = 256, GWM = 2, GWN = 4;
constexpr int GNT = 64 * GWM * GWN;                 // threads per block
constexpr int GWTM = GBM / GWM, GWTN = GBN / GWN;   // wave tile (128 x 64)
constexpr int GTM = GWTM / 32, GTN = GWTN / 32;     // MFMA tiles per wave
constexpr int GCPR = GBK / 8;                       // 16-byte chunks per stage row
constexpr int GSA = GBM * GBK, GSB = GBN * GBK;     // elements per operand stage
// threads that copy one operand, and copies per such thread per K tile
constexpr int GCT = GPP ? GNT / 2 : GNT;
constexpr int GCA = GBM * GCPR / GCT, GCB = GBN * GCPR / GCT;
constexpr int GMINWAVES = 2;                        // waves per SIMD the kernels are built for
static_assert(GWTM == 128 && GWTN == 64, "wave tile 128 x 64");
static_assert(GNST * (GSA + GSB) * 2 <= 163840, "LDS ring");
static_assert(!GPP || (GCA == GCB && GWM == 2 && GBK == 32 && GNST == 5),
              "ping-pong: one operand per group, one 32-wide K tile per phase, 5 stages");

// Ping-pong group of this wave (0: waves 0-3, 1: waves 4-7), as a
// wave-uniform (scalar) value so that role branches stay scalar.
__device__ __forceinline__ bool g_group1() {
  return __builtin_amdgcn_readfirstlane((int)threadIdx.x) >= GCT;
}

typedef f32x16 GAcc[GTM][GTN];

struct GemmLds {
  uint16_t *A[GNST];
  uint16_t *B[GNST];
};

#define MOE_GEMM_LDS(name)                                                         \
  __shared__ __attribute__((aligned(16))) uint16_t name##_ring[GNST * (GSA + GSB)];   \
  GemmLds name;                                                                     \
  _Pragma("unroll") for (int _s = 0; _s < GNST; ++_s) {                             \
    name.A[_s] = name##_ring + _s * (GSA + GSB);                                    \
    name.B[_s] = name##_ring + _s * (GSA + GSB) + GSA;                              \
  }

// Chunk permutation of a stage row.  It depends on row bits 0..4 only, so
// fragment tiles 32 rows apart share it and their addresses differ by an
// immediate.  Both forms were chosen by measurement: for 4 chunks per row,
// ((r >> 1) ^ (r >> 3)) & 3 reads at half rate while (r ^ (r >> 2)) & 3 is
// conflict-free; for 8 chunks per row the form below is conflict-free.
__device__ __forceinline__ int g_swz(int row) {
  return GCPR == 4 ? ((row ^ (row >> 2)) & 3) : ((row & 6) | ((row ^ (row >> 3)) & 1));
}

// Tile row whose chunk this thread copies in copy slot i (in the ping-pong
// loop group 1 copies A and group 0 copies B, 256 threads each).
__device__ __forceinline__ int g_load_row(int i) {
  return (i * GCT + (int)threadIdx.x % GCT) / GCPR;
}

// Operand source of one block tile: a wave-uniform base address (row 0 of
// the tile region, K column 0) and, per copy slot of this thread, the byte
// offset of its row and (swizzled) chunk.  K tile kt adds kt * GBK * 2 bytes
// to the base, so the per-lane state is one 32-bit offset per slot.
template <int NC>
struct GOperand {
  const uint16_t *base;
  uint32_t off[NC];
};

__device__ __forceinline__ const uint16_t *g_uniform(const uint16_t *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint16_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Slot i of this thread copies chunk c = lane % GCPR (stored swizzled) of
// tile row g_load_row(i); operand rows are `ld` elements apart and
// row_of(r) maps the tile row to the source row (clamping, gathering).
template <int NC, class RowOf>
__device__ __forceinline__ GOperand<NC> g_operand(const uint16_t *base, int64_t ld,
                                                  RowOf row_of) {
  GOperand<NC> o;
  o.base = g_uniform(base);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int r = g_load_row(i);
    const int c = (lane_id() % GCPR) ^ g_swz(r);
    o.off[i] = (uint32_t)((int64_t)row_of(r) * ld * 2 + c * 16);
  }
  return o;
}

// LDS byte address of a generic pointer into LDS: the low 32 bits of its
// flat address (the LDS aperture maps offset o to aperture base + o).  An
// address-space cast would add a null check per use, in scalar registers the
// GEMM loops are short of.
__device__ __forceinline__ uint32_t g_lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

// One 16-byte-per-lane copy global -> LDS: the wave's 64 chunks land at
// lds_base + 16 * lane.  Written as inline asm so that the compiler does not
// guard later LDS reads with waits of its own: completion is tracked
// explicitly (vmcnt) and published to the block with a barrier.  M0 (the
// LDS destination) is restored afterwards.
__device__ __forceinline__ void g_copy16(const uint16_t *sbase, uint32_t voff,
                                         const uint16_t *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(g_lds_addr(lds_base));
  sbase = g_uniform(sbase);  // uniform by construction; keep it in SGPRs for the asm
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(sbase)
      : "memory");
}

// LDS position of copy slot i of this thread's wave within a stage:
// i * GCT + 64 * (wave within the copying threads), in 16-byte chunks.
__device__ __forceinline__ uint16_t *g_slot_dst(uint16_t *stage, int i) {
  const int w = ((int)threadIdx.x % GCT) >> 6;
  return stage + (i * GCT + w * 64) * 8;
}

// The same position as an LDS byte address in a scalar register (the M0
// value of the copy), computed from the stage's address and the wave index
// without a per-lane pointer.
__device__ __forceinline__ uint32_t g_slot_m0(const uint16_t *stage, int i) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(g_lds_addr(stage));
  const uint32_t w = __builtin_amdgcn_readfirstlane(((int)threadIdx.x % GCT) >> 6);
  return base + (uint32_t)(i * GCT + w * 64) * 16;
}

// Direct copy with the LDS destination given as a scalar byte address.
__device__ __forceinline__ void g_copy16_m0(const uint16_t *sbase, uint32_t voff, uint32_t m0) {
  sbase = g_uniform(sbase);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(sbase)
      : "memory");
}

// Copy K tile `kt` of one operand into its stage.
template <int NC>
__device__ __forceinline__ void g_copy_operand(const GOperand<NC> &o, int kt, uint16_t *dst) {
  const uint16_t *src = o.base + kt * GBK;
#pragma unroll
  for (int i = 0; i < NC; ++i) g_copy16_m0(src, o.off[i], g_slot_m0(dst, i));
}

// An operand whose K range is split into NS segments, each with its own
// base and row stride (a product over a concatenated K with one rounding).
// Each slot keeps its byte offset in every segment; a copy takes the scalar
// branch of its segment, so every copy site sees constant indices.
constexpr int GMAXSEG = 5;
template <int NC, int NS>
struct GSegOperand {
  const uint16_t *base[NS];  // row 0 of the tile region, K column 0
  int kend[NS];              // K tiles up to the end of each segment
  uint32_t off[NS][NC];
  int kbeg;                  // K tile where segment 0 starts (0, or -k0 to copy from k0 on)
};

template <int S, int NC, int NS, class RowOf>
__device__ __forceinline__ void g_seg_set(GSegOperand<NC, NS> &o, const uint16_t *base,
                                          int64_t ld, int kend, RowOf row_of) {
  o.base[S] = g_uniform(base);
  o.kend[S] = __builtin_amdgcn_readfirstlane(kend);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int r = g_load_row(i);
    const int c = (lane_id() % GCPR) ^ g_swz(r);
    o.off[S][i] = (uint32_t)((int64_t)row_of(r) * ld * 2 + c * 16);
  }
}

template <int S, int NC, int NS>
__device__ __forceinline__ void g_copy_seg(const GSegOperand<NC, NS> &o, int kt, uint16_t *dst) {
  if constexpr (S + 1 < NS) {
    if (kt >= o.kend[S]) {
      g_copy_seg<S + 1>(o, kt, dst);
      return;
    }
  }
  const uint16_t *src = o.base[S] + (kt - (S ? o.kend[S ? S - 1 : 0] : o.kbeg)) * GBK;
#pragma unroll
  for (int i = 0; i < NC; ++i) g_copy16_m0(src, o.off[S][i], g_slot_m0(dst, i));
}

template <int NC, int NS>
__device__ __forceinline__ void g_copy_operand(const GSegOperand<NC, NS> &o, int kt,
                                               uint16_t *dst) {
  g_copy_seg<0>(o, kt, dst);
}

// The copy sources of one block tile: both operands (every thread copies
// both), or in the ping-pong loop the operand of this thread's group (the
// other one is never read).
template <class OA, class OB>
struct GOps {
  OA a;
  OB b;
};

template <class RowA, class RowB>
__device__ __forceinline__ GOps<GOperand<GCA>, GOperand<GCB>> g_operands(
    const uint16_t *a, int64_t lda, RowA row_a, const uint16_t *b, int64_t ldb, RowB row_b) {
  GOps<GOperand<GCA>, GOperand<GCB>> o;
  if (!GPP || g_group1()) o.a = g_operand<GCA>(a, lda, row_a);
  if (!GPP || !g_group1()) o.b = g_operand<GCB>(b, ldb, row_b);
  return o;
}

typedef const __attribute__((address_space(3))) bf16x8 *lds_frag_ptr;

// LDS address of a stage as an opaque wave-uniform value: every fragment read
// of the stage is then that base plus a per-lane part plus an immediate
// (stage bases beyond 64 KB would otherwise not fold into the 16-bit DS
// offset and each read would hold its own address register).
__device__ __forceinline__ lds_frag_ptr g_stage_ptr(const uint16_t *p) {
  uint32_t a = g_lds_addr(p);
  asm volatile("" : "+s"(a));
  return (lds_frag_ptr)(uintptr_t)a;
}

__device__ __forceinline__ void g_read_frags(lds_frag_ptr A, lds_frag_ptr B, int kk,
                                             bf16x8 (&a)[GTM], bf16x8 (&b)[GTN]) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int wm = w / GWN, wn = w % GWN;
  const int lr = lane & 31, c = kk * 2 + (lane >> 5);  // logical chunk of this lane's 8 k
#pragma unroll
  for (int i = 0; i < GTM; ++i) {
    const int r = wm * GWTM + i * 32 + lr;
    a[i] = A[r * GCPR + (c ^ g_swz(r))];
  }
#pragma unroll
  for (int j = 0; j < GTN; ++j) {
    const int r = wn * GWTN + j * 32 + lr;
    b[j] = B[r * GCPR + (c ^ g_swz(r))];
  }
}

__device__ __forceinline__ void g_mma(const bf16x8 (&a)[GTM], const bf16x8 (&b)[GTN], GAcc &acc) {
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int j = 0; j < GTN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// MFMAs over one stage; the fragments of k-step kk + 1 are read from LDS
// while the MFMAs of k-step kk run.
__device__ __forceinline__ void g_mma_stage(const uint16_t *As, const uint16_t *Bs, GAcc &acc) {
  const lds_frag_ptr A = g_stage_ptr(As), B = g_stage_ptr(Bs);
  constexpr int NK = GBK / 16;
  bf16x8 a[2][GTM], b[2][GTN];
  g_read_frags(A, B, 0, a[0], b[0]);
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if (kk + 1 < NK) g_read_frags(A, B, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    g_mma(a[kk & 1], b[kk & 1], acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4] = 7, lgkmcnt[11:8] = 15, vmcnt[5:4] at [15:14]).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x70 | 0xF00)

// s_waitcnt vmcnt(PER_TILE * min(tiles, 3)): at most `tiles` later K tiles'
// copies of this thread outstanding (an immediate per case).
template <int PER_TILE>
__device__ __forceinline__ void g_wait_tiles(int tiles) {
  if (tiles >= 3) MOE_WAIT_VMCNT(3 * PER_TILE);
  else if (tiles == 2) MOE_WAIT_VMCNT(2 * PER_TILE);
  else if (tiles == 1) MOE_WAIT_VMCNT(PER_TILE);
  else MOE_WAIT_VMCNT(0);
}

// ---- two-stage ring (MOE_GEMM_CFG 1)
template <int S, class Ops>
__device__ __forceinline__ void g_ring_step(const Ops &o, int kt, int ktiles, GAcc &acc,
                                            const GemmLds &L) {
  if (kt >= ktiles) return;
  MOE_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  constexpr int NX = (S + 1) % GNST;
  if (kt + 1 < ktiles) {
    g_copy_operand(o.a, kt + 1, L.A[NX]);
    g_copy_operand(o.b, kt + 1, L.B[NX]);
  }
  __builtin_amdgcn_sched_barrier(0);
  g_mma_stage(L.A[S], L.B[S], acc);
}

// ---- ping-pong (MOE_GEMM_CFG 2)
//
// Phases 2s and 2s + 1 belong to K tile s.  Phase 2s: group 0 runs tile s's
// MFMAs; group 1 reads its fragments of tile s and copies A of tile s + 4.
// Phase 2s + 1: group 1 runs tile s's MFMAs; group 0 reads its fragments of
// tile s + 1 and copies B of tile s + 4.  (Fragment reads go first: the
// copies' issue then no longer delays them; measured 0.4-3% faster.)  Every phase ends in a barrier
// (reads of the phase are waited for before it: lgkmcnt).  Tile s is read in
// phases 2s - 1 and 2s, so it must have landed at the barrier closing phase
// 2s - 2 (each thread first waits for its own copies of it: vmcnt), and its
// stage is refilled (with tile s + 5) from phase 2s + 2 on.
constexpr int GPP_AHEAD = GNST - 1;

__device__ __forceinline__ void g_pp_mma(const bf16x8 (&a)[2][GTM], const bf16x8 (&b)[2][GTN],
                                         GAcc &acc) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) g_mma(a[kk], b[kk], acc);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void g_pp_frags(const uint16_t *As, const uint16_t *Bs,
                                           bf16x8 (&a)[2][GTM], bf16x8 (&b)[2][GTN]) {
  const lds_frag_ptr A = g_stage_ptr(As), B = g_stage_ptr(Bs);
  g_read_frags(A, B, 0, a[0], b[0]);
  g_read_frags(A, B, 1, a[1], b[1]);
}

__device__ __forceinline__ void g_pp_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this phase's LDS reads are done
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// One K tile s (phases 2s, 2s + 1) as group 0 sees it ...
template <int S, class Ops>
__device__ __forceinline__ void g_pp_tile_g0(const Ops &o, int s, int ktiles, GAcc &acc,
                                             const GemmLds &L, bf16x8 (&a)[2][GTM],
                                             bf16x8 (&b)[2][GTN]) {
  if (s >= ktiles) return;
  g_pp_mma(a, b, acc);
  // tile s + 1 lands before phase 2s + 1; B is copied up to tile s + 3
  g_wait_tiles<GCB>(min(GPP_AHEAD - 2, ktiles - 2 - s));
  g_pp_sync();
  if (s + 1 < ktiles) g_pp_frags(L.A[(S + 1) % GNST], L.B[(S + 1) % GNST], a, b);
  if (s + GPP_AHEAD < ktiles) g_copy_operand(o.b, s + GPP_AHEAD, L.B[(S + GPP_AHEAD) % GNST]);
  // nothing is shared after the last phase (a later call starts with a barrier)
  if (s + 1 < ktiles) g_pp_sync();
}

// ... and as group 1 sees it.
template <int S, class Ops>
__device__ __forceinline__ void g_pp_tile_g1(const Ops &o, int s, int ktiles, GAcc &acc,
                                             const GemmLds &L, bf16x8 (&a)[2][GTM],
                                             bf16x8 (&b)[2][GTN]) {
  if (s >= ktiles) return;
  g_pp_frags(L.A[S], L.B[S], a, b);
  if (s + GPP_AHEAD < ktiles) g_copy_operand(o.a, s + GPP_AHEAD, L.A[(S + GPP_AHEAD) % GNST]);
  // tile s + 1 lands before phase 2s + 1; A is copied up to tile s + 4
  g_wait_tiles<GCA>(min(GPP_AHEAD - 1, ktiles - 2 - s));
  g_pp_sync();
  g_pp_mma(a, b, acc);
  if (s + 1 < ktiles) g_pp_sync();
}

// The main loop in two parts.  gemm_mainloop_issue issues the copies of the
// first K tiles (everything before the loop's first wait); gemm_mainloop_rest
// runs the rest.  A block that runs several tiles issues the first copies of
// its next tile before the epilogue of the current one, so their latency
// hides behind it; stage GNST - 1 is not written until the rest's first
// barriers (the epilogue's staging area meanwhile).  Other memory operations issued between
// the two parts only make the rest's vmcnt waits wait longer: copies
// complete in issue order, so "at most n outstanding" still implies that the
// older copies landed.
template <class Ops>
__device__ __forceinline__ void gemm_mainloop_issue(const Ops &o, int ktiles, const GemmLds &L) {
  if (ktiles <= 0) return;
  if constexpr (!GPP) {
    g_copy_operand(o.a, 0, L.A[0]);
    g_copy_operand(o.b, 0, L.B[0]);
  } else if (g_group1()) {
    // A of tiles 0..3
#pragma unroll
    for (int p = 0; p < GPP_AHEAD; ++p)
      if (p < ktiles) g_copy_operand(o.a, p, L.A[p]);
  } else {
    // B of tiles 0..2 (tile 3 follows the first barrier)
#pragma unroll
    for (int p = 0; p < GPP_AHEAD - 1; ++p)
      if (p < ktiles) g_copy_operand(o.b, p, L.B[p]);
  }
}

template <class Ops>
__device__ __forceinline__ void gemm_mainloop_rest(const Ops &o, int ktiles, GAcc &acc,
                                                   const GemmLds &L) {
  if (ktiles <= 0) return;
  if constexpr (!GPP) {
    for (int kt = 0; kt < ktiles; kt += 2) {
      g_ring_step<0>(o, kt, ktiles, acc, L);
      g_ring_step<1>(o, kt + 1, ktiles, acc, L);
    }
  } else {
    // The two groups run separate loops with the same sequence of barriers.
    bf16x8 a[2][GTM], b[2][GTN];
    if (g_group1()) {
      // tile 0 landed; phase -1 idle
      g_wait_tiles<GCA>(min(GPP_AHEAD - 1, ktiles - 1));
      g_pp_sync();
      g_pp_sync();
      for (int s = 0; s < ktiles; s += GNST) {
        g_pp_tile_g1<0>(o, s, ktiles, acc, L, a, b);
        g_pp_tile_g1<1>(o, s + 1, ktiles, acc, L, a, b);
        g_pp_tile_g1<2>(o, s + 2, ktiles, acc, L, a, b);
        g_pp_tile_g1<3>(o, s + 3, ktiles, acc, L, a, b);
        g_pp_tile_g1<4>(o, s + 4, ktiles, acc, L, a, b);
      }
    } else {
      // tile 0 landed; phase -1: the fragments of tile 0 and B of tile 3
      g_wait_tiles<GCB>(min(GPP_AHEAD - 2, ktiles - 1));
      g_pp_sync();
      g_pp_frags(L.A[0], L.B[0], a, b);
      if (GPP_AHEAD - 1 < ktiles) g_copy_operand(o.b, GPP_AHEAD - 1, L.B[GPP_AHEAD - 1]);
      g_pp_sync();
      for (int s = 0; s < ktiles; s += GNST) {
        g_pp_tile_g0<0>(o, s, ktiles, acc, L, a, b);
        g_pp_tile_g0<1>(o, s + 1, ktiles, acc, L, a, b);
        g_pp_tile_g0<2>(o, s + 2, ktiles, acc, L, a, b);
        g_pp_tile_g0<3>(o, s + 3, ktiles, acc, L, a, b);
        g_pp_tile_g0<4>(o, s + 4, ktiles, acc, L, a, b);
      }
    }
  }
}

// Accumulate ktiles K tiles (GBK wide) of the two operands.
template <class Ops>
__device__ __forceinline__ void gemm_mainloop(const Ops &o, int ktiles, GAcc &acc,
                                              const GemmLds &L) {
  __builtin_amdgcn_s_barrier();  // the ring may still be read from a previous call
  __builtin_amdgcn_sched_barrier(0);
  gemm_mainloop_issue(o, ktiles, L);
  gemm_mainloop_rest(o, ktiles, acc, L);
}

__device__ __forceinline__ void gemm_zero(GAcc &acc) {
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int j = 0; j < GTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
}

// Position of accumulator element v of MFMA tile (i, j) in the block tile.
__device__ __forceinline__ int g_acc_row(int i, int v) {
  const int lane = lane_id(), wm = (int)(threadIdx.x >> 6) / GWN;
  return wm * GWTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int g_acc_col(int j) {
  const int lane = lane_id(), wn = (int)(threadIdx.x >> 6) % GWN;
  return wn * GWTN + j * 32 + (lane & 31);
}

// ---- epilogue stores through LDS
//
// The MFMA layout gives a lane one column of 4-row groups, so storing the
// accumulators directly takes one 2-byte store per element.  g_wave_store
// instead writes the wave's bf16 tile into its own LDS region and stores it
// back by 16-byte row chunks (8 full rows per instruction for 64 columns).
// Inside every group of 4 lanes (4 neighbouring columns) a 4 x 4 transpose of
// the lanes' 4-row groups (two DPP swaps) first gives each lane 4 consecutive
// columns of one row: one 8-byte LDS write.  For 64-column tiles the 16-byte
// chunk index is XORed with bit 1 of the row, so the 8 rows of one write
// instruction fall on distinct banks.  The global stores are non-temporal:
// the output streams past L2 instead of evicting operand panels that the
// next tiles still read (measured: 1-3% faster GEMMs).
//
// The regions (8 waves x 128 rows x 32*NJ columns, at most 128 KB) lie in the
// operand ring.  In the ping-pong loop every LDS read of the ring precedes the
// loop's last barrier, which every wave has passed on return, so no barrier is
// needed here; the two-stage loop gets one.
constexpr int GSTAGE = GNT / 64 * GWTM * GWTN;  // elements of the largest regions
static_assert(GSTAGE <= GNST * (GSA + GSB), "store regions inside the ring");

template <int NJ>
__device__ __forceinline__ int g_stage_chunk(int row, int c) {
  return NJ == 2 ? c ^ (((row >> 1) & 1) << 2) : c;
}

// 4 x 4 transpose inside each group of 4 lanes (4 neighbouring columns): in,
// p0 = rows 0, 1 and p1 = rows 2, 3 of one 4-row group of this lane's column
// (bf16 pairs); out, (o0, o1) = columns col4 .. col4 + 3 of row (lane & 3) of
// the group, col4 = (lane & 31) & ~3.
__device__ __forceinline__ void g_tr4x4(uint32_t p0, uint32_t p1, uint32_t &o0, uint32_t &o1) {
  const int lane = lane_id();
  const bool b1 = lane & 2, b0 = lane & 1;
  // with lane ^ 2: keep rows 2*b1, 2*b1 + 1 of both columns
  const uint32_t r1 =
      (uint32_t)__builtin_amdgcn_mov_dpp((int)(b1 ? p0 : p1), 0x4E, 0xF, 0xF, false);
  const uint32_t keep = b1 ? p1 : p0;
  const uint32_t x = b1 ? r1 : keep;  // column col4 + b0
  const uint32_t y = b1 ? keep : r1;  // column col4 + 2 + b0
  // with lane ^ 1: keep row 2*b1 + b0 of all four columns
  const uint32_t s = b0 ? ((x & 0xffffu) | (y << 16)) : ((x >> 16) | (y & 0xffff0000u));
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s, 0xB1, 0xF, 0xF, false);
  if (b0) {
    o0 = (r2 & 0xffffu) | (x & 0xffff0000u);
    o1 = (r2 >> 16) | (y & 0xffff0000u);
  } else {
    o0 = (x & 0xffffu) | (r2 << 16);
    o1 = (y & 0xffffu) | (r2 & 0xffff0000u);
  }
}

// pair(i, j, k): bf16 values of accumulator elements 2k (low half) and
// 2k + 1 (high half) of MFMA tile (i, j) of this wave; row_ptr(r): output row
// of wave-tile row r at the wave's first column (nullptr: row not stored),
// 16-byte aligned; ncols: valid columns from there (a multiple of 8).  Every
// lane of the wave must call it.  Row groups I0 .. I0 + NI - 1 only, staged
// in a region of NI * 32 rows per wave.
template <int NJ, int I0 = 0, int NI = GTM, class Pair, class RowPtr>
__device__ __forceinline__ void g_wave_store_pairs(uint16_t *ring, Pair pair, RowPtr row_ptr,
                                                   int ncols) {
  static_assert(NJ == 1 || NJ == 2, "32 or 64 columns per wave");
  static_assert(I0 >= 0 && NI >= 1 && I0 + NI <= GTM, "row groups of the wave tile");
  constexpr int W = NJ * 32, CH = W / 8, ROWS = NI * 32;
  if constexpr (!GPP) __syncthreads();
  const int lane = lane_id();
  uint16_t *st = ring + (threadIdx.x >> 6) * (ROWS * W);
  const int col4 = (lane & 31) & ~3;
#pragma unroll
  for (int i = I0; i < I0 + NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // rows 0,1 and 2,3 of this lane's column
        uint32_t o0, o1;
        g_tr4x4(pair(i, j, 2 * q), pair(i, j, 2 * q + 1), o0, o1);
        const int row = (i - I0) * 32 + 8 * q + 4 * (lane >> 5) + (lane & 3);
        const int col = j * 32 + col4;
        uint32_t *dst = reinterpret_cast<uint32_t *>(
            st + row * W + g_stage_chunk<NJ>(row, col >> 3) * 8 + (col & 7));
        dst[0] = o0;
        dst[1] = o1;
      }
#pragma unroll
  for (int it = 0; it < ROWS * CH / 64; ++it) {
    const int q = it * 64 + lane, row = q / CH, c = q % CH;
    const u32x4 v =
        *reinterpret_cast<const u32x4 *>(st + row * W + g_stage_chunk<NJ>(row, c) * 8);
    uint16_t *p = row_ptr(I0 * 32 + row);
    if (p && c * 8 < ncols) __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p + c * 8));
  }
}

// val(i, j, v): fp32 value of accumulator element v of MFMA tile (i, j),
// rounded to bf16 here.
template <int NJ, int I0 = 0, int NI = GTM, class Val, class RowPtr>
__device__ __forceinline__ void g_wave_store(uint16_t *ring, Val val, RowPtr row_ptr, int ncols) {
  g_wave_store_pairs<NJ, I0, NI>(
      ring, [&](int i, int j, int k) { return pack_bf16x2(val(i, j, 2 * k), val(i, j, 2 * k + 1)); },
      row_ptr, ncols);
}

// The same through one ring stage (GSA + GSB elements: 4 KB per wave), in
// passes of as many row groups as fit.
constexpr int GSTAGE_ELEMS = GSA + GSB;
template <int NJ, class Val, class RowPtr>
__device__ __forceinline__ void g_wave_store_staged(uint16_t *stage, Val val, RowPtr row_ptr,
                                                    int ncols) {
  constexpr int NI = GSTAGE_ELEMS / (GNT / 64) / (32 * NJ * 32);  // row groups per pass
  static_assert(NI >= 1 && GTM % NI == 0, "passes of whole row groups");
  g_wave_store<NJ, 0, NI>(stage, val, row_ptr, ncols);
  if constexpr (NI < GTM) g_wave_store<NJ, NI % GTM, NI>(stage, val, row_ptr, ncols);
  if constexpr (2 * NI < GTM) {
    g_wave_store<NJ, (2 * NI) % GTM, NI>(stage, val, row_ptr, ncols);
    g_wave_store<NJ, (3 * NI) % GTM, NI>(stage, val, row_ptr, ncols);
  }
}

// Whether a bf16 output (base, row stride ld, columns n) takes 16-byte
// stores.
__device__ __forceinline__ bool g_vec_out(const void *base, int64_t ld, int n) {
  return (((uintptr_t)base & 15) | (ld & 7) | (n & 7)) == 0;
}

// SwiGLU tiles: in every wave's column range, MFMA column tiles alternate
// gate (even j) and up (odd j) weight rows of the same 32 intermediate
// columns, so a lane holds a = u.W_g in tile 2p and b = u.W_u in tile 2p + 1.
// B-tile row br -> (is_up, intermediate column offset within the block).
__device__ __forceinline__ void g_swiglu_brow(int br, bool &is_up, int &f_off) {
  const int wn = br / GWTN, j = (br % GWTN) / 32;
  is_up = j & 1;
  f_off = wn * (GWTN / 2) + (j >> 1) * 32 + (br & 31);
}
// Intermediate column offset of accumulator pair p of this lane.
__device__ __forceinline__ int g_swiglu_col(int p) {
  const int wn = (int)(threadIdx.x >> 6) % GWN;
  return wn * (GWTN / 2) + p * 32 + (lane_id() & 31);
}

// Tile order within a GEMM of tm x tn tiles: groups of 8 tile-rows, column
// by column inside a group (neighbouring tiles share A or B panels).
__device__ __forceinline__ void g_tile_coords(int logical, int tm, int tn, int &m, int &n) {
  constexpr int GM = 8;
  const int per_group = GM * tn;
  const int g = logical / per_group;
  const int first = g * GM;
  const int gs = min(tm - first, GM);
  const int r = logical - g * per_group;
  m = first + r % gs;
  n = r / gs;
}

}  // namespace moe
