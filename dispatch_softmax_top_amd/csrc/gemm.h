// gemm.h -- bf16 GEMM core for gfx950: C[m, n] = sum_k A[m, k] * B[n, k],
// fp32 accumulation in MFMA (v_mfma_f32_32x32x16_bf16).  Both operands are
// K-contiguous ("out x in" weights), so every copy and every LDS fragment
// read is 16 bytes per lane.
//
// Block tile GBM x GBN over a GWM x GWN grid of waves, each wave 128 x 64 =
// 4 x 2 MFMA tiles (128 fp32 accumulators per lane, at most 256 registers,
// two waves per SIMD).  Two configurations:
//   MOE_GEMM_CFG 1 (default): 256 x 256 tile, 8 waves, K tiles of 64,
//                   2-stage ring (2 x 64 KB): one block per CU.
//   MOE_GEMM_CFG 2: 128 x 256 tile, 4 waves, K tiles of 32, 3-stage ring
//                   (3 x 24 KB): two blocks per CU, so one block's MFMAs
//                   can cover the other's barrier waits.  On MI355X it ran
//                   8-15% slower than configuration 1 on every GEMM of the
//                   4096-token share (half the operand reuse per tile costs
//                   more L2 traffic than the overlap wins back).
//
// Global -> LDS moves use the gfx950 direct path (global_load_lds_dwordx4:
// no register staging), issued GNST - 1 tiles ahead.  Per K tile: wait until
// this thread's copies of the tile have landed (vmcnt), barrier (then every
// wave's copies have landed and every wave is done reading the stage that
// is refilled next), issue the copy of tile + GNST - 1 into that stage, then
// run the MFMAs.  The loop is unrolled by the ring size so every stage
// address is static.  The copy engine writes each wave's 64 x 16 B
// contiguously, so lane l of copy slot i in wave w fetches the chunk that
// belongs at stage position GNT * i + 64 w + l.
//
// A stage row is GBK * 2 bytes = GCPR chunks of 16 B; chunk c of row r is
// stored at c ^ g_swz(r).  A fragment read has 16 consecutive lanes on 16
// consecutive rows at one logical chunk; g_swz makes both the 8 lanes of a
// 128-byte LDS phase and the 16 lanes of a 256-byte phase land on distinct
// 16-byte bank groups.
#pragma once
#include "common.h"

namespace moe {

#ifndef MOE_GEMM_CFG
#define MOE_GEMM_CFG 1
#endif
#if MOE_GEMM_CFG == 1
constexpr int GBM = 256, GBN = 256, GBK = 64, GWM = 2, GWN = 4, GNST = 2;
#else
constexpr int GBM = 128, GBN = 256, GBK = 32, GWM = 1, GWN = 4, GNST = 3;
#endif
constexpr int GNT = 64 * GWM * GWN;                 // threads per block
constexpr int GWTM = GBM / GWM, GWTN = GBN / GWN;   // wave tile (128 x 64)
constexpr int GTM = GWTM / 32, GTN = GWTN / 32;     // MFMA tiles per wave
constexpr int GCPR = GBK / 8;                       // 16-byte chunks per stage row
constexpr int GSA = GBM * GBK, GSB = GBN * GBK;     // elements per operand stage
constexpr int GCA = GBM * GCPR / GNT, GCB = GBN * GCPR / GNT;  // copies per thread per stage
constexpr int GMINWAVES = 2;                        // waves per SIMD the kernels are built for
static_assert(GWTM == 128 && GWTN == 64, "wave tile 128 x 64");
static_assert(GNST * (GSA + GSB) * 2 <= (MOE_GEMM_CFG == 1 ? 131072 : 81920), "LDS ring");

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
// immediate.  For 8 chunks per row it is a permutation of 0..7 over any 8
// consecutive rows and over the even (and the odd) rows of any 16.
__device__ __forceinline__ int g_swz(int row) {
  return GCPR == 4 ? (((row >> 1) ^ (row >> 3)) & 3) : ((row & 6) | ((row ^ (row >> 3)) & 1));
}

// Tile row whose chunk thread t copies in copy slot i (either operand).
__device__ __forceinline__ int g_load_row(int i) { return (i * GNT + (int)threadIdx.x) / GCPR; }

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

// One 16-byte-per-lane copy global -> LDS: the wave's 64 chunks land at
// lds_base + 16 * lane.  Written as inline asm so that the compiler does not
// guard later LDS reads with waits of its own: completion is tracked
// explicitly (vmcnt) and published to the block with a barrier.  M0 (the
// LDS destination) is restored afterwards.
__device__ __forceinline__ void g_copy16(const uint16_t *sbase, uint32_t voff,
                                         const uint16_t *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_base);
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

// Copy K tile `kt` of both operands into one stage.
__device__ __forceinline__ void g_copy_tile(const GOperand<GCA> &a, const GOperand<GCB> &b,
                                            int kt, uint16_t *As, uint16_t *Bs) {
  const int w = threadIdx.x >> 6;
  const uint16_t *ab = a.base + kt * GBK, *bb = b.base + kt * GBK;
#pragma unroll
  for (int i = 0; i < GCA; ++i) g_copy16(ab, a.off[i], As + (i * GNT + w * 64) * 8);
#pragma unroll
  for (int i = 0; i < GCB; ++i) g_copy16(bb, b.off[i], Bs + (i * GNT + w * 64) * 8);
}

typedef const __attribute__((address_space(3))) bf16x8 *lds_frag_ptr;

// LDS address of a stage as an opaque wave-uniform value: every fragment read
// of the stage is then that base plus a per-lane part plus an immediate
// (stage bases beyond 64 KB would otherwise not fold into the 16-bit DS
// offset and each read would hold its own address register).
__device__ __forceinline__ lds_frag_ptr g_stage_ptr(const uint16_t *p) {
  uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
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

template <int S>
__device__ __forceinline__ void g_ring_step(const GOperand<GCA> &ap, const GOperand<GCB> &bp,
                                            int kt, int ktiles, GAcc &acc, const GemmLds &L) {
  if (kt >= ktiles) return;
  // copies issued after those of tile kt: min(GNST - 2, ktiles - 1 - kt) tiles
  constexpr int PER_TILE = GCA + GCB;
  if constexpr (GNST >= 3) {
    if (kt + 1 < ktiles) MOE_WAIT_VMCNT(PER_TILE);
    else MOE_WAIT_VMCNT(0);
  } else {
    MOE_WAIT_VMCNT(0);
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  constexpr int NX = (S + GNST - 1) % GNST;  // stage of tile kt + GNST - 1
  if (kt + GNST - 1 < ktiles) g_copy_tile(ap, bp, kt + GNST - 1, L.A[NX], L.B[NX]);
  __builtin_amdgcn_sched_barrier(0);
  g_mma_stage(L.A[S], L.B[S], acc);
}

// Accumulate ktiles K tiles (GBK wide) of the two operands.
__device__ __forceinline__ void gemm_mainloop(const GOperand<GCA> &ap, const GOperand<GCB> &bp,
                                              int ktiles, GAcc &acc, const GemmLds &L) {
  __builtin_amdgcn_s_barrier();  // the ring may still be read from a previous call
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < GNST - 1; ++p)
    if (p < ktiles) g_copy_tile(ap, bp, p, L.A[p], L.B[p]);
  for (int kt = 0; kt < ktiles; kt += GNST) {
    g_ring_step<0>(ap, bp, kt, ktiles, acc, L);
    g_ring_step<1>(ap, bp, kt + 1, ktiles, acc, L);
    if constexpr (GNST >= 3) g_ring_step<2 % GNST>(ap, bp, kt + 2, ktiles, acc, L);
  }
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
