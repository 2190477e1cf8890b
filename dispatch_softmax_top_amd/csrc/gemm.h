// gemm.h -- bf16 GEMM core for gfx950: C[m, n] = sum_k A[m, k] * B[n, k],
// fp32 accumulation in MFMA (v_mfma_f32_32x32x16_bf16).  Both operands are
// K-contiguous ("out x in" weights), so every global load, LDS store and
// LDS fragment read is 16 bytes per lane.
//
// Block tile 256 x 256 x 64, 512 threads = 8 waves in a 2 (M) x 4 (N) grid,
// each wave 128 x 64 = 4 x 2 MFMA tiles (128 fp32 accumulators per lane; two
// waves per SIMD so one can issue MFMAs while the other waits on LDS).
// LDS holds two stages of A and B (2 x 64 KB): the next K tile is fetched
// into registers while the current one feeds the MFMAs, then stored to the
// other stage; one barrier per K tile.  Rows of a stage are 128 bytes (8
// chunks of 16 B); chunk c of row r lives at c ^ (r & 7), so the 8 lanes
// served together by a ds_read_b128 / ds_write_b128 hit 8 distinct 16-byte
// bank groups.
//
// Thread t loads rows (t >> 3) + 64 i (i = 0..3) of each operand tile, chunk
// t & 7; callers hand the mainloop those 4 row pointers per operand.
#pragma once
#include "common.h"

namespace moe {

constexpr int GBM = 256, GBN = 256, GBK = 64, GNT = 512;
constexpr int GSTAGE = GBM * GBK;               // bf16 elements per operand stage
constexpr int G_LDS_BYTES = 4 * GSTAGE * 2;     // A0 A1 B0 B1 = 128 KB
constexpr int GROWS = GBM * 8 / GNT;            // rows per thread per operand (4)
constexpr int GTM = 4, GTN = 2;                 // MFMA tiles per wave

typedef f32x16 GAcc[GTM][GTN];

__device__ __forceinline__ void g_store_stage(uint16_t *stage, const u32x4 (&r)[GROWS]) {
  const int t = threadIdx.x;
  const int c = t & 7, r0 = t >> 3;
  u32x4 *s = reinterpret_cast<u32x4 *>(stage);
#pragma unroll
  for (int i = 0; i < GROWS; ++i) {
    const int row = r0 + 64 * i;
    s[row * 8 + (c ^ (row & 7))] = r[i];
  }
}

__device__ __forceinline__ void g_load_regs(const uint16_t *const (&p)[GROWS], int koff,
                                            u32x4 (&r)[GROWS]) {
#pragma unroll
  for (int i = 0; i < GROWS; ++i) r[i] = *reinterpret_cast<const u32x4 *>(p[i] + koff);
}

__device__ __forceinline__ void g_mma_stage(const uint16_t *As, const uint16_t *Bs, GAcc &acc) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int lr = lane & 31, lh = lane >> 5;
  const bf16x8 *A = reinterpret_cast<const bf16x8 *>(As);
  const bf16x8 *B = reinterpret_cast<const bf16x8 *>(Bs);
#pragma unroll
  for (int kk = 0; kk < GBK / 16; ++kk) {
    const int ch = (kk * 2 + lh) ^ (lr & 7);
    bf16x8 a[GTM], b[GTN];
#pragma unroll
    for (int i = 0; i < GTM; ++i) a[i] = A[(wm * 128 + i * 32 + lr) * 8 + ch];
#pragma unroll
    for (int j = 0; j < GTN; ++j) b[j] = B[(wn * 64 + j * 32 + lr) * 8 + ch];
#pragma unroll
    for (int i = 0; i < GTM; ++i)
#pragma unroll
      for (int j = 0; j < GTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Accumulate ktiles K tiles (64 wide) starting at the given row pointers.
// The stage in use is picked by offset, not by branch, so there is a single
// MFMA chain in the loop and the accumulators stay in place.
__device__ __forceinline__ void gemm_mainloop(const uint16_t *const (&ap)[GROWS],
                                              const uint16_t *const (&bp)[GROWS], int ktiles,
                                              GAcc &acc, uint16_t *lds) {
  const int c8 = (threadIdx.x & 7) * 8;
  u32x4 ra[GROWS], rb[GROWS];
  g_load_regs(ap, c8, ra);
  g_load_regs(bp, c8, rb);
  g_store_stage(lds, ra);
  g_store_stage(lds + 2 * GSTAGE, rb);
  __syncthreads();
  for (int kt = 0; kt + 1 < ktiles; ++kt) {
    const int cur = (kt & 1) * GSTAGE, nxt = GSTAGE - cur;
    g_load_regs(ap, (kt + 1) * GBK + c8, ra);
    g_load_regs(bp, (kt + 1) * GBK + c8, rb);
    g_mma_stage(lds + cur, lds + 2 * GSTAGE + cur, acc);
    g_store_stage(lds + nxt, ra);
    g_store_stage(lds + 2 * GSTAGE + nxt, rb);
    __syncthreads();
  }
  const int last = ((ktiles - 1) & 1) * GSTAGE;
  g_mma_stage(lds + last, lds + 2 * GSTAGE + last, acc);
  __syncthreads();
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
  const int lane = lane_id(), wm = (threadIdx.x >> 6) >> 2;
  return wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int g_acc_col(int j) {
  const int lane = lane_id(), wn = (threadIdx.x >> 6) & 3;
  return wn * 64 + j * 32 + (lane & 31);
}

// Row (within the block tile) that thread t loads in slot i.
__device__ __forceinline__ int g_load_row(int i) { return (int)(threadIdx.x >> 3) + 64 * i; }

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
