// gemm.hip -- the dense contractions of the path, all on the bf16 MFMA core
// of gemm.h:
//   gemm_latent_down    z = x . W_ld                  (model width -> latent)
//   gemm_shared_swiglu  h_s = silu(x.W_sg,s) * (x.W_su,s) for each shared expert
//   gemm_up_shared      out = ylat . W_lu + sum_s h_s . W_sd,s (one K-concatenated
//                       product, one rounding)
//   gemm_expert_swiglu  h = silu(u.W_g,j) * (u.W_u,j) over every bank group
//   gemm_expert_down    y = h . W_d,j, rows scattered to their receive position
//
// SwiGLU tiles: a block owns 128 intermediate columns f0 .. f0+127 and loads
// their 128 gate and 128 up weight rows, interleaved per 32-row MFMA tile
// (g_swiglu_brow), so one lane holds a = u.W_g and b = u.W_u of the same
// (row, f) and the epilogue writes bf16(silu(a) * b) directly.
#include <algorithm>

#include "gemm.h"
#include "kernels.h"

namespace moe {

constexpr int MAXSEG = GMAXSEG;

// ---------------------------------------------------------------------------
// Tail split.  total block tiles on ncu CUs (one resident block per CU) run
// in ceil(total / ncu) rounds, the last holding only r = total % ncu tiles.
// When r <= ncu / 2, each of those r tiles is cut along K into S parts,
// S = min(ncu / r, GSPLIT_MAX), run as r * S blocks of the last round; the
// parts write fp32 partial tiles and a second kernel sums each tile's parts
// in part order and runs the tile's epilogue.
// ---------------------------------------------------------------------------

constexpr int GSPLIT_MAX = 8;      // parts per split tile at most
constexpr int GSPLIT_MIN_KT = 16;  // K tiles per part at least
constexpr int GSPLIT_UNITS = 256;  // partial tiles a split buffer holds

// Work queue of a persistent grouped kernel.  Without one, block k runs
// units k, k + grid, k + 2 grid, ... .  With one, the units are dealt per
// XCD (block k sits in XCD k % 8, whose units are 8 l + k % 8): block k runs
// k, k + grid and k + 2 grid, and then one unit per ticket it draws from its
// XCD's counter, so that blocks that started late (the CUs busy with another
// stream's kernel) or run slow tiles take fewer units.  A ticket drawn
// during the block's tile n names its tile n + 3: unit 8 (3 grid / 8 +
// ticket) + k % 8.  Thread 0 draws it before the tile's main loop and
// stores it after; the other waves load it after the next tile's main loop.
// By then the store is complete (thread 0's wave waited for copies issued
// after it, in issue order) and a barrier lies between, and the value is
// used one tile later still, so neither the atomic nor the load is waited
// for.  A block's units only grow, so the first one past the end ends it.
struct GQueue {
  int32_t *count;  // [8] tickets drawn per XCD, zero at launch; NULL: no queue
  int32_t *slot;   // [2][grid] tickets passed from thread 0 to its block
};
constexpr int GQ_MAX_GRID = 1024;                       // blocks a queue serves
constexpr int64_t GQ_BYTES = 256 + 2 * GQ_MAX_GRID * 4;  // two counter sets, slots

struct GSplit {
  float *part;    // partial tiles (see g_part_store); NULL: no split
  int ncu;        // CUs of the device
  int max_units;  // partial tiles the buffer holds
  int max_parts;  // parts per split tile at most (K tiles / GSPLIT_MIN_KT)
  GQueue q;       // persistent grouped kernels only
};

// A persistent block's unit sequence (GQueue).
struct GSeq {
  int next;  // unit of the block's next tile (wave-uniform)
  int tk;    // ticket drawn during the current tile (thread 0)
  int n;     // tiles begun before the current one
};

__device__ __forceinline__ GSeq gseq_start() {
  return GSeq{(int)(blockIdx.x + gridDim.x), 0, 0};
}

// Before the current tile's main loop.
__device__ __forceinline__ void gseq_draw(const GQueue &q, GSeq &s) {
  if (q.count && threadIdx.x == 0) s.tk = atomicAdd(q.count + blockIdx.x % 8, 1);
}

// After the main loop: hand the ticket to the block.
__device__ __forceinline__ void gseq_post(const GQueue &q, const GSeq &s) {
  if (q.count && threadIdx.x == 0)
    __hip_atomic_store(q.slot + (s.n & 1) * gridDim.x + blockIdx.x, s.tk, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// After the tile's closing barrier, the next tile's unit (s.next, read
// before the barrier) taken: fetch the unit of the tile after it.
__device__ __forceinline__ void gseq_fetch(const GQueue &q, GSeq &s) {
  if (!q.count || s.n == 0) {
    s.next = (int)blockIdx.x + (s.n + 2) * (int)gridDim.x;
  } else {
    asm volatile("" ::: "memory");  // the load stays behind the barrier before this call
    const int tk = __hip_atomic_load(q.slot + ((s.n - 1) & 1) * gridDim.x + blockIdx.x,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s.next = __builtin_amdgcn_readfirstlane(8 * (3 * (int)(gridDim.x / 8) + tk) +
                                            (int)(blockIdx.x % 8));
  }
  ++s.n;
}

struct GUnit {
  int tile;    // logical tile
  int part;    // K part of a split tile (0 if whole)
  int nparts;  // 1 if whole
  int tail;    // index among the split tiles
};

__device__ __forceinline__ int g_split_parts(const GSplit &sp, int total) {
  if (!sp.part) return 1;
  const int r = total % sp.ncu;
  if (r == 0 || 2 * r > sp.ncu) return 1;
  return max(1, min(min(sp.ncu / r, sp.max_parts), sp.max_units / r));
}

// Block b of a launch: whole tiles first (each XCD a contiguous range of
// them, or with spread, groups of 32 dealt round the XCDs: xcd_spread), then
// the parts of the split tiles.  False past the last unit.
__device__ __forceinline__ bool g_unit(const GSplit &sp, int total, int b, GUnit &u,
                                       bool spread = false) {
  const int S = g_split_parts(sp, total);
  const int whole = S > 1 ? total - total % sp.ncu : total;
  u.part = 0;
  u.nparts = 1;
  u.tail = 0;
  if (b < whole) {
    u.tile = __builtin_amdgcn_readfirstlane(spread ? xcd_spread<32>(b, whole) : xcd_remap(b, whole));
    return true;
  }
  const int t = b - whole;
  if (S == 1 || t >= (total - whole) * S) return false;
  u.tail = __builtin_amdgcn_readfirstlane(t / S);
  u.tile = whole + u.tail;
  u.part = __builtin_amdgcn_readfirstlane(t - u.tail * S);
  u.nparts = __builtin_amdgcn_readfirstlane(S);
  return true;
}

// K tiles [k0, k1) of the unit's part of kt K tiles (wave-uniform values,
// kept in scalar registers).
__device__ __forceinline__ void g_part_range(int kt, const GUnit &u, int &k0, int &k1) {
  k0 = __builtin_amdgcn_readfirstlane((int)((int64_t)kt * u.part / u.nparts));
  k1 = __builtin_amdgcn_readfirstlane((int)((int64_t)kt * (u.part + 1) / u.nparts));
}

// Partial tile `unit`: chunk c (4 accumulators) of thread x at
// (unit * GACC_CHUNKS + c) * GNT + x, in 16-byte units.
constexpr int GACC_CHUNKS = GTM * GTN * 4;
constexpr int64_t GPART_BYTES = (int64_t)GACC_CHUNKS * GNT * 16;

__device__ __forceinline__ void g_part_store(float *part, int unit, const GAcc &acc) {
  f32x4 *p = reinterpret_cast<f32x4 *>(part) + (int64_t)unit * GACC_CHUNKS * GNT + threadIdx.x;
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int j = 0; j < GTN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
        __builtin_nontemporal_store(v, p + ((i * GTN + j) * 4 + q) * GNT);
      }
}

// acc[I][*] = sum of the S parts of split tile `tail` (MFMA row group I of
// every wave), added in part order; a part's loads are all issued first.
template <int I>
__device__ __forceinline__ void g_part_sum_rows(const float *part, int tail, int S, GAcc &acc) {
#pragma unroll
  for (int j = 0; j < GTN; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[I][j][v] = 0.f;
  // two parts' loads in flight at a time (a missing second part re-reads
  // the first and is not added)
  for (int k = 0; k < S; k += 2) {
    const f32x4 *p = reinterpret_cast<const f32x4 *>(part) +
                     (int64_t)(tail * S + k) * GACC_CHUNKS * GNT + threadIdx.x;
    const int64_t next = k + 1 < S ? (int64_t)GACC_CHUNKS * GNT : 0;
    f32x4 v[2][GTN * 4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < GTN * 4; ++c)
        v[h][c] = __builtin_nontemporal_load(p + h * next + (I * GTN * 4 + c) * GNT);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && k + 1 >= S) break;
#pragma unroll
      for (int j = 0; j < GTN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[I][j][4 * q + e] += v[h][j * 4 + q][e];
    }
  }
}

// Tail kernels run GTM blocks per split tile, one per MFMA row group.  The
// split tile of tail block b: false if there is none (no split, or fewer
// split tiles than tail blocks).
__device__ __forceinline__ bool g_tail_tile(const GSplit &sp, int total, int b, GUnit &u) {
  const int S = g_split_parts(sp, total);
  if (S == 1 || b >= total % sp.ncu) return false;
  u.tail = b;
  u.tile = total - total % sp.ncu + u.tail;
  u.part = 0;
  u.nparts = S;
  return true;
}

// Row group I of a tail tile: sum of parts, then store(acc) (which stores
// only row group I).
#define MOE_TAIL_ROWS(store_rows)                      \
  switch (blockIdx.x % GTM) {                          \
    case 0: store_rows(0); break;                      \
    case 1: store_rows(1); break;                      \
    case 2: store_rows(2); break;                      \
    default: store_rows(3); break;                     \
  }
static_assert(GTM == 4, "tail kernels: four MFMA row groups per wave");

struct DenseArgs {
  int M, N, nseg;
  const uint16_t *A[MAXSEG];
  int64_t lda[MAXSEG];
  const uint16_t *B[MAXSEG];
  int64_t ldb[MAXSEG];
  int ktiles[MAXSEG];
  uint16_t *C;
  int64_t ldc;
  // batched products (one K segment): nbatch products of the same shape,
  // product b at A + b*bsA, B + b*bsB, C + b*bsC
  int nbatch;
  int64_t bsA, bsB, bsC;
  GSplit sp;
};

// Product and tile of logical tile `tile` of a (possibly batched) product.
template <bool BATCHED>
__device__ __forceinline__ int dense_batch(const DenseArgs &g, int per, int &tile) {
  if constexpr (!BATCHED) return 0;
  const int b = tile / per;
  tile -= b * per;
  return b;
}

// ONLY >= 0: store MFMA row group ONLY alone.
// ONLY < 0 (the operand ring given): the whole tile through LDS
// (g_wave_store) when the output allows 16-byte stores.
template <int ONLY = -1>
__device__ __forceinline__ void dense_store(const DenseArgs &g, uint16_t *C, int mt, int nt,
                                            const GAcc &acc, uint16_t *ring = nullptr) {
  if (ONLY < 0 && g_vec_out(C, g.ldc, g.N)) {
    const int w = (int)(threadIdx.x >> 6);
    const int m0 = mt * GBM + (w / GWN) * GWTM, n0 = nt * GBN + (w % GWN) * GWTN;
    g_wave_store<GTN>(
        ring, [&](int i, int j, int v) { return acc[i][j][v]; },
        [&](int r) -> uint16_t * {
          return m0 + r < g.M ? C + (int64_t)(m0 + r) * g.ldc + n0 : nullptr;
        },
        g.N - n0);
    return;
  }
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int j = 0; j < GTN; ++j) {
      if (ONLY >= 0 && i != ONLY) continue;
      const int n = nt * GBN + g_acc_col(j);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mt * GBM + g_acc_row(i, v);
        if (m < g.M && n < g.N) C[(int64_t)m * g.ldc + n] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

// Segment S of the operand sources (compile-time indices throughout).
template <int S, int NS, class RowA, class RowB>
__device__ __forceinline__ void dense_segs(const DenseArgs &g, int mt, int nt, RowA row_a,
                                           RowB row_b, int &kend,
                                           GOps<GSegOperand<GCA, NS>, GSegOperand<GCB, NS>> &ops) {
  kend += g.ktiles[S];
  // in the ping-pong loop a group copies one operand only
  if (!GPP || g_group1())
    g_seg_set<S>(ops.a, g.A[S] + (int64_t)mt * GBM * g.lda[S], g.lda[S], kend, row_a);
  if (!GPP || !g_group1())
    g_seg_set<S>(ops.b, g.B[S] + (int64_t)nt * GBN * g.ldb[S], g.ldb[S], kend, row_b);
  if constexpr (S + 1 < NS) dense_segs<S + 1>(g, mt, nt, row_a, row_b, kend, ops);
}

// NS: number of K segments (one K range, one rounding).  BATCHED: nbatch
// products of one segment each.
template <int NS, bool BATCHED = false>
__device__ __forceinline__ void dense_body(const DenseArgs &g, const GemmLds &lds) {
  static_assert(!BATCHED || NS == 1, "batched products have one K segment");
  const int tm = (g.M + GBM - 1) / GBM, tn = (g.N + GBN - 1) / GBN;
  GUnit u;
  if (!g_unit(g.sp, tm * tn * (BATCHED ? g.nbatch : 1), blockIdx.x, u)) return;
  int tile = u.tile;
  const int b = dense_batch<BATCHED>(g, tm * tn, tile);
  int mt, nt;
  g_tile_coords(tile, tm, tn, mt, nt);
  const int mv = g.M - mt * GBM, nv = g.N - nt * GBN;  // valid rows / columns
  const auto row_a = [&](int r) { return min(r, mv - 1); };
  const auto row_b = [&](int r) { return min(r, nv - 1); };
  int kt = 0;
  for (int i = 0; i < NS; ++i) kt += g.ktiles[i];
  int k0, k1;
  g_part_range(kt, u, k0, k1);
  GAcc acc;
  gemm_zero(acc);
  if constexpr (NS == 1) {
    const auto ops = g_operands(
        g.A[0] + b * g.bsA + (int64_t)mt * GBM * g.lda[0] + k0 * GBK, g.lda[0], row_a,
        g.B[0] + b * g.bsB + (int64_t)nt * GBN * g.ldb[0] + k0 * GBK, g.ldb[0], row_b);
    gemm_mainloop(ops, k1 - k0, acc, lds);
  } else {
    GOps<GSegOperand<GCA, NS>, GSegOperand<GCB, NS>> ops;
    int kend = 0;
    dense_segs<0>(g, mt, nt, row_a, row_b, kend, ops);
    // copy K tiles k0 .. k1 - 1 of the concatenated range as tiles 0 .. k1 - k0 - 1
    ops.a.kbeg = ops.b.kbeg = -k0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      ops.a.kend[i] -= k0;
      ops.b.kend[i] -= k0;
    }
    gemm_mainloop(ops, k1 - k0, acc, lds);
  }
  if (u.nparts > 1) {
    g_part_store(g.sp.part, u.tail * u.nparts + u.part, acc);
    return;
  }
  dense_store(g, g.C + b * g.bsC, mt, nt, acc, lds.A[0]);
}

// Operand sources of dense tile (b, mt, nt) from K tile k0 on.
template <int NS>
struct DenseOps {
  typedef GOps<GSegOperand<GCA, NS>, GSegOperand<GCB, NS>> type;
};
template <>
struct DenseOps<1> {
  typedef GOps<GOperand<GCA>, GOperand<GCB>> type;
};

template <int NS>
__device__ __forceinline__ typename DenseOps<NS>::type dense_ops(const DenseArgs &g, int b, int mt,
                                                                 int nt, int k0) {
  const int mv = g.M - mt * GBM, nv = g.N - nt * GBN;  // valid rows / columns
  const auto row_a = [&](int r) { return min(r, mv - 1); };
  const auto row_b = [&](int r) { return min(r, nv - 1); };
  if constexpr (NS == 1) {
    return g_operands(g.A[0] + b * g.bsA + (int64_t)mt * GBM * g.lda[0] + k0 * GBK, g.lda[0],
                      row_a, g.B[0] + b * g.bsB + (int64_t)nt * GBN * g.ldb[0] + k0 * GBK,
                      g.ldb[0], row_b);
  } else {
    typename DenseOps<NS>::type ops;
    int kend = 0;
    dense_segs<0>(g, mt, nt, row_a, row_b, kend, ops);
    ops.a.kbeg = ops.b.kbeg = -k0;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      ops.a.kend[i] -= k0;
      ops.b.kend[i] -= k0;
    }
    return ops;
  }
}

// Whole-tile epilogue of a persistent dense block: 16-byte row stores staged
// through one ring stage, or (outputs without 16-byte alignment) direct stores.
__device__ __forceinline__ void dense_finish(const DenseArgs &g, uint16_t *C, int mt, int nt,
                                             const GAcc &acc, uint16_t *stage) {
  if (g_vec_out(C, g.ldc, g.N)) {
    const int w = (int)(threadIdx.x >> 6);
    const int m0 = mt * GBM + (w / GWN) * GWTM, n0 = nt * GBN + (w % GWN) * GWTN;
    g_wave_store_staged<GTN>(
        stage, [&](int i, int j, int v) { return acc[i][j][v]; },
        [&](int r) -> uint16_t * {
          return m0 + r < g.M ? C + (int64_t)(m0 + r) * g.ldc + n0 : nullptr;
        },
        g.N - n0);
    return;
  }
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int j = 0; j < GTN; ++j) {
      const int n = nt * GBN + g_acc_col(j);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mt * GBM + g_acc_row(i, v);
        if (m < g.M && n < g.N) C[(int64_t)m * g.ldc + n] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

// Persistent form of dense_body (see the grouped kernels): block b runs
// units b, b + gridDim.x, ...; only the tile's coordinates live across the
// main loop.
template <int NS, bool BATCHED = false>
__device__ __forceinline__ void dense_body_persistent(const DenseArgs &g, const GemmLds &lds) {
  static_assert(!BATCHED || NS == 1, "batched products have one K segment");
  const int tm = (g.M + GBM - 1) / GBM, tn = (g.N + GBN - 1) / GBN;
  const int total = tm * tn * (BATCHED ? g.nbatch : 1);
  int kt = 0;
  for (int i = 0; i < NS; ++i) kt += g.ktiles[i];
  int bid = blockIdx.x;
  GUnit u;
  if (!g_unit(g.sp, total, bid, u)) return;
  int tile = u.tile;
  int b = dense_batch<BATCHED>(g, tm * tn, tile);
  int mt, nt;
  g_tile_coords(tile, tm, tn, mt, nt);
  int k0, k1;
  g_part_range(kt, u, k0, k1);
  typename DenseOps<NS>::type ops = dense_ops<NS>(g, b, mt, nt, k0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  gemm_mainloop_issue(ops, k1 - k0, lds);
  GAcc acc;
  for (;;) {
    const int cb = b, cmt = mt, cnt = nt, nparts = u.nparts, punit = u.tail * u.nparts + u.part;
    gemm_zero(acc);
    gemm_mainloop_rest(ops, k1 - k0, acc, lds);
    bid += gridDim.x;
    const bool more = g_unit(g.sp, total, bid, u);
    __builtin_amdgcn_s_barrier();  // every wave is past its last read of the ring
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
      tile = u.tile;
      b = dense_batch<BATCHED>(g, tm * tn, tile);
      g_tile_coords(tile, tm, tn, mt, nt);
      g_part_range(kt, u, k0, k1);
      ops = dense_ops<NS>(g, b, mt, nt, k0);
      gemm_mainloop_issue(ops, k1 - k0, lds);
    }
    if (nparts > 1) g_part_store(g.sp.part, punit, acc);
    else dense_finish(g, g.C + cb * g.bsC, cmt, cnt, acc, lds.A[GNST - 1]);
    if (!more) break;
  }
}

__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_latent_down_kernel(DenseArgs g) {
  MOE_GEMM_LDS(lds);
  dense_body_persistent<1>(g, lds);
}

// up-projection + shared experts: 1 + S segments
// (persistent with at most one shared expert: with more segments the loop
// needs more than 256 VGPRs)
template <int NS>
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_up_shared_kernel(DenseArgs g) {
  MOE_GEMM_LDS(lds);
  if constexpr (NS <= 2) dense_body_persistent<NS>(g, lds);
  else dense_body<NS>(g, lds);
}

// products of the backward pass: NS K segments, or a batch of products
template <int NS, bool BATCHED>
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_nt_kernel(DenseArgs g) {
  MOE_GEMM_LDS(lds);
  dense_body_persistent<NS, BATCHED>(g, lds);
}

// the split tiles of a dense product: sum of parts, then the store
template <bool BATCHED = false>
__global__ __launch_bounds__(GNT) void gemm_dense_tail_kernel(DenseArgs g) {
  const int tm = (g.M + GBM - 1) / GBM, tn = (g.N + GBN - 1) / GBN;
  GUnit u;
  if (!g_tail_tile(g.sp, tm * tn * (BATCHED ? g.nbatch : 1), blockIdx.x / GTM, u)) return;
  int tile = u.tile;
  const int b = dense_batch<BATCHED>(g, tm * tn, tile);
  int mt, nt;
  g_tile_coords(tile, tm, tn, mt, nt);
  uint16_t *C = g.C + b * g.bsC;
  GAcc acc;
#define MOE_ROWS(I)                                       \
  g_part_sum_rows<I>(g.sp.part, u.tail, u.nparts, acc); \
  dense_store<I>(g, C, mt, nt, acc)
  MOE_TAIL_ROWS(MOE_ROWS)
#undef MOE_ROWS
}

// ---------------------------------------------------------------------------
// several independent products with one K in one launch (the backward's
// weight gradients): product p owns logical tiles first[p] .. first[p+1]-1
// ---------------------------------------------------------------------------

constexpr int GMAXPROD = 18;

struct MultiArgs {
  int nprod, ktiles;
  // kfill != NULL: product p's K is the sum of kfill[w * kEl + kgroup[p]]
  // over w < kW (rounded up to whole K tiles, at least min(GSPLIT_MAX,
  // ktiles) so that every split part has one), at most ktiles; the operands
  // hold zeros from there to ktiles.  kpack: the groups' K ranges lie one
  // after another in the same operands (group q from the sum of
  // kpack_len(earlier groups) on), instead of each group's own operands.
  const int32_t *kfill;
  int kW, kEl, kpack;
  int kgroup[GMAXPROD];
  int first[GMAXPROD + 1];
  const uint16_t *A[GMAXPROD];
  const uint16_t *B[GMAXPROD];
  uint16_t *C[GMAXPROD];
  int64_t lda[GMAXPROD], ldb[GMAXPROD], ldc[GMAXPROD];
  int M[GMAXPROD], N[GMAXPROD];
  GSplit sp;
};

// Product of logical tile `tile` (wave-uniform scan of the prefix table).
__device__ __forceinline__ int multi_product(const MultiArgs &g, int tile) {
  int p = 0;
  while (p + 1 < g.nprod && tile >= g.first[p + 1]) ++p;
  return p;
}

__device__ __forceinline__ int multi_group_rows(const MultiArgs &g, int q) {
  int f = 0;
  for (int w = 0; w < g.kW; ++w) f += g.kfill[w * g.kEl + q];
  return f;
}

__device__ __forceinline__ int multi_ktiles(const MultiArgs &g, int p) {
  if (!g.kfill) return g.ktiles;
  const int kt = max((multi_group_rows(g, g.kgroup[p]) + GBK - 1) / GBK, min(GSPLIT_MAX, g.ktiles));
  return __builtin_amdgcn_readfirstlane(min(kt, g.ktiles));
}

// First K element of product p's range in packed operands (0 otherwise).
__device__ __forceinline__ int64_t multi_kstart(const MultiArgs &g, int p) {
  if (!g.kpack) return 0;
  int64_t k = 0;
  for (int q = 0; q < g.kgroup[p]; ++q) k += kpack_len(multi_group_rows(g, q));
  return __builtin_amdgcn_readfirstlane((int)k);
}

template <int ONLY = -1>
__device__ __forceinline__ void multi_store(uint16_t *C, int64_t ldc, int M, int N, int mt, int nt,
                                            const GAcc &acc, uint16_t *ring = nullptr) {
  if (ONLY < 0 && g_vec_out(C, ldc, N)) {
    const int w = (int)(threadIdx.x >> 6);
    const int m0 = mt * GBM + (w / GWN) * GWTM, n0 = nt * GBN + (w % GWN) * GWTN;
    g_wave_store<GTN>(
        ring, [&](int i, int j, int v) { return acc[i][j][v]; },
        [&](int r) -> uint16_t * { return m0 + r < M ? C + (int64_t)(m0 + r) * ldc + n0 : nullptr; },
        N - n0);
    return;
  }
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int j = 0; j < GTN; ++j) {
      if (ONLY >= 0 && i != ONLY) continue;
      const int n = nt * GBN + g_acc_col(j);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mt * GBM + g_acc_row(i, v);
        if (m < M && n < N) C[(int64_t)m * ldc + n] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_nt_multi_kernel(MultiArgs g) {
  MOE_GEMM_LDS(lds);
  GUnit u;
  // with K from the device, tile costs differ by product
  if (!g_unit(g.sp, g.first[g.nprod], blockIdx.x, u, g.kfill != nullptr)) return;
  const int p = multi_product(g, u.tile);
  const int M = g.M[p], N = g.N[p];
  const int tm = (M + GBM - 1) / GBM, tn = (N + GBN - 1) / GBN;
  int mt, nt;
  g_tile_coords(u.tile - g.first[p], tm, tn, mt, nt);
  const int mv = M - mt * GBM, nv = N - nt * GBN;
  int k0, k1;
  g_part_range(multi_ktiles(g, p), u, k0, k1);
  const int64_t kb = multi_kstart(g, p) + (int64_t)k0 * GBK;
  const auto ops = g_operands(
      g.A[p] + (int64_t)mt * GBM * g.lda[p] + kb, g.lda[p], [&](int r) { return min(r, mv - 1); },
      g.B[p] + (int64_t)nt * GBN * g.ldb[p] + kb, g.ldb[p], [&](int r) { return min(r, nv - 1); });
  GAcc acc;
  gemm_zero(acc);
  gemm_mainloop(ops, k1 - k0, acc, lds);
  if (u.nparts > 1) {
    g_part_store(g.sp.part, u.tail * u.nparts + u.part, acc);
    return;
  }
  multi_store(g.C[p], g.ldc[p], M, N, mt, nt, acc, lds.A[0]);
}

__global__ __launch_bounds__(GNT) void gemm_nt_multi_tail_kernel(MultiArgs g) {
  GUnit u;
  if (!g_tail_tile(g.sp, g.first[g.nprod], blockIdx.x / GTM, u)) return;
  const int p = multi_product(g, u.tile);
  const int M = g.M[p], N = g.N[p];
  const int tm = (M + GBM - 1) / GBM, tn = (N + GBN - 1) / GBN;
  int mt, nt;
  g_tile_coords(u.tile - g.first[p], tm, tn, mt, nt);
  GAcc acc;
#define MOE_ROWS(I)                                       \
  g_part_sum_rows<I>(g.sp.part, u.tail, u.nparts, acc); \
  multi_store<I>(g.C[p], g.ldc[p], M, N, mt, nt, acc)
  MOE_TAIL_ROWS(MOE_ROWS)
#undef MOE_ROWS
}

// ---------------------------------------------------------------------------
// grouped rows: the bank's groups (wave w, local expert j) = group w * El + j
// ---------------------------------------------------------------------------

constexpr int GMAXW = 4;  // waves merged into one product group at most

// nw == 1: every bank group is a product group.  nw == n_waves: product
// group j holds local expert j's rows of every wave (same weights), in wave
// order, so its last 256-row tile is padded once instead of once per wave.
struct GroupArgs {
  int G, El, cap, nw;
  const int32_t *count;    // [G] rows per bank group
  const int64_t *offsets;  // ragged: [G+1] first row per bank group; NULL if fixed
};

// One block tile of a grouped product: its product group's segments (one
// per merged wave) and the tile's first row within the group.
struct GTile {
  int expert, rows, mt, nt, nseg, v0;
  int64_t start[GMAXW];  // bank row of each segment's first row
  int cum[GMAXW];        // group rows up to the end of each segment
  // bank row of tile row m (m < rows)
  __device__ __forceinline__ int64_t row(int m) const {
    const int v = v0 + m;
    int64_t r = start[0] + v;
#pragma unroll
    for (int s = 1; s < GMAXW; ++s)
      if (s < nseg && v >= cum[s - 1]) r = start[s] + (v - cum[s - 1]);
    return r;
  }
};

__device__ __forceinline__ int group_seg(const GroupArgs &a, int pg, int s) {
  return a.nw == 1 ? pg : s * a.El + pg;
}

__device__ __forceinline__ int group_rows(const GroupArgs &a, int pg) {
  int c = 0;
  for (int s = 0; s < a.nw; ++s) c += a.count[group_seg(a, pg, s)];
  return c;
}

// Tiles of a grouped product: product groups in order, each contributing
// ceil(rows / 256) * tn tiles.  The counts are known only on the device, so
// the launch grid is an upper bound and blocks past the last unit exit.
__device__ __forceinline__ int group_total(const GroupArgs &a, int tn) {
  const int npg = a.G / a.nw;
  int total = 0;
  for (int pg = 0; pg < npg; ++pg) total += ((group_rows(a, pg) + GBM - 1) / GBM) * tn;
  return total;
}

// Logical tile `rem` of a grouped product; false (t.rows = 0) if rem is not
// below group_total.
__device__ __forceinline__ bool group_tile_at(const GroupArgs &a, int tn, int rem, GTile &t) {
  const int npg = a.G / a.nw;
  t.rows = 0;
  for (int pg = 0; pg < npg; ++pg) {
    const int c = group_rows(a, pg);
    const int tmg = (c + GBM - 1) / GBM;
    if (rem < tmg * tn) {
      g_tile_coords(rem, tmg, tn, t.mt, t.nt);
      t.expert = group_seg(a, pg, 0) % a.El;
      t.v0 = t.mt * GBM;
      t.rows = min(GBM, c - t.v0);
      t.nseg = a.nw;
      int cum = 0;
#pragma unroll
      for (int s = 0; s < GMAXW; ++s) {
        if (s < a.nw) {
          const int g = group_seg(a, pg, s);
          t.start[s] = a.offsets ? a.offsets[g] : (int64_t)g * a.cap;
          cum += a.count[g];
        } else {
          t.start[s] = 0;
        }
        t.cum[s] = cum;
      }
      return t.rows > 0;
    }
    rem -= tmg * tn;
  }
  return false;
}

// The same table read into registers once per wave (at most 64 bank groups
// and 64 product groups): lane g holds bank group g's row count and first
// row, lane pg the first logical tile of product group pg.  One round of
// independent loads, where the walk above waits for one load after another
// (bank counts written by an earlier kernel sit in another XCD's L2, about a
// microsecond away).  With more groups the walk is used.
struct GroupRegs {
  bool fast;
  int total;      // tiles (wave-uniform)
  int count;      // lane g: rows of bank group g
  int64_t start;  // lane g: first bank row of bank group g
  int prefix;     // lane pg: tiles of the product groups before pg
};

__device__ __forceinline__ GroupRegs group_regs(const GroupArgs &a, int tn) {
  GroupRegs r{};
  const int npg = a.G / a.nw;
  r.fast = a.G <= 64;
  if (!r.fast) {
    r.total = group_total(a, tn);
    return r;
  }
  const int l = lane_id();
  r.count = l < a.G ? a.count[l] : 0;
  r.start = l < a.G ? (a.offsets ? a.offsets[l] : (int64_t)l * a.cap) : 0;
  int rows = 0;
  for (int s = 0; s < a.nw; ++s) rows += __shfl(r.count, l < npg ? group_seg(a, l, s) : 0);
  const int tiles = l < npg ? (rows + GBM - 1) / GBM * tn : 0;
  int inc = tiles;  // inclusive prefix over the lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(inc, d);
    if (l >= d) inc += v;
  }
  r.prefix = inc - tiles;
  r.total = __builtin_amdgcn_readlane(inc, 63);
  return r;
}

// group_tile_at from the registers.
__device__ __forceinline__ bool group_tile_regs(const GroupArgs &a, const GroupRegs &r, int tn,
                                                int rem, GTile &t) {
  if (!r.fast) return group_tile_at(a, tn, rem, t);
  t.rows = 0;
  if (rem < 0 || rem >= r.total) return false;
  const int npg = a.G / a.nw;
  // prefixes never decrease: the last group starting at or before rem holds it
  const uint64_t m = __ballot(lane_id() < npg && r.prefix <= rem);
  const int pg = __builtin_amdgcn_readfirstlane(63 - __clzll(m));
  rem -= __builtin_amdgcn_readlane(r.prefix, pg);
  int c = 0;
  for (int s = 0; s < a.nw; ++s) c += __builtin_amdgcn_readlane(r.count, group_seg(a, pg, s));
  const int tmg = (c + GBM - 1) / GBM;
  g_tile_coords(rem, tmg, tn, t.mt, t.nt);
  t.expert = group_seg(a, pg, 0) % a.El;
  t.v0 = t.mt * GBM;
  t.rows = min(GBM, c - t.v0);
  t.nseg = a.nw;
  int cum = 0;
#pragma unroll
  for (int s = 0; s < GMAXW; ++s) {
    if (s < a.nw) {
      const int g = group_seg(a, pg, s);
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)r.start, g);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)r.start >> 32), g);
      t.start[s] = (int64_t)(((uint64_t)hi << 32) | lo);
      cum += __builtin_amdgcn_readlane(r.count, g);
    } else {
      t.start[s] = 0;
    }
    t.cum[s] = cum;
  }
  return t.rows > 0;
}

// ---------------------------------------------------------------------------
// SwiGLU
// ---------------------------------------------------------------------------

struct SwigluArgs {
  const uint16_t *A;  // rows
  int64_t lda;
  int ktiles;
  const uint16_t *Bg, *Bu;  // [experts][F][K]
  int64_t ldb;
  int F, ftiles;  // ftiles = F / 128
  uint16_t *H;
  int64_t ldh;
  // backward epilogue: dH (gradient of h, read at column dh_col0 + the h
  // column), AB (d_a at the h column, d_b ab_off columns further)
  const uint16_t *dH;
  int64_t ld_dh;
  int dh_col0;
  uint16_t *AB;
  int64_t ld_ab;
  int ab_off;
  // backward, grouped, merged product groups (one per local expert): also
  // h and d_a | d_b transposed, in the layout the weight gradients read (K =
  // the expert's filled bank rows, packed): HT [F][ldt], ABT [2F][ldt] (d_a at
  // column c, d_b at F + c) per expert block (fixed: expert e's at e * F *
  // ldt and e * 2F * ldt, k from 0) or one block (kpack: expert e's range
  // from the sum of kpack_len over the experts before it); k from the
  // expert's fill up to its padded end is written as zero.  HT NULL: none
  // (then h goes to H).
  uint16_t *HT, *ABT;
  int64_t ldt;
  int kpack;
  // dense (shared experts): M rows, expert = f-tile / ftiles along N
  int M, S;
  // grouped (routed experts)
  GroupArgs grp;
  GSplit sp;
};

// row_of(m): row of A and H for tile row m < rows (contiguous rows, or the
// bank rows of a grouped tile).  K tiles [k0, k1) into acc.
typedef GOps<GOperand<GCA>, GOperand<GCB>> GOps2;

template <class RowOf>
__device__ __forceinline__ GOps2 swiglu_ops(const SwigluArgs &g, RowOf row_of, int rows,
                                            int expert, int ft, int k0) {
  const int f0 = ft * 128;
  const int64_t eoff = (int64_t)expert * g.F * g.ldb + (int64_t)f0 * g.ldb + k0 * GBK;
  // whether a thread copies gate or up rows depends on the thread only (its
  // copy rows are 64 apart, g_swiglu_brow sees row % 64), so the base stays
  // wave-uniform
  bool up;
  int foff;
  g_swiglu_brow(g_load_row(0), up, foff);
  const int64_t r0 = row_of(0);
  return g_operands(
      g.A + r0 * g.lda + k0 * GBK, g.lda,
      [&](int r) { return (int)(row_of(min(r, rows - 1)) - r0); }, (up ? g.Bu : g.Bg) + eoff,
      g.ldb, [&](int r) {
        bool u;
        int f;
        g_swiglu_brow(r, u, f);
        return f;
      });
}

template <class RowOf>
__device__ __forceinline__ void swiglu_acc(const SwigluArgs &g, RowOf row_of, int rows, int expert,
                                           int ft, int k0, int k1, const GemmLds &lds,
                                           GAcc &acc) {
  const auto ops = swiglu_ops(g, row_of, rows, expert, ft, k0);
  gemm_zero(acc);
  gemm_mainloop(ops, k1 - k0, acc, lds);
}

// The backward's three outputs (h, d_a, d_b) of row groups I0 .. I1 - 1,
// stored straight from registers.  d_h of every row group is loaded first
// (all of it before any store), 4 consecutive columns of one row per lane
// with one 8-byte load, and turned into this lane's column by the 4 x 4
// transpose inside groups of 4 lanes (g_tr4x4, its own inverse); each
// output's bf16 pairs go through the same transpose, and every lane stores 4
// consecutive columns of one row with one 8-byte store (16 loads and 48
// stores per wave instead of 64 and 192 two-byte ones).  d_h and the
// outputs 8-byte aligned (swiglu_bwd_vec checks it).
__device__ __forceinline__ bool swiglu_bwd_vec(const SwigluArgs &g, int h_col0, int f0) {
  const int c = h_col0 + f0;
  return ((((uintptr_t)(g.H + c)) | ((uintptr_t)(g.AB + c)) | ((uintptr_t)(g.AB + g.ab_off + c)) |
           ((uintptr_t)(g.dH + g.dh_col0 + c))) &
          7) == 0 &&
         (g.ldh & 3) == 0 && (g.ld_ab & 3) == 0 && (g.ld_dh & 3) == 0;
}

// Where tile t's rows go in the transposed outputs: tile row m at k = tk0 + m
// of its expert's block (ht, abt), for m < krows (rows past t.rows there are
// the expert's zero padding: up to its fill rounded to whole K tiles, and at
// least min(256, ldt) -- the weight gradients read at least 8 K tiles).  An
// expert with no rows has no tile: its range is zeroed elsewhere.
struct SwigluTPos {
  uint16_t *ht, *abt;
  int64_t tk0;
  int krows;
};

__device__ __forceinline__ SwigluTPos swiglu_tpos(const SwigluArgs &g, const GTile &t) {
  SwigluTPos p;
  const int e = t.expert, fill = group_rows(g.grp, e);
  int64_t kb = 0;
  if (g.kpack) {
    for (int x = 0; x < e; ++x) kb += kpack_len(group_rows(g.grp, x));
    p.ht = g.HT;
    p.abt = g.ABT;
  } else {
    p.ht = g.HT + (int64_t)e * g.F * g.ldt;
    p.abt = g.ABT + (int64_t)e * 2 * g.F * g.ldt;
  }
  const int64_t pend =
      g.kpack ? kpack_len(fill) : max((int64_t)(fill + 31) / 32 * 32, min<int64_t>(256, g.ldt));
  p.tk0 = kb + t.v0;
  p.krows = (int)min<int64_t>(GBM, pend - t.v0);
  return p;
}

// Transposed outputs of two MFMA row groups (64 rows x 32 columns of the
// wave) through the wave's LDS region, GTR_OUTS outputs of 32 columns x
// GTR_LD elements: each lane writes its column's 4-row groups (8 bytes each,
// rows past `rows` zero), then reads 16-byte runs of k back and stores them
// to row c0 + c of its output (k from tk0 + the pair's first row), so that 8
// lanes write one column's 128 bytes (a whole line).  The padded row length
// spreads the columns over the LDS banks.
constexpr int GTR_ROWS = 64, GTR_LD = GTR_ROWS + 8, GTR_OUTS = 3;
static_assert(GNT / 64 * GTR_OUTS * 32 * GTR_LD <= GNST * (GSA + GSB),
              "transpose regions inside the ring");

template <class Pairs, class Out>
__device__ __forceinline__ void swiglu_tr_pair(uint16_t *region, Pairs pairs, int r0, int rows,
                                               Out out, int64_t ldt, int64_t k0, int krows) {
  const int lane = lane_id(), c = lane & 31;
#pragma unroll
  for (int o = 0; o < GTR_OUTS; ++o)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = ii * 32 + 8 * q + 4 * (lane >> 5), mg = r0 + r;
        uint32_t p0 = pairs(o, ii, 2 * q), p1 = pairs(o, ii, 2 * q + 1);
        if (mg + 4 > rows) {
          p0 &= (mg < rows ? 0xffffu : 0u) | (mg + 1 < rows ? 0xffff0000u : 0u);
          p1 &= (mg + 2 < rows ? 0xffffu : 0u) | (mg + 3 < rows ? 0xffff0000u : 0u);
        }
        *reinterpret_cast<u32x2 *>(region + (o * 32 + c) * GTR_LD + r) = u32x2{p0, p1};
      }
#pragma unroll
  for (int o = 0; o < GTR_OUTS; ++o)
#pragma unroll
    for (int j = 0; j < 32 * (GTR_ROWS / 8) / 64; ++j) {
      const int idx = j * 64 + lane, cc = idx / (GTR_ROWS / 8), kc = idx % (GTR_ROWS / 8);
      const u32x4 v = *reinterpret_cast<const u32x4 *>(region + (o * 32 + cc) * GTR_LD + kc * 8);
      if (r0 + kc * 8 < krows) *reinterpret_cast<u32x4 *>(out(o) + cc * ldt + k0 + r0 + kc * 8) = v;
    }
}

// tr: also the transposed outputs, at the tile's position tp (then h is not
// stored row-major): with LDS_TR through the wave's region of `ring` (an
// even number of row groups), else with one 8-byte store per lane and 4-row
// group.
template <int I0, int I1, bool LDS_TR = false, class RowOf>
__device__ __forceinline__ void swiglu_bwd_store(const SwigluArgs &g, RowOf row_of, int rows,
                                                 int h_col0, int f0, const GAcc &acc,
                                                 bool tr = false, SwigluTPos tp = {},
                                                 uint16_t *ring = nullptr) {
  static_assert(GTN == 2, "one gate and one up tile per wave");
  constexpr int NI = I1 - I0;
  const int lane = lane_id(), w = (int)(threadIdx.x >> 6);
  const int wm0 = (w / GWN) * GWTM, c0 = h_col0 + f0 + (w % GWN) * (GWTN / 2);
  const int col4 = (lane & 31) & ~3;
  constexpr int NP = NI >= 2 ? 2 : 1;  // row groups per pass
  // d_h: 4 columns of one row per lane, loaded a pass ahead (before the
  // previous pass's stores)
  const auto load_dh = [&](int i2, u32x2 (&gr)[NP][4]) {
#pragma unroll
    for (int ii = 0; ii < NP; ++ii)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm0 + (i2 + ii) * 32 + 8 * q + 4 * (lane >> 5) + (lane & 3);
        gr[ii][q] = *reinterpret_cast<const u32x2 *>(
            g.dH + row_of(min(m, rows - 1)) * g.ld_dh + g.dh_col0 + c0 + col4);
      }
  };
  u32x2 gr[NP][4];
  load_dh(I0, gr);
  static_assert(!LDS_TR || NI % 2 == 0, "LDS transposes take row groups in pairs");
  const auto T = [&](int o) {
    return o == 0 ? tp.ht + (int64_t)c0 * g.ldt
                  : tp.abt + (int64_t)(c0 + (o == 2 ? g.F : 0)) * g.ldt;
  };
  // row groups NP at a time: h, d_a, d_b as bf16 pairs of this lane's column
#pragma unroll
  for (int i2 = I0; i2 < I1; i2 += NP) {
    uint32_t P[GTR_OUTS][NP][8];
#pragma unroll
    for (int ii = 0; ii < NP; ++ii)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i2 + ii;
        uint32_t gh[2];
        g_tr4x4(gr[ii][q][0], gr[ii][q][1], gh[0], gh[1]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = 2 * q + h;
          float vh[2], va[2], vb[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float a = acc[i][0][2 * k + e], b = acc[i][1][2 * k + e];
            const float dh = bf16_to_f32((uint16_t)(gh[h] >> (16 * e)));
            const float sg = sigmoid_f32(a);
            const float sa = a * sg;
            vh[e] = sa * b;
            va[e] = dh * b * (sg * (1.0f + a * (1.0f - sg)));
            vb[e] = dh * sa;
          }
          P[0][ii][k] = pack_bf16x2(vh[0], vh[1]);
          P[1][ii][k] = pack_bf16x2(va[0], va[1]);
          P[2][ii][k] = pack_bf16x2(vb[0], vb[1]);
        }
      }
    if (i2 + NP < I1) load_dh(i2 + NP, gr);
    // row-major stores first (d_a | d_b; h unless transposed), so that the
    // pairs die at the LDS writes of the transposed outputs
#pragma unroll
    for (int ii = 0; ii < NP; ++ii) {
      const int i = i2 + ii;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wm0 + i * 32 + 8 * q + 4 * (lane >> 5) + (lane & 3);
        uint32_t h0, h1, a0, a1, b0, b1;
        if (!tr) g_tr4x4(P[0][ii][2 * q], P[0][ii][2 * q + 1], h0, h1);
        g_tr4x4(P[1][ii][2 * q], P[1][ii][2 * q + 1], a0, a1);
        g_tr4x4(P[2][ii][2 * q], P[2][ii][2 * q + 1], b0, b1);
        if (m < rows) {
          const int64_t r = row_of(m);
          uint16_t *ab = g.AB + r * g.ld_ab + c0 + col4;
          if (!tr) *reinterpret_cast<u32x2 *>(g.H + r * g.ldh + c0 + col4) = u32x2{h0, h1};
          *reinterpret_cast<u32x2 *>(ab) = u32x2{a0, a1};
          *reinterpret_cast<u32x2 *>(ab + g.ab_off) = u32x2{b0, b1};
        }
      }
    }
    if constexpr (LDS_TR) {
      if (tr)
        swiglu_tr_pair(ring + w * (GTR_OUTS * 32 * GTR_LD),
                       [&](int o, int ii, int k) { return P[o][ii][k]; }, wm0 + i2 * 32, rows, T,
                       g.ldt, tp.tk0, tp.krows);
    } else if (tr) {
      // transposed: this lane's column, 4 consecutive rows (k) per 8-byte
      // store, zero past the tile's rows
      const int64_t c = lane & 31;
#pragma unroll
      for (int ii = 0; ii < NP; ++ii)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mg = wm0 + (i2 + ii) * 32 + 8 * q + 4 * (lane >> 5);
          if (mg >= tp.krows) continue;
#pragma unroll
          for (int o = 0; o < GTR_OUTS; ++o) {
            uint32_t v0 = P[o][ii][2 * q], v1 = P[o][ii][2 * q + 1];
            if (mg + 4 > rows) {
              v0 &= (mg < rows ? 0xffffu : 0u) | (mg + 1 < rows ? 0xffff0000u : 0u);
              v1 &= (mg + 2 < rows ? 0xffffu : 0u) | (mg + 3 < rows ? 0xffff0000u : 0u);
            }
            *reinterpret_cast<u32x2 *>(T(o) + c * g.ldt + tp.tk0 + mg) = u32x2{v0, v1};
          }
        }
    }
  }
}

// BWD: with dh = dH at the same (row, column), also
//   d_a = bf16(dh * b * silu'(a)),  d_b = bf16(dh * silu(a)),
//   silu'(a) = s (1 + a (1 - s)), s = 1 / (1 + e^-a).
// tr (backward with transposed outputs, which the launcher enables only for
// 8-byte aligned outputs): also those, at the tile's position tp.
template <int ONLY = -1, bool BWD = false, class RowOf>
__device__ __forceinline__ void swiglu_store(const SwigluArgs &g, RowOf row_of, int rows, int ft,
                                             int h_col0, const GAcc &acc,
                                             uint16_t *ring = nullptr, bool tr = false,
                                             SwigluTPos tp = {}) {
  const int f0 = ft * 128;
  if (BWD && swiglu_bwd_vec(g, h_col0, f0)) {
    if constexpr (ONLY < 0) swiglu_bwd_store<0, GTM>(g, row_of, rows, h_col0, f0, acc, tr, tp);
    else swiglu_bwd_store<ONLY, ONLY + 1>(g, row_of, rows, h_col0, f0, acc, tr, tp);
    return;
  }
  // the backward's three outputs keep the direct stores: staged, they need
  // more than 256 VGPRs
  if (!BWD && ONLY < 0 && g_vec_out(g.H + h_col0, g.ldh, 8)) {
    static_assert(GTN == 2, "one gate and one up tile per wave");
    const int w = (int)(threadIdx.x >> 6);
    const int m0 = (w / GWN) * GWTM, c0 = h_col0 + f0 + (w % GWN) * (GWTN / 2);
    const auto val = [&](int i, int, int v) { return silu_f32(acc[i][0][v]) * acc[i][1][v]; };
    const auto row_ptr = [&](int r) -> uint16_t * {
      return m0 + r < rows ? g.H + row_of(m0 + r) * g.ldh + c0 : nullptr;
    };
    g_wave_store<1>(ring, val, row_ptr, GWTN / 2);
    return;
  }
#pragma unroll
  for (int i = 0; i < GTM; ++i) {
    if (ONLY >= 0 && i != ONLY) continue;
    // BWD: the row group's d_h values are all loaded before the first store
    // (the stores could alias them, so loads after a store would wait for it)
    float gh[16][GTN / 2];
    if constexpr (BWD) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = g_acc_row(i, v);
        const uint16_t *dh = g.dH + row_of(min(m, rows - 1)) * g.ld_dh + g.dh_col0 + h_col0 + f0;
#pragma unroll
        for (int p = 0; p < GTN / 2; ++p) gh[v][p] = bf16_to_f32(dh[g_swiglu_col(p)]);
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = g_acc_row(i, v);
      if (m >= rows) continue;
      const int64_t r = row_of(m);
      uint16_t *h = g.H + r * g.ldh + h_col0 + f0;
      if constexpr (!BWD) {
#pragma unroll
        for (int p = 0; p < GTN / 2; ++p) {
          const float a = acc[i][2 * p][v], b = acc[i][2 * p + 1][v];
          h[g_swiglu_col(p)] = f32_to_bf16(silu_f32(a) * b);
        }
      } else {
        uint16_t *da = g.AB + r * g.ld_ab + h_col0 + f0;
#pragma unroll
        for (int p = 0; p < GTN / 2; ++p) {
          const float a = acc[i][2 * p][v], b = acc[i][2 * p + 1][v];
          const int c = g_swiglu_col(p);
          const float s = sigmoid_f32(a);
          const float sa = a * s;
          h[c] = f32_to_bf16(sa * b);
          da[c] = f32_to_bf16(gh[v][p] * b * (s * (1.0f + a * (1.0f - s))));
          da[g.ab_off + c] = f32_to_bf16(gh[v][p] * sa);
        }
      }
    }
  }
}

template <bool BWD>
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_shared_swiglu_kernel(SwigluArgs g) {
  MOE_GEMM_LDS(lds);
  const int tm = (g.M + GBM - 1) / GBM, tn = g.S * g.ftiles;
  GUnit u;
  if (!g_unit(g.sp, tm * tn, blockIdx.x, u)) return;
  int mt, nt;
  g_tile_coords(u.tile, tm, tn, mt, nt);
  const int s = nt / g.ftiles, ft = nt % g.ftiles;
  const int64_t row0 = (int64_t)mt * GBM;
  const auto row_of = [&](int m) { return row0 + m; };
  const int rows = min(GBM, g.M - mt * GBM);
  int k0, k1;
  g_part_range(g.ktiles, u, k0, k1);
  GAcc acc;
  swiglu_acc(g, row_of, rows, s, ft, k0, k1, lds, acc);
  if (u.nparts > 1) {
    g_part_store(g.sp.part, u.tail * u.nparts + u.part, acc);
    return;
  }
  swiglu_store<-1, BWD>(g, row_of, rows, ft, s * g.F, acc, lds.A[0]);
}

template <bool BWD>
__global__ __launch_bounds__(GNT) void gemm_shared_swiglu_tail_kernel(SwigluArgs g) {
  const int tm = (g.M + GBM - 1) / GBM, tn = g.S * g.ftiles;
  GUnit u;
  if (!g_tail_tile(g.sp, tm * tn, blockIdx.x / GTM, u)) return;
  int mt, nt;
  g_tile_coords(u.tile, tm, tn, mt, nt);
  const int s = nt / g.ftiles, ft = nt % g.ftiles;
  const int64_t row0 = (int64_t)mt * GBM;
  const int rows = min(GBM, g.M - mt * GBM);
  const auto row_of = [&](int m) { return row0 + m; };
  GAcc acc;
#define MOE_ROWS(I)                                       \
  g_part_sum_rows<I>(g.sp.part, u.tail, u.nparts, acc); \
  swiglu_store<I, BWD>(g, row_of, rows, ft, s * g.F, acc)
  MOE_TAIL_ROWS(MOE_ROWS)
#undef MOE_ROWS
}

// Persistent grouped kernels: block b runs units b, b + gridDim.x, ...
// (gridDim.x a multiple of 8, so that a block's units all fall in its XCD's
// tile range) and issues the first copies of its next unit before the
// epilogue of the current one (gemm_mainloop_issue), staging that epilogue
// in ring stage GNST - 1.  Across the main loop a unit keeps only what its
// epilogue needs (a few scalars and, per lane, the output rows of two of
// its wave's tile rows): with the whole tile description live there, the
// loop needs more than 256 VGPRs.
__device__ __forceinline__ int32_t wave_tile_row(const GTile &t, int m) {
  return m < t.rows ? (int32_t)t.row(m) : -1;
}

// Row of wave-tile row r (0 .. 127): lane r % 64 holds it in rr[r / 64].
__device__ __forceinline__ int32_t wave_row_of(int32_t r0, int32_t r1, int r) {
  return __shfl(r < 64 ? r0 : r1, r & 63);
}

__device__ __forceinline__ void swiglu_finish(const SwigluArgs &g, int ft, int nparts, int punit,
                                              int32_t r0, int32_t r1, const GAcc &acc,
                                              uint16_t *stage) {
  if (nparts > 1) {
    g_part_store(g.sp.part, punit, acc);
    return;
  }
  static_assert(GTN == 2, "one gate and one up tile per wave");
  const int w = (int)(threadIdx.x >> 6);
  const int c0 = ft * 128 + (w % GWN) * (GWTN / 2);
  g_wave_store_staged<1>(
      stage, [&](int i, int, int v) { return silu_f32(acc[i][0][v]) * acc[i][1][v]; },
      [&](int r) -> uint16_t * {
        const int32_t row = wave_row_of(r0, r1, r);
        return row >= 0 ? g.H + (int64_t)row * g.ldh + c0 : nullptr;
      },
      GWTN / 2);
}

// The backward form (three outputs, stored directly) runs one unit per block:
// it keeps more registers live.
template <bool BWD>
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_expert_swiglu_kernel(SwigluArgs g) {
  MOE_GEMM_LDS(lds);
  const GroupRegs gr = group_regs(g.grp, g.ftiles);
  GUnit u;
  GTile t;
  int b = blockIdx.x;
  if (!g_unit(g.sp, gr.total, b, u) || !group_tile_regs(g.grp, gr, g.ftiles, u.tile, t))
    return;
  int k0, k1;
  g_part_range(g.ktiles, u, k0, k1);
  if constexpr (BWD) {
    const auto row_of = [&](int m) { return t.row(m); };
    GAcc acc;
    swiglu_acc(g, row_of, t.rows, t.expert, t.nt, k0, k1, lds, acc);
    if (u.nparts > 1) {
      g_part_store(g.sp.part, u.tail * u.nparts + u.part, acc);
    } else if (g.HT) {
      // transposed outputs through the ring, which is free: every wave is
      // past the main loop's last barrier (the launcher set HT only for
      // 8-byte aligned outputs)
      swiglu_bwd_store<0, GTM, true>(g, row_of, t.rows, 0, t.nt * 128, acc, true,
                                     swiglu_tpos(g, t), lds.A[0]);
    } else {
      swiglu_store<-1, true>(g, row_of, t.rows, t.nt, 0, acc);
    }
  } else {
    // H rows take 16-byte stores (the launcher checks it)
    GOps2 ops = swiglu_ops(g, [&](int m) { return t.row(m); }, t.rows, t.expert, t.nt, k0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    gemm_mainloop_issue(ops, k1 - k0, lds);
    GAcc acc;
    GSeq seq = gseq_start();
    for (;;) {
      const int m0 = ((int)(threadIdx.x >> 6) / GWN) * GWTM;
      const int32_t r0 = wave_tile_row(t, m0 + lane_id()), r1 = wave_tile_row(t, m0 + 64 + lane_id());
      const int ft = t.nt, nparts = u.nparts, punit = u.tail * u.nparts + u.part, kt = k1 - k0;
      gseq_draw(g.sp.q, seq);
      gemm_zero(acc);
      gemm_mainloop_rest(ops, kt, acc, lds);
      gseq_post(g.sp.q, seq);
      b = seq.next;
      const bool more =
          g_unit(g.sp, gr.total, b, u) && group_tile_regs(g.grp, gr, g.ftiles, u.tile, t);
      __builtin_amdgcn_s_barrier();  // every wave is past its last read of the ring
      __builtin_amdgcn_sched_barrier(0);
      gseq_fetch(g.sp.q, seq);
      if (more) {
        g_part_range(g.ktiles, u, k0, k1);
        ops = swiglu_ops(g, [&](int m) { return t.row(m); }, t.rows, t.expert, t.nt, k0);
        gemm_mainloop_issue(ops, k1 - k0, lds);
      }
      swiglu_finish(g, ft, nparts, punit, r0, r1, acc, lds.A[GNST - 1]);
      if (!more) break;
    }
  }
}

template <bool BWD>
__global__ __launch_bounds__(GNT) void gemm_expert_swiglu_tail_kernel(SwigluArgs g) {
  GUnit u;
  GTile t;
  const GroupRegs gr = group_regs(g.grp, g.ftiles);
  if (!g_tail_tile(g.sp, gr.total, blockIdx.x / GTM, u) ||
      !group_tile_regs(g.grp, gr, g.ftiles, u.tile, t))
    return;
  const auto row_of = [&](int m) { return t.row(m); };
  GAcc acc;
  const bool tr = BWD && g.HT;
  SwigluTPos tp{};
  if (tr) tp = swiglu_tpos(g, t);
#define MOE_ROWS(I)                                       \
  g_part_sum_rows<I>(g.sp.part, u.tail, u.nparts, acc); \
  swiglu_store<I, BWD>(g, row_of, t.rows, t.nt, 0, acc, nullptr, tr, tp)
  MOE_TAIL_ROWS(MOE_ROWS)
#undef MOE_ROWS
}

// ---------------------------------------------------------------------------
// expert down-projection with scatter to the receive layout
// ---------------------------------------------------------------------------

struct DownArgs {
  const uint16_t *H;  // [bank rows][F]
  int F, ktiles;
  const uint16_t *Wd;  // [El][L][F]
  int L, tn;
  GroupArgs grp;
  const int32_t *bank_src;
  uint16_t *ret;  // [ret rows][L]
  int64_t n_ret;
  GSplit sp;
};

// dst_of(m): receive row of tile row m (negative or >= n_ret: not stored).
template <int ONLY = -1, class DstOf>
__device__ __forceinline__ void down_store(const DownArgs &g, const GTile &t, DstOf dst_of,
                                           const GAcc &acc, uint16_t *ring = nullptr) {
  if (ONLY < 0 && g_vec_out(g.ret, g.L, g.L)) {
    const int w = (int)(threadIdx.x >> 6);
    const int m0 = (w / GWN) * GWTM, n0 = t.nt * GBN + (w % GWN) * GWTN;
    g_wave_store<GTN>(
        ring, [&](int i, int j, int v) { return acc[i][j][v]; },
        [&](int r) -> uint16_t * {
          if (m0 + r >= t.rows) return nullptr;
          const int64_t dr = dst_of(m0 + r);
          return dr >= 0 && dr < g.n_ret ? g.ret + dr * g.L + n0 : nullptr;
        },
        g.L - n0);
    return;
  }
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (ONLY >= 0 && i != ONLY) continue;
      const int m = g_acc_row(i, v);
      if (m >= t.rows) continue;
      const int64_t dr = dst_of(m);
      if (dr < 0 || dr >= g.n_ret) continue;
      const int64_t dst = dr * g.L;
#pragma unroll
      for (int j = 0; j < GTN; ++j) {
        const int n = t.nt * GBN + g_acc_col(j);
        if (n < g.L) g.ret[dst + n] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

__device__ __forceinline__ GOps2 down_ops(const DownArgs &g, const GTile &t, int k0) {
  const uint16_t *W = g.Wd + (int64_t)t.expert * g.L * g.F;
  const int nv = g.L - t.nt * GBN, rows = t.rows;
  const int64_t r0 = t.row(0);
  return g_operands(
      g.H + r0 * g.F + k0 * GBK, g.F,
      [&](int r) { return (int)(t.row(min(r, rows - 1)) - r0); },
      W + (int64_t)t.nt * GBN * g.F + k0 * GBK, g.F, [&](int r) { return min(r, nv - 1); });
}

// Receive row of wave-tile row m0 + lane + 64 * h of a whole tile (-1: none).
__device__ __forceinline__ int32_t down_dst(const DownArgs &g, const GUnit &u, const GTile &t,
                                            int m) {
  return u.nparts == 1 && m < t.rows ? g.bank_src[t.row(m)] : -1;
}

__device__ __forceinline__ void down_finish(const DownArgs &g, int nt, int nparts, int punit,
                                            int32_t d0, int32_t d1, const GAcc &acc,
                                            uint16_t *stage) {
  if (nparts > 1) {
    g_part_store(g.sp.part, punit, acc);
    return;
  }
  const int w = (int)(threadIdx.x >> 6);
  const int n0 = nt * GBN + (w % GWN) * GWTN;
  g_wave_store_staged<GTN>(
      stage, [&](int i, int j, int v) { return acc[i][j][v]; },
      [&](int r) -> uint16_t * {
        const int32_t dr = wave_row_of(d0, d1, r);
        return dr >= 0 && dr < g.n_ret ? g.ret + (int64_t)dr * g.L + n0 : nullptr;
      },
      g.L - n0);
}

// Persistent like the forward SwiGLU; output rows 16-byte aligned (the
// launcher checks it).
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_expert_down_kernel(DownArgs g) {
  MOE_GEMM_LDS(lds);
  const GroupRegs gr = group_regs(g.grp, g.tn);
  GUnit u;
  GTile t;
  int b = blockIdx.x;
  if (!g_unit(g.sp, gr.total, b, u) || !group_tile_regs(g.grp, gr, g.tn, u.tile, t)) return;
  int k0, k1;
  g_part_range(g.ktiles, u, k0, k1);
  GOps2 ops = down_ops(g, t, k0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  gemm_mainloop_issue(ops, k1 - k0, lds);
  GAcc acc;
  GSeq seq = gseq_start();
  for (;;) {
    // receive rows of this wave's tile rows, loaded while the main loop runs
    const int m0 = ((int)(threadIdx.x >> 6) / GWN) * GWTM;
    const int32_t d0 = down_dst(g, u, t, m0 + lane_id()), d1 = down_dst(g, u, t, m0 + 64 + lane_id());
    const int nt = t.nt, nparts = u.nparts, punit = u.tail * u.nparts + u.part, kt = k1 - k0;
    gseq_draw(g.sp.q, seq);
    gemm_zero(acc);
    gemm_mainloop_rest(ops, kt, acc, lds);
    gseq_post(g.sp.q, seq);
    // d0, d1 waited for here, while no copy is outstanding
    asm volatile("" ::"v"(d0), "v"(d1));
    b = seq.next;
    const bool more = g_unit(g.sp, gr.total, b, u) && group_tile_regs(g.grp, gr, g.tn, u.tile, t);
    __builtin_amdgcn_s_barrier();  // every wave is past its last read of the ring
    __builtin_amdgcn_sched_barrier(0);
    gseq_fetch(g.sp.q, seq);
    if (more) {
      g_part_range(g.ktiles, u, k0, k1);
      ops = down_ops(g, t, k0);
      gemm_mainloop_issue(ops, k1 - k0, lds);
    }
    down_finish(g, nt, nparts, punit, d0, d1, acc, lds.A[GNST - 1]);
    if (!more) break;
  }
}

__global__ __launch_bounds__(GNT) void gemm_expert_down_tail_kernel(DownArgs g) {
  __shared__ int32_t dst_rows[GBM];
  GUnit u;
  GTile t;
  const GroupRegs gr = group_regs(g.grp, g.tn);
  if (!g_tail_tile(g.sp, gr.total, blockIdx.x / GTM, u) ||
      !group_tile_regs(g.grp, gr, g.tn, u.tile, t))
    return;
  if ((int)threadIdx.x < GBM)
    dst_rows[threadIdx.x] = (int)threadIdx.x < t.rows ? g.bank_src[t.row(threadIdx.x)] : -1;
  __syncthreads();
  const auto dst_of = [&](int m) { return (int64_t)dst_rows[m]; };
  GAcc acc;
#define MOE_ROWS(I)                                       \
  g_part_sum_rows<I>(g.sp.part, u.tail, u.nparts, acc); \
  down_store<I>(g, t, dst_of, acc)
  MOE_TAIL_ROWS(MOE_ROWS)
#undef MOE_ROWS
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

// CUs the launchers plan for: those of the current device (cached per
// device), or fewer if MOE_GEMM_CUS (read at every call; the entry points
// have checked it) asks for it.  The count sets the persistent grids (one
// block per planned CU) and where a last round is split along K; results of
// tiles that are not split do not depend on it.
static int cu_count(int *ncu) {
  static int cache[64];
  int dev = 0;
  MOE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  int n = dev >= 0 && dev < 64 ? cache[dev] : 0;
  if (n <= 0) {
    MOE_TRY(hip_status(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev),
                       "hipDeviceGetAttribute"));
    if (n < 1) return fail(MOE_ERR_HIP, "device reports %d compute units", n);
    if (dev >= 0 && dev < 64) cache[dev] = n;
  }
  int cus = 0;
  MOE_TRY(gemm_cus_env(&cus));
  *ncu = cus > 0 ? std::min(n, cus) : n;
  return MOE_OK;
}

int64_t gemm_split_bytes() { return (int64_t)GSPLIT_UNITS * GPART_BYTES; }

// Split description for a product of kt K tiles; part == NULL, or too few
// K tiles for two parts, turns splitting off.
static int make_split(float *part, int kt, GSplit &sp) {
  sp.max_parts = std::min(GSPLIT_MAX, kt / GSPLIT_MIN_KT);
  sp.part = sp.max_parts >= 2 ? part : nullptr;
  sp.ncu = 1;
  sp.max_units = sp.part ? GSPLIT_UNITS : 0;
  return sp.part ? cu_count(&sp.ncu) : MOE_OK;
}

// Host mirror of g_split_parts.
static int split_parts(const GSplit &sp, int64_t total) {
  if (!sp.part) return 1;
  const int64_t r = total % sp.ncu;
  if (r == 0 || 2 * r > sp.ncu) return 1;
  return (int)std::max<int64_t>(
      1, std::min<int64_t>(std::min<int64_t>(sp.ncu / r, sp.max_parts), sp.max_units / r));
}

// persistent: k runs units b, b + grid, ... (dense_body_persistent); the grid
// is then one block per CU at most, a multiple of 8.
static int dense(const char *name, const char *tail_name, void (*k)(DenseArgs), int M, int N,
                 int nseg, const DenseSeg *segs, uint16_t *C, int64_t ldc, float *part,
                 hipStream_t s, bool persistent, int nbatch = 1, int64_t bsA = 0,
                 int64_t bsB = 0, int64_t bsC = 0) {
  if (nseg < 1 || nseg > MAXSEG) return fail(MOE_ERR_INVALID, "%s: bad segment count", name);
  if (nbatch < 1 || (nbatch > 1 && nseg != 1))
    return fail(MOE_ERR_INVALID, "%s: bad batch", name);
  DenseArgs a{};
  a.M = M;
  a.N = N;
  a.nseg = nseg;
  a.nbatch = nbatch;
  a.bsA = bsA;
  a.bsB = bsB;
  a.bsC = bsC;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].K % GBK) return fail(MOE_ERR_UNSUPPORTED, "%s: K %% %d != 0", name, GBK);
    // copy offsets within one 256-row tile are 32-bit
    if ((segs[i].lda | segs[i].ldb) < 0 || segs[i].lda * 2 * GBM > INT32_MAX ||
        segs[i].ldb * 2 * GBN > INT32_MAX)
      return fail(MOE_ERR_UNSUPPORTED, "%s: row stride too large", name);
    a.A[i] = segs[i].A;
    a.lda[i] = segs[i].lda;
    a.B[i] = segs[i].B;
    a.ldb[i] = segs[i].ldb;
    a.ktiles[i] = segs[i].K / GBK;
  }
  a.C = C;
  a.ldc = ldc;
  const int64_t tiles = cdiv(M, GBM) * cdiv(N, GBN) * nbatch;
  if (tiles > INT32_MAX / 2) return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", name);
  int kt = 0;
  for (int i = 0; i < nseg; ++i) kt += a.ktiles[i];
  MOE_TRY(make_split(part, kt, a.sp));
  int ncu = 0;
  MOE_TRY(cu_count(&ncu));
  const int64_t cap = persistent ? std::max(8, ncu / 8 * 8) : INT32_MAX;
  const int S = split_parts(a.sp, tiles);
  if (S == 1) {
    a.sp.part = nullptr;
    return launch(name, k, dim3((unsigned)std::min<int64_t>(tiles, cap)), dim3(GNT), 0, s, a);
  }
  const int64_t r = tiles % a.sp.ncu;
  MOE_TRY(launch(name, k, dim3((unsigned)std::min<int64_t>(tiles - r + r * S, cap)), dim3(GNT), 0,
                 s, a));
  return launch(tail_name, nbatch > 1 ? gemm_dense_tail_kernel<true> : gemm_dense_tail_kernel<false>,
                dim3((unsigned)(r * GTM)), dim3(GNT), 0, s, a);
}

int gemm_latent_down(int M, int N, const DenseSeg &seg, uint16_t *C, int64_t ldc, hipStream_t s) {
  return dense("gemm_latent_down", "gemm_latent_down_tail", gemm_latent_down_kernel, M, N, 1, &seg,
               C, ldc, nullptr, s, true);
}

int gemm_up_shared(int M, int N, int nseg, const DenseSeg *segs, uint16_t *C, int64_t ldc,
                   float *part, hipStream_t s) {
  static void (*const k[MAXSEG])(DenseArgs) = {gemm_up_shared_kernel<1>, gemm_up_shared_kernel<2>,
                                               gemm_up_shared_kernel<3>, gemm_up_shared_kernel<4>,
                                               gemm_up_shared_kernel<5>};
  if (nseg < 1 || nseg > MAXSEG) return fail(MOE_ERR_INVALID, "gemm_up_shared: bad segment count");
  return dense("gemm_up_shared", "gemm_up_shared_tail", k[nseg - 1], M, N, nseg, segs, C, ldc,
               part, s, nseg <= 2);
}

static int shared_swiglu(const char *name, const char *tail_name, void (*k)(SwigluArgs),
                         void (*tk)(SwigluArgs), SwigluArgs &a, int M, const uint16_t *x,
                         int64_t ldx, int K, const uint16_t *wg, const uint16_t *wu, int S, int F,
                         uint16_t *H, float *part, hipStream_t s) {
  a.A = x;
  a.lda = ldx;
  a.ktiles = K / GBK;
  a.Bg = wg;
  a.Bu = wu;
  a.ldb = K;
  a.F = F;
  a.ftiles = F / 128;
  a.H = H;
  a.ldh = (int64_t)S * F;
  a.M = M;
  a.S = S;
  MOE_TRY(make_split(part, a.ktiles, a.sp));
  const int64_t tiles = cdiv(M, GBM) * (int64_t)S * a.ftiles;
  const int P = split_parts(a.sp, tiles);
  if (P == 1) {
    a.sp.part = nullptr;
    return launch(name, k, dim3((unsigned)tiles), dim3(GNT), 0, s, a);
  }
  const int64_t r = tiles % a.sp.ncu;
  MOE_TRY(launch(name, k, dim3((unsigned)(tiles - r + r * P)), dim3(GNT), 0, s, a));
  return launch(tail_name, tk, dim3((unsigned)(r * GTM)), dim3(GNT), 0, s, a);
}

// Product groups of the bank: each local expert over every wave when the
// merged rows stay within 32-bit copy offsets of a tile's first row, else
// every (wave, expert) group alone.
static GroupArgs group_args(const moe_dims &d, const int64_t *bank_offsets, const int32_t *bfill,
                            int64_t n_bank_rows, int64_t width) {
  GroupArgs g{};
  g.El = experts_per_rank(d);
  g.G = d.n_waves * g.El;
  g.cap = d.cap_recv;
  g.count = bfill;
  g.offsets = ragged(d) ? bank_offsets : nullptr;
  const bool merge = d.n_waves <= GMAXW && n_bank_rows * width * 2 < INT32_MAX;
  g.nw = merge ? d.n_waves : 1;
  return g;
}

int gemm_shared_swiglu(int M, const uint16_t *x, int64_t ldx, int K, const uint16_t *wg,
                       const uint16_t *wu, int S, int F, uint16_t *H, float *part,
                       hipStream_t s) {
  if (S == 0) return MOE_OK;
  SwigluArgs a{};
  return shared_swiglu("gemm_shared_swiglu", "gemm_shared_swiglu_tail",
                       gemm_shared_swiglu_kernel<false>, gemm_shared_swiglu_tail_kernel<false>, a,
                       M, x, ldx, K, wg, wu, S, F, H, part, s);
}

int gemm_shared_swiglu_bwd(int M, const uint16_t *x, int64_t ldx, int K, const uint16_t *wg,
                           const uint16_t *wu, int S, int F, const uint16_t *dH, int64_t ld_dh,
                           int dh_col0, uint16_t *H, uint16_t *AB, float *part, hipStream_t s) {
  if (S == 0) return MOE_OK;
  SwigluArgs a{};
  a.dH = dH;
  a.ld_dh = ld_dh;
  a.dh_col0 = dh_col0;
  a.AB = AB;
  a.ld_ab = 2ll * S * F;
  a.ab_off = S * F;
  return shared_swiglu("gemm_shared_swiglu_bwd", "gemm_shared_swiglu_bwd_tail",
                       gemm_shared_swiglu_kernel<true>, gemm_shared_swiglu_tail_kernel<true>, a,
                       M, x, ldx, K, wg, wu, S, F, H, part, s);
}

static int64_t grouped_tiles_bound(const moe_dims &d, int64_t n_bank_rows, int tn) {
  const int64_t G = (int64_t)d.n_waves * experts_per_rank(d);
  const int64_t mt = ragged(d) ? cdiv(n_bank_rows, GBM) + G : G * cdiv(d.cap_recv, GBM);
  return mt * tn;
}

// A grouped product and, when splitting is on, its tail kernel.  The real
// tile count is known only on the device: the grid bounds it plus the ncu
// extra blocks a split can add; the tail kernel gets GTM blocks for each of
// ncu / 2 possible split tiles (a split never has more) and exits where
// there is none.
// queue: counters and slots of a work queue (GQueue; NULL: static units),
// the counters zeroed before the launch; used when the grid is persistent,
// a multiple of 8 and at most GQ_MAX_GRID blocks.
template <class Args>
static int grouped(const char *name, const char *tail_name, void (*k)(Args),
                   void (*tk)(Args), int64_t bound, int ktiles, Args &a, float *part,
                   hipStream_t s, bool persistent, int32_t *queue_count = nullptr,
                   int32_t *queue_slot = nullptr) {
  MOE_TRY(make_split(part, ktiles, a.sp));
  int ncu = 0;
  MOE_TRY(cu_count(&ncu));
  const int64_t units = bound + (a.sp.part ? a.sp.ncu : 0);
  // persistent: one block per CU at most, a multiple of 8 (the XCDs)
  const int64_t grid = persistent ? std::min<int64_t>(units, std::max(8, ncu / 8 * 8)) : units;
  const bool queued = persistent && queue_count && queue_slot && grid % 8 == 0 &&
                      grid <= GQ_MAX_GRID && units > grid;
  a.sp.q = queued ? GQueue{queue_count, queue_slot} : GQueue{nullptr, nullptr};
  MOE_TRY(launch(name, k, dim3((unsigned)grid), dim3(GNT), 0, s, a));
  if (!a.sp.part || a.sp.ncu < 2) return MOE_OK;
  return launch(tail_name, tk, dim3((unsigned)(a.sp.ncu / 2 * GTM)), dim3(GNT), 0, s, a);
}

static int expert_swiglu(const char *name, const char *tail_name, void (*k)(SwigluArgs),
                         void (*tk)(SwigluArgs), SwigluArgs &a, const moe_dims &d,
                         const uint16_t *bank, const int64_t *bank_offsets, const int32_t *bfill,
                         int64_t n_bank_rows, const uint16_t *wg, const uint16_t *wu, uint16_t *H,
                         float *part, hipStream_t s, int32_t *queue = nullptr) {
  a.A = bank;
  a.lda = d.latent;
  a.ktiles = d.latent / GBK;
  a.Bg = wg;
  a.Bu = wu;
  a.ldb = d.latent;
  a.F = d.d_ff;
  a.ftiles = d.d_ff / 128;
  a.H = H;
  a.ldh = d.d_ff;
  a.grp = group_args(d, bank_offsets, bfill, n_bank_rows, std::max(d.latent, d.d_ff));
  if (((uintptr_t)H & 15) || (a.ldh & 7)) return fail(MOE_ERR_INVALID, "%s: H rows not 16-byte aligned", name);
  return grouped(name, tail_name, k, tk, grouped_tiles_bound(d, n_bank_rows, a.ftiles), a.ktiles,
                 a, part, s, a.dH == nullptr, queue, queue ? queue + 64 : nullptr);
}

int64_t gemm_queue_bytes() { return GQ_BYTES; }

int gemm_expert_swiglu(const moe_dims &d, const uint16_t *bank, const int64_t *bank_offsets,
                       const int32_t *bfill, int64_t n_bank_rows, const uint16_t *wg,
                       const uint16_t *wu, uint16_t *H, float *part, int32_t *queue,
                       hipStream_t s) {
  SwigluArgs a{};
  return expert_swiglu("gemm_expert_swiglu", "gemm_expert_swiglu_tail",
                       gemm_expert_swiglu_kernel<false>, gemm_expert_swiglu_tail_kernel<false>, a,
                       d, bank, bank_offsets, bfill, n_bank_rows, wg, wu, H, part, s, queue);
}

int gemm_expert_swiglu_bwd(const moe_dims &d, const uint16_t *bank, const int64_t *bank_offsets,
                           const int32_t *bfill, int64_t n_bank_rows, const uint16_t *wg,
                           const uint16_t *wu,
                           const uint16_t *dH, uint16_t *H, uint16_t *AB, float *part,
                           hipStream_t s, uint16_t *HT, uint16_t *ABT, int64_t ldt, bool kpack,
                           bool *transposed) {
  SwigluArgs a{};
  a.dH = dH;
  a.ld_dh = d.d_ff;
  a.AB = AB;
  a.ld_ab = 2ll * d.d_ff;
  a.ab_off = d.d_ff;
  // transposed outputs: one product group per local expert (merged waves),
  // 8-byte aligned rows
  const GroupArgs ga = group_args(d, bank_offsets, bfill, n_bank_rows, std::max(d.latent, d.d_ff));
  const bool tr = HT && ABT && ga.nw == d.n_waves && ldt % 4 == 0 &&
                  (((uintptr_t)HT | (uintptr_t)ABT | (uintptr_t)H | (uintptr_t)AB |
                    (uintptr_t)dH) & 7) == 0;
  a.HT = tr ? HT : nullptr;
  a.ABT = tr ? ABT : nullptr;
  a.ldt = ldt;
  a.kpack = kpack;
  if (transposed) *transposed = tr;
  return expert_swiglu("gemm_expert_swiglu_bwd", "gemm_expert_swiglu_bwd_tail",
                       gemm_expert_swiglu_kernel<true>, gemm_expert_swiglu_tail_kernel<true>, a,
                       d, bank, bank_offsets, bfill, n_bank_rows, wg, wu, H, part, s);
}

// out[dst[r]] = bf16(A[r] . B_j^T) for the bank rows r of every group (w, j):
// A [bank rows][K], B [E_l][N][K]; dst rows < 0 or >= n_out are not stored.
static int grouped_nt(const char *name, const char *tail_name, const moe_dims &d,
                      const uint16_t *A, int K, const int64_t *bank_offsets, const int32_t *bfill,
                      const int32_t *dst, int64_t n_bank_rows, const uint16_t *B, int N,
                      uint16_t *out, int64_t n_out, float *part, hipStream_t s,
                      int32_t *queue = nullptr) {
  if (K % GBK) return fail(MOE_ERR_UNSUPPORTED, "%s: K %% %d != 0", name, GBK);
  DownArgs a{};
  a.n_ret = n_out;
  a.H = A;
  a.F = K;
  a.ktiles = K / GBK;
  a.Wd = B;
  a.L = N;
  a.tn = (int)cdiv(N, GBN);
  a.grp = group_args(d, bank_offsets, bfill, n_bank_rows, std::max(K, N));
  a.bank_src = dst;
  a.ret = out;
  if (((uintptr_t)out & 15) || (N & 7)) return fail(MOE_ERR_INVALID, "%s: output rows not 16-byte aligned", name);
  return grouped(name, tail_name, gemm_expert_down_kernel, gemm_expert_down_tail_kernel,
                 grouped_tiles_bound(d, n_bank_rows, a.tn), a.ktiles, a, part, s, true,
                 queue ? queue + 8 : nullptr, queue ? queue + 64 : nullptr);
}

int gemm_expert_down(const moe_dims &d, const uint16_t *H, const int64_t *bank_offsets,
                     const int32_t *bfill, const int32_t *bank_src, int64_t n_bank_rows,
                     const uint16_t *wd, uint16_t *ret, int64_t n_ret, float *part,
                     int32_t *queue, hipStream_t s) {
  return grouped_nt("gemm_expert_down", "gemm_expert_down_tail", d, H, d.d_ff, bank_offsets, bfill,
                    bank_src, n_bank_rows, wd, d.latent, ret, n_ret, part, s, queue);
}

int gemm_grouped_nt(const char *name, const char *tail_name, const moe_dims &d,
                    const uint16_t *A, int K, const int64_t *bank_offsets, const int32_t *bfill,
                    const int32_t *dst, int64_t n_bank_rows, const uint16_t *B, int N,
                    uint16_t *out, int64_t n_out, float *part, int32_t *queue, hipStream_t s) {
  return grouped_nt(name, tail_name, d, A, K, bank_offsets, bfill, dst, n_bank_rows, B, N, out,
                    n_out, part, s, queue);
}

int gemm_nt(const char *name, const char *tail_name, int M, int N, int nseg,
            const DenseSeg *segs, uint16_t *C, int64_t ldc, float *part, hipStream_t s) {
  static void (*const k[2])(DenseArgs) = {gemm_nt_kernel<1, false>, gemm_nt_kernel<2, false>};
  if (nseg < 1 || nseg > 2) return fail(MOE_ERR_INVALID, "%s: bad segment count", name);
  return dense(name, tail_name, k[nseg - 1], M, N, nseg, segs, C, ldc, part, s, true);
}

int gemm_nt_multi(const char *name, const char *tail_name, int nprod, const NtProd *prods, int K,
                  float *part, hipStream_t s, const int32_t *kfill, int kW, int kEl, bool kpack) {
  if (nprod < 1 || nprod > GMAXPROD) return fail(MOE_ERR_INVALID, "%s: bad product count", name);
  if (K % GBK) return fail(MOE_ERR_UNSUPPORTED, "%s: K %% %d != 0", name, GBK);
  MultiArgs a{};
  a.nprod = nprod;
  a.ktiles = K / GBK;
  a.kfill = kfill;
  a.kW = kW;
  a.kEl = kEl;
  a.kpack = kpack && kfill ? 1 : 0;
  int64_t total = 0;
  for (int p = 0; p < nprod; ++p) {
    const NtProd &q = prods[p];
    if (q.M < 1 || q.N < 1 || q.lda * 2 * GBM > INT32_MAX || q.ldb * 2 * GBN > INT32_MAX)
      return fail(MOE_ERR_UNSUPPORTED, "%s: product %d shape", name, p);
    a.first[p] = (int)total;
    a.A[p] = q.A;
    a.B[p] = q.B;
    a.C[p] = q.C;
    a.lda[p] = q.lda;
    a.ldb[p] = q.ldb;
    a.ldc[p] = q.ldc;
    a.M[p] = q.M;
    a.N[p] = q.N;
    a.kgroup[p] = q.kgroup;
    total += cdiv(q.M, GBM) * cdiv(q.N, GBN);
  }
  if (total > INT32_MAX / 2) return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", name);
  a.first[nprod] = (int)total;
  MOE_TRY(make_split(part, a.ktiles, a.sp));
  const int S = split_parts(a.sp, total);
  if (S == 1) {
    a.sp.part = nullptr;
    return launch(name, gemm_nt_multi_kernel, dim3((unsigned)total), dim3(GNT), 0, s, a);
  }
  const int64_t r = total % a.sp.ncu;
  MOE_TRY(launch(name, gemm_nt_multi_kernel, dim3((unsigned)(total - r + r * S)), dim3(GNT), 0, s,
                 a));
  return launch(tail_name, gemm_nt_multi_tail_kernel, dim3((unsigned)(r * GTM)), dim3(GNT), 0, s,
                a);
}

int gemm_nt_batched(const char *name, const char *tail_name, int M, int N, const DenseSeg &seg,
                    int nbatch, int64_t bsA, int64_t bsB, uint16_t *C, int64_t ldc, int64_t bsC,
                    float *part, hipStream_t s) {
  if (nbatch == 1) return gemm_nt(name, tail_name, M, N, 1, &seg, C, ldc, part, s);
  return dense(name, tail_name, gemm_nt_kernel<1, true>, M, N, 1, &seg, C, ldc, part, s, true,
               nbatch, bsA, bsB, bsC);
}

}  // namespace moe
