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
#include "gemm.h"
#include "kernels.h"

namespace moe {

constexpr int MAXSEG = GMAXSEG;

struct DenseArgs {
  int M, N, nseg;
  const uint16_t *A[MAXSEG];
  int64_t lda[MAXSEG];
  const uint16_t *B[MAXSEG];
  int64_t ldb[MAXSEG];
  int ktiles[MAXSEG];
  uint16_t *C;
  int64_t ldc;
};

__device__ __forceinline__ void dense_store(const DenseArgs &g, int mt, int nt, const GAcc &acc) {
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int j = 0; j < GTN; ++j) {
      const int n = nt * GBN + g_acc_col(j);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = mt * GBM + g_acc_row(i, v);
        if (m < g.M && n < g.N) g.C[(int64_t)m * g.ldc + n] = f32_to_bf16(acc[i][j][v]);
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

// NS: number of K segments (one K range, one rounding).
template <int NS>
__device__ __forceinline__ void dense_body(const DenseArgs &g, const GemmLds &lds) {
  const int tm = (g.M + GBM - 1) / GBM, tn = (g.N + GBN - 1) / GBN;
  int mt, nt;
  g_tile_coords(xcd_remap(blockIdx.x, gridDim.x), tm, tn, mt, nt);
  const int mv = g.M - mt * GBM, nv = g.N - nt * GBN;  // valid rows / columns
  const auto row_a = [&](int r) { return min(r, mv - 1); };
  const auto row_b = [&](int r) { return min(r, nv - 1); };
  GAcc acc;
  gemm_zero(acc);
  if constexpr (NS == 1) {
    const auto ops = g_operands(g.A[0] + (int64_t)mt * GBM * g.lda[0], g.lda[0], row_a,
                                g.B[0] + (int64_t)nt * GBN * g.ldb[0], g.ldb[0], row_b);
    gemm_mainloop(ops, g.ktiles[0], acc, lds);
  } else {
    GOps<GSegOperand<GCA, NS>, GSegOperand<GCB, NS>> ops;
    int kend = 0;
    dense_segs<0>(g, mt, nt, row_a, row_b, kend, ops);
    gemm_mainloop(ops, kend, acc, lds);
  }
  dense_store(g, mt, nt, acc);
}

__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_latent_down_kernel(DenseArgs g) {
  MOE_GEMM_LDS(lds);
  dense_body<1>(g, lds);
}

// up-projection + shared experts: 1 + S segments
template <int NS>
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_up_shared_kernel(DenseArgs g) {
  MOE_GEMM_LDS(lds);
  dense_body<NS>(g, lds);
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

// This block's tile: product groups in order, each contributing
// ceil(rows / 256) * tn tiles.  The grid is an upper bound; the real count
// is known only here, so blocks remap over it (each XCD gets a contiguous
// range of real tiles) and blocks past it exit (returns false).
__device__ __forceinline__ bool group_tile(const GroupArgs &a, int tn, GTile &t) {
  const int npg = a.G / a.nw;
  int total = 0;
  for (int pg = 0; pg < npg; ++pg) total += ((group_rows(a, pg) + GBM - 1) / GBM) * tn;
  if ((int)blockIdx.x >= total) return false;
  int rem = xcd_remap(blockIdx.x, total);
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
      return true;
    }
    rem -= tmg * tn;
  }
  return false;
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
  // dense (shared experts): M rows, expert = f-tile / ftiles along N
  int M, S;
  // grouped (routed experts)
  GroupArgs grp;
};

// row_of(m): row of A and H for tile row m < rows (contiguous rows, or the
// bank rows of a grouped tile).
template <class RowOf>
__device__ __forceinline__ void swiglu_tile(const SwigluArgs &g, RowOf row_of, int rows, int expert,
                                            int ft, int h_col0, const GemmLds &lds) {
  const int f0 = ft * 128;
  const int64_t eoff = (int64_t)expert * g.F * g.ldb + (int64_t)f0 * g.ldb;
  // whether a thread copies gate or up rows depends on the thread only (its
  // copy rows are 64 apart, g_swiglu_brow sees row % 64), so the base stays
  // wave-uniform
  bool up;
  int foff;
  g_swiglu_brow(g_load_row(0), up, foff);
  const int64_t r0 = row_of(0);
  const auto ops = g_operands(
      g.A + r0 * g.lda, g.lda, [&](int r) { return (int)(row_of(min(r, rows - 1)) - r0); },
      (up ? g.Bu : g.Bg) + eoff, g.ldb, [&](int r) {
        bool u;
        int f;
        g_swiglu_brow(r, u, f);
        return f;
      });
  GAcc acc;
  gemm_zero(acc);
  gemm_mainloop(ops, g.ktiles, acc, lds);
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = g_acc_row(i, v);
      if (m >= rows) continue;
      uint16_t *h = g.H + row_of(m) * g.ldh + h_col0 + f0;
#pragma unroll
      for (int p = 0; p < GTN / 2; ++p) {
        const float a = acc[i][2 * p][v], b = acc[i][2 * p + 1][v];
        h[g_swiglu_col(p)] = f32_to_bf16(silu_f32(a) * b);
      }
    }
}

__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_shared_swiglu_kernel(SwigluArgs g) {
  MOE_GEMM_LDS(lds);
  const int tm = (g.M + GBM - 1) / GBM, tn = g.S * g.ftiles;
  int mt, nt;
  g_tile_coords(xcd_remap(blockIdx.x, gridDim.x), tm, tn, mt, nt);
  const int s = nt / g.ftiles, ft = nt % g.ftiles;
  const int64_t row0 = (int64_t)mt * GBM;
  swiglu_tile(g, [&](int m) { return row0 + m; }, min(GBM, g.M - mt * GBM), s, ft, s * g.F, lds);
}

__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_expert_swiglu_kernel(SwigluArgs g) {
  MOE_GEMM_LDS(lds);
  GTile t;
  if (!group_tile(g.grp, g.ftiles, t)) return;
  swiglu_tile(g, [&](int m) { return t.row(m); }, t.rows, t.expert, t.nt, 0, lds);
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
};

__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(GMINWAVES, GMINWAVES))) void gemm_expert_down_kernel(DownArgs g) {
  MOE_GEMM_LDS(lds);
  GTile t;
  if (!group_tile(g.grp, g.tn, t)) return;
  const uint16_t *W = g.Wd + (int64_t)t.expert * g.L * g.F;
  const int nv = g.L - t.nt * GBN, rows = t.rows;
  const int64_t r0 = t.row(0);
  // receive row of tile row threadIdx.x: fetched before the main loop (its
  // latency hides there), handed to the epilogue through LDS
  int32_t my_dst = -1;
  if ((int)threadIdx.x < rows) my_dst = g.bank_src[t.row(threadIdx.x)];
  const auto ops = g_operands(
      g.H + r0 * g.F, g.F, [&](int r) { return (int)(t.row(min(r, rows - 1)) - r0); },
      W + (int64_t)t.nt * GBN * g.F, g.F, [&](int r) { return min(r, nv - 1); });
  GAcc acc;
  gemm_zero(acc);
  gemm_mainloop(ops, g.ktiles, acc, lds);
  int32_t *dst_rows = reinterpret_cast<int32_t *>(lds.A[0]);
  __syncthreads();  // every wave is past its last fragment read of the ring
  if ((int)threadIdx.x < GBM) dst_rows[threadIdx.x] = my_dst;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < GTM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = g_acc_row(i, v);
      if (m >= rows) continue;
      const int64_t dr = dst_rows[m];
      if (dr < 0 || dr >= g.n_ret) continue;
      const int64_t dst = dr * g.L;
#pragma unroll
      for (int j = 0; j < GTN; ++j) {
        const int n = t.nt * GBN + g_acc_col(j);
        if (n < g.L) g.ret[dst + n] = f32_to_bf16(acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

static int dense(const char *name, void (*k)(DenseArgs), int M, int N, int nseg,
                 const DenseSeg *segs, uint16_t *C, int64_t ldc, hipStream_t s) {
  if (nseg < 1 || nseg > MAXSEG) return fail(MOE_ERR_INVALID, "%s: bad segment count", name);
  DenseArgs a{};
  a.M = M;
  a.N = N;
  a.nseg = nseg;
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
  const int64_t tiles = cdiv(M, GBM) * cdiv(N, GBN);
  return launch(name, k, dim3((unsigned)tiles), dim3(GNT), 0, s, a);
}

int gemm_latent_down(int M, int N, const DenseSeg &seg, uint16_t *C, int64_t ldc, hipStream_t s) {
  return dense("gemm_latent_down", gemm_latent_down_kernel, M, N, 1, &seg, C, ldc, s);
}

int gemm_up_shared(int M, int N, int nseg, const DenseSeg *segs, uint16_t *C, int64_t ldc,
                   hipStream_t s) {
  static void (*const k[MAXSEG])(DenseArgs) = {gemm_up_shared_kernel<1>, gemm_up_shared_kernel<2>,
                                               gemm_up_shared_kernel<3>, gemm_up_shared_kernel<4>,
                                               gemm_up_shared_kernel<5>};
  if (nseg < 1 || nseg > MAXSEG) return fail(MOE_ERR_INVALID, "gemm_up_shared: bad segment count");
  return dense("gemm_up_shared", k[nseg - 1], M, N, nseg, segs, C, ldc, s);
}

int gemm_shared_swiglu(int M, const uint16_t *x, int64_t ldx, int K, const uint16_t *wg,
                       const uint16_t *wu, int S, int F, uint16_t *H, hipStream_t s) {
  if (S == 0) return MOE_OK;
  SwigluArgs a{};
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
  const int64_t tiles = cdiv(M, GBM) * (int64_t)S * a.ftiles;
  return launch("gemm_shared_swiglu", gemm_shared_swiglu_kernel, dim3((unsigned)tiles), dim3(GNT),
                0, s, a);
}

// Product groups of the bank: each local expert over every wave when the
// merged rows stay within 32-bit copy offsets of a tile's first row, else
// every (wave, expert) group alone.
static GroupArgs group_args(const moe_dims &d, const int64_t *bank_offsets, const int32_t *bfill,
                            int64_t n_bank_rows) {
  GroupArgs g{};
  g.El = experts_per_rank(d);
  g.G = d.n_waves * g.El;
  g.cap = d.cap_recv;
  g.count = bfill;
  g.offsets = ragged(d) ? bank_offsets : nullptr;
  const int64_t width = d.latent > d.d_ff ? d.latent : d.d_ff;
  const bool merge = d.n_waves <= GMAXW && n_bank_rows * width * 2 < INT32_MAX;
  g.nw = merge ? d.n_waves : 1;
  return g;
}

static int64_t grouped_tiles_bound(const moe_dims &d, int64_t n_bank_rows, int tn) {
  const int64_t G = (int64_t)d.n_waves * experts_per_rank(d);
  const int64_t mt = ragged(d) ? cdiv(n_bank_rows, GBM) + G : G * cdiv(d.cap_recv, GBM);
  return mt * tn;
}

int gemm_expert_swiglu(const moe_dims &d, const uint16_t *bank, const int64_t *bank_offsets,
                       const int32_t *bfill, int64_t n_bank_rows, const uint16_t *wg,
                       const uint16_t *wu, uint16_t *H, hipStream_t s) {
  SwigluArgs a{};
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
  a.grp = group_args(d, bank_offsets, bfill, n_bank_rows);
  const int64_t tiles = grouped_tiles_bound(d, n_bank_rows, a.ftiles);
  return launch("gemm_expert_swiglu", gemm_expert_swiglu_kernel, dim3((unsigned)tiles), dim3(GNT),
                0, s, a);
}

int gemm_expert_down(const moe_dims &d, const uint16_t *H, const int64_t *bank_offsets,
                     const int32_t *bfill, const int32_t *bank_src, int64_t n_bank_rows,
                     const uint16_t *wd, uint16_t *ret, int64_t n_ret, hipStream_t s) {
  DownArgs a{};
  a.n_ret = n_ret;
  a.H = H;
  a.F = d.d_ff;
  a.ktiles = d.d_ff / GBK;
  a.Wd = wd;
  a.L = d.latent;
  a.tn = (int)cdiv(d.latent, GBN);
  a.grp = group_args(d, bank_offsets, bfill, n_bank_rows);
  a.bank_src = bank_src;
  a.ret = ret;
  const int64_t tiles = grouped_tiles_bound(d, n_bank_rows, a.tn);
  return launch("gemm_expert_down", gemm_expert_down_kernel, dim3((unsigned)tiles), dim3(GNT), 0,
                s, a);
}

}  // namespace moe
