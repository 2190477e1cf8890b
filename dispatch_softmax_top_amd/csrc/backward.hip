// backward.hip -- gradients of the branch (fixed capacities or ragged), for training:
// "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK) describes a
// model in open training; its pages give the forward pass, and every
// gradient here follows from the forward definitions by the chain rule.
//
// Rounding points: gradients are stored like the values they belong to
// (bf16 activations and weights, fp32 gates and logits); a, b = u.W_g,
// u.W_u are recomputed from the forward inputs by the forward's own GEMMs.
//
// Every contraction runs on the forward's bf16 MFMA engine, which takes both
// operands K-contiguous (C = A . B^T).  Weight gradients (a sum over tokens
// or bank rows) and input gradients through a weight stored output-major need
// the other operand orders; they get them from 64x64 LDS-tiled transposes
// into the workspace (HBM-bound copies, two to four per launch).
//
// Calls and kernels, in stream order:
//   moe_combine_backward  transposes of W_lu, W_sd; [d_ylat | d_h_s] =
//                         d_out . [W_lu ; W_sd]; shared experts recomputed
//                         with the SwiGLU gradient epilogue (d_shared, h_s);
//                         combine_backward (d_returned, d_gates, zero rows);
//                         transposes of d_out, ylat, h_s; dW_lu, dW_sd
//   moe_expert_ffn_backward  transposes of W_d, [W_g | W_u]; gather of the
//                         return gradients into bank order; d_h (grouped);
//                         experts recomputed with the gradient epilogue
//                         (d_a | d_b, h); d_u scattered to receive rows
//                         (grouped); bank-order transposes; dW_d, dW_g, dW_u
//                         (batched over the local experts)
//   moe_pack_backward     dz (gather-sum of the pool-row gradients);
//                         transposes of W_ld, W_sg, W_su; dx = [dz | d_shared]
//                         . [W_ld ; W_sg ; W_su]; transposes of x, dz,
//                         d_shared; dW_ld, dW_sg, dW_su
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// transpose: out[b][c][k] = in(b, row(b, k))[c] for c < cols, k < kpad, and 0
// where row(b, k) does not exist.  Plain: row = k for k < rows.  Bank order
// (bfill != NULL): the filled bank positions of local expert b, wave after
// wave, packed: k = (fills of the waves before w) + p is bank slot (wave w,
// expert b, position p < bfill[w * El + b]); k past the expert's total fill
// has no row.  Ragged bank order (boff != NULL, one batch): every expert's
// range in one row of out, expert b from the sum of kpack_len(rows of the
// experts before b) on, and bank slot (w, b, p) at boff[w * El + b] + p.
// ---------------------------------------------------------------------------

struct TransposeArgs {
  const uint16_t *in;
  int64_t ld_in, bs_in;
  uint16_t *out;
  int64_t ld_out, bs_out;
  int rows, cols, kpad;
  const int32_t *bfill;
  int cap, El, W;
  const int64_t *boff;
};

// Bank row of packed column k (ragged bank order), or -1.
__device__ __forceinline__ int64_t tp_ragged_row(const TransposeArgs &a, int k) {
  int64_t base = 0;
  for (int b = 0; b < a.El; ++b) {
    int rows = 0;
    for (int w = 0; w < a.W; ++w) rows += a.bfill[w * a.El + b];
    const int64_t len = kpack_len(rows);
    if (k < base + len) {
      int kk = (int)(k - base);
      if (kk >= rows) return -1;
      for (int w = 0; w < a.W; ++w) {
        const int f = a.bfill[w * a.El + b];
        if (kk < f) return a.boff[w * a.El + b] + kk;
        kk -= f;
      }
      return -1;
    }
    base += len;
  }
  return -1;
}

constexpr int TP = 64;  // tile edge

// The tile is [k][c] with 128-byte rows; 16-byte chunk ch of row kk sits at
// chunk ch ^ (kk / 8 % 8), so the column reads of the second phase (rows
// 8 apart, one per lane group) fall on different banks.
__device__ __forceinline__ int tp_chunk(int kk, int ch) { return ch ^ ((kk >> 3) & 7); }

// Up to four transposes in one launch (one ramp-up and drain for all):
// blocks first[i] .. first[i+1]-1 belong to transpose i, laid out as its
// (k tile, c tile, batch) grid.
constexpr int TMAX = 4;
struct TransposeBatch {
  int n;
  int first[TMAX + 1];
  int gk[TMAX], gc[TMAX];  // k tiles and c tiles of each
  TransposeArgs t[TMAX];
};

__global__ __launch_bounds__(256) void transpose_kernel(TransposeBatch tb) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TP][TP];
  int i = 0;
  while (i + 1 < tb.n && (int)blockIdx.x >= tb.first[i + 1]) ++i;
  const TransposeArgs &a = tb.t[i];
  const int l = (int)blockIdx.x - tb.first[i];
  const int k0 = (l % tb.gk[i]) * TP, c0 = (l / tb.gk[i] % tb.gc[i]) * TP;
  const int b = l / (tb.gk[i] * tb.gc[i]);
  const uint16_t *in = a.in + b * a.bs_in;
  for (int q = threadIdx.x; q < TP * TP / 8; q += 256) {
    const int kk = q >> 3, ch = q & 7;
    const int k = k0 + kk, c = c0 + ch * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k < a.kpad && c < a.cols && k < a.rows) {
      int64_t row = k;
      if (a.boff) {
        row = tp_ragged_row(a, k);
      } else if (a.bfill) {
        int base = 0, w = 0;
        for (; w < a.W; ++w) {
          const int f = a.bfill[w * a.El + b];
          if (k < base + f) break;
          base += f;
        }
        row = w < a.W ? (int64_t)(w * a.El + b) * a.cap + (k - base) : -1;
      }
      if (row >= 0) v = *reinterpret_cast<const u32x4 *>(in + row * a.ld_in + c);
    }
    *reinterpret_cast<u32x4 *>(&tile[kk][tp_chunk(kk, ch) * 8]) = v;
  }
  __syncthreads();
  uint16_t *out = a.out + b * a.bs_out;
  for (int q = threadIdx.x; q < TP * TP / 8; q += 256) {
    const int cc = q >> 3, ch = q & 7;
    const int c = c0 + cc, k = k0 + ch * 8;
    if (c >= a.cols || k >= a.kpad) continue;
    u32x4 v;
    const int cs = cc & 7;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int k_lo = ch * 8 + 2 * h, k_hi = k_lo + 1;
      v[h] = (uint32_t)tile[k_lo][tp_chunk(k_lo, cc >> 3) * 8 + cs] |
             ((uint32_t)tile[k_hi][tp_chunk(k_hi, cc >> 3) * 8 + cs] << 16);
    }
    *reinterpret_cast<u32x4 *>(out + (int64_t)c * a.ld_out + k) = v;
  }
}

// Host side: every size and stride a multiple of 8 elements, pointers 16-byte
// aligned (the callers' buffers and workspace offsets are).
struct Tr {
  const uint16_t *in;
  int64_t ld_in, bs_in;
  uint16_t *out;
  int64_t ld_out, bs_out;
  int rows, cols, kpad, nbatch;
  const int32_t *bfill;
  int cap, El, W;
  const int64_t *boff;
};

static int transposes(const char *name, int n, const Tr *tr, hipStream_t s) {
  if (n < 1 || n > TMAX) return fail(MOE_ERR_INVALID, "%s: bad transpose count", name);
  TransposeBatch tb{};
  tb.n = n;
  int64_t total = 0;
  for (int i = 0; i < n; ++i) {
    const Tr &q = tr[i];
    if (q.cols % 8 || q.kpad % 8 || q.ld_in % 8 || q.ld_out % 8 || q.bs_in % 8 || q.bs_out % 8)
      return fail(MOE_ERR_UNSUPPORTED, "%s: sizes must be multiples of 8", name);
    tb.t[i] = TransposeArgs{q.in,   q.ld_in, q.bs_in, q.out, q.ld_out, q.bs_out, q.rows,
                            q.cols, q.kpad,  q.bfill, q.cap, q.El,   q.W,      q.boff};
    tb.gk[i] = (int)cdiv(q.kpad, TP);
    tb.gc[i] = (int)cdiv(q.cols, TP);
    tb.first[i] = (int)total;
    total += (int64_t)tb.gk[i] * tb.gc[i] * q.nbatch;
  }
  if (total >= INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: too many tiles", name);
  tb.first[n] = (int)total;
  return launch(name, transpose_kernel, dim3((unsigned)total), dim3(256), 0, s, tb);
}

// ---------------------------------------------------------------------------
// combine side: one wave per token.  For each kept choice j (pool row r):
//   d_returned[r] = bf16(g[t,j] * d_ylat[t]),  d_gates[t,j] = returned[r] . d_ylat[t]
// (fp32, lane partial sums then a wave sum); dropped choices get d_gates 0.
// Ragged (offsets != NULL): pool row = offsets[seg] + slot, and a slot at or
// past its segment's length has no row (d_gates 0).  Extra blocks: one wave
// per returned row, zeroing rows past their pool's fill (the own shard's
// slots of a pool are 0 .. fill - 1).
// ---------------------------------------------------------------------------

template <int CH>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const uint16_t *__restrict__ returned, const int64_t *__restrict__ offsets, int n_seg,
    const uint16_t *__restrict__ dy, int64_t ld_dy,
    const int32_t *__restrict__ topk, const int32_t *__restrict__ slot,
    const float *__restrict__ gates, const int32_t *__restrict__ fill,
    uint16_t *__restrict__ d_returned, float *__restrict__ d_gates, int T, int k, int L, int El,
    int Wk, int Tw, int pool_rows, int cap, int token_blocks, int64_t n_slots) {
  const int lane = lane_id();
  const int nch = L / 8;
  if ((int)blockIdx.x >= token_blocks) {
    const int64_t idx = (int64_t)(blockIdx.x - token_blocks) * 4 + (threadIdx.x >> 6);
    if (idx >= n_slots) return;
    int p, i;
    if (offsets) {  // last segment starting at or before idx
      int lo = 0, hi = n_seg - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= idx) lo = mid;
        else hi = mid - 1;
      }
      p = lo;
      i = (int)(idx - offsets[p]);
    } else {
      p = (int)(idx / cap);
      i = (int)(idx - (int64_t)p * cap);
    }
    if (i < fill[p]) return;
    u32x4 *o = reinterpret_cast<u32x4 *>(d_returned + idx * L);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int c = lane; c < nch; c += 64) o[c] = zero;
    return;
  }
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int64_t my_row = -1;
  float my_g = 0.f;
  if (lane < k) {
    const int s = slot[(int64_t)t * k + lane];
    const int e = topk[(int64_t)t * k + lane];
    const float g = gates[(int64_t)t * k + lane];
    if (s >= 0) {
      const int seg = (e / El) * Wk + t / Tw;
      if (!offsets) my_row = (int64_t)seg * pool_rows + s;
      else if (s < offsets[seg + 1] - offsets[seg]) my_row = offsets[seg] + s;
      my_g = g;
    }
  }
  const u32x4 *src = reinterpret_cast<const u32x4 *>(dy + (int64_t)t * ld_dy);
  u32x4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = src[min(lane + 64 * c, nch - 1)];
  float my_dg = 0.f;
  const u32x4 *ret16 = reinterpret_cast<const u32x4 *>(returned);
  u32x4 *dret16 = reinterpret_cast<u32x4 *>(d_returned);
  uint64_t valid = ballot(my_row >= 0);
  while (valid) {
    const int j = (int)__builtin_ctzll(valid);
    valid &= valid - 1;
    const int64_t row = ((int64_t)__shfl((int)(my_row >> 32), j) << 32) |
                        (uint32_t)__shfl((int)my_row, j);
    const float g = __shfl(my_g, j);
    u32x4 r[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) r[c] = ld16<true>(ret16 + row * nch + min(lane + 64 * c, nch - 1));
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lane + 64 * c >= nch) continue;
      u32x4 o;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float y0 = __uint_as_float(v[c][h] << 16),
                                         y1 = __uint_as_float(v[c][h] & 0xffff0000u);
        dot = fmaf(__uint_as_float(r[c][h] << 16), y0, dot);
        dot = fmaf(__uint_as_float(r[c][h] & 0xffff0000u), y1, dot);
        o[h] = pack_bf16x2(g * y0, g * y1);
      }
      dret16[row * nch + lane + 64 * c] = o;
    }
    dot = wave_sum_f32(dot);
    if (lane == j) my_dg = dot;
  }
  if (lane < k) d_gates[(int64_t)t * k + lane] = my_dg;
}

// ---------------------------------------------------------------------------
// bank order: out[r] = in[src[r]] (latent-wide rows) for every bank row with
// src[r] >= 0; other rows are left as they are (nothing reads them).  One wave
// per row, the whole row in flight.
// ---------------------------------------------------------------------------

template <int CH>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ in,
                                                          int64_t n_in,
                                                          const int32_t *__restrict__ src,
                                                          int64_t n, uint16_t *__restrict__ out,
                                                          int L) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int sr = src[r];
  if (sr < 0 || sr >= n_in) return;
  const int lane = lane_id(), nch = L / 8;
  const u32x4 *a = reinterpret_cast<const u32x4 *>(in + (int64_t)sr * L);
  u32x4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = ld16<true>(a + min(lane + 64 * c, nch - 1));
  u32x4 *o = reinterpret_cast<u32x4 *>(out + r * L);
#pragma unroll
  for (int c = 0; c < CH; ++c)
    if (lane + 64 * c < nch) o[lane + 64 * c] = v[c];
}

// The transposed bank-order operands the backward SwiGLU writes directly
// (HT [F rows], ABT [2F rows] per expert block, or one block of packed expert
// ranges with kpack): an expert with no filled rows has no tile there, yet
// the weight gradients read its first kz = min(256, K columns) columns, which
// are zeroed here.  Block: 4 rows of one expert, 64 threads per row.
__global__ __launch_bounds__(256) void zero_empty_k_kernel(uint16_t *HT, uint16_t *ABT,
                                                           int64_t ldt, int F, int El, int W,
                                                           const int32_t *__restrict__ bfill,
                                                           int kpack, int kz) {
  const int per = 3 * F / 4;
  const int e = (int)(blockIdx.x / per), r = (int)(blockIdx.x % per) * 4 + (int)(threadIdx.x >> 6);
  int fill = 0;
  for (int w = 0; w < W; ++w) fill += bfill[w * El + e];
  if (fill) return;
  int64_t kb = 0;
  if (kpack)
    for (int x = 0; x < e; ++x) {
      int f = 0;
      for (int w = 0; w < W; ++w) f += bfill[w * El + x];
      kb += kpack_len(f);
    }
  uint16_t *row = r < F ? (kpack ? HT : HT + (int64_t)e * F * ldt) + (int64_t)r * ldt
                        : (kpack ? ABT : ABT + (int64_t)e * 2 * F * ldt) + (int64_t)(r - F) * ldt;
  const u32x2 zero = {0u, 0u};
  for (int k = (int)(threadIdx.x & 63) * 4; k < kz; k += 256)
    *reinterpret_cast<u32x2 *>(row + kb + k) = zero;
}

// o[i] = i; zero16: NULL, or 16 ints set to zero (a GEMM work queue's counters).
__global__ __launch_bounds__(256) void iota_kernel(int32_t *o, int64_t n, int32_t *zero16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) o[i] = (int32_t)i;
  if (zero16 && i < 16) zero16[i] = 0;
}

// Dispatch on the 16-byte chunks per lane a latent row needs (latent <= 8192).
template <class F>
static int by_chunks(int L, F f) {
  const int ch = (int)cdiv(L / 8, 64);
  if (ch <= 1) return f(std::integral_constant<int, 1>());
  if (ch <= 2) return f(std::integral_constant<int, 2>());
  if (ch <= 4) return f(std::integral_constant<int, 4>());
  if (ch <= 6) return f(std::integral_constant<int, 6>());
  if (ch <= 8) return f(std::integral_constant<int, 8>());
  return f(std::integral_constant<int, 16>());
}

// ---------------------------------------------------------------------------
// workspace layouts
// ---------------------------------------------------------------------------

// Buffers carved from ws in order, each 256-byte aligned.
struct Carve {
  char *base;
  int64_t off = 0;
  template <class T>
  T *take(int64_t elems) {
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += align_up(elems * (int64_t)sizeof(T), 256);
    return p;
  }
};

inline int64_t pad32(int64_t n) { return align_up(n, 32); }

struct CombineBwdWs {
  uint16_t *Bt, *C1, *Hs, *doT, *ylT, *HsT;
  float *part;
};
static int64_t combine_bwd_ws(const moe_dims &d, char *base, CombineBwdWs &w) {
  const int64_t T = d.T, L = d.latent, D = d.d_model, SF = (int64_t)d.n_shared * d.d_ff_shared,
                Tp = pad32(T);
  Carve c{base};
  w.Bt = c.take<uint16_t>((L + SF) * D);
  w.C1 = c.take<uint16_t>(T * (L + SF));
  w.Hs = c.take<uint16_t>(T * SF);
  w.doT = c.take<uint16_t>(D * Tp);
  w.ylT = c.take<uint16_t>(L * Tp);
  w.HsT = c.take<uint16_t>(SF * Tp);
  w.part = c.take<float>(gemm_split_bytes() / 4);
  return c.off;
}

struct FfnBwdWs {
  uint16_t *WdT, *WguT, *dY, *dH, *Hb, *dAB, *dYT, *HT, *dABT, *UT;
  int32_t *iota, *flags, *queue;
  float *part;
};
// Bank rows and receive rows of the expert backward: fixed mode from the
// capacities; ragged mode n_rows both (the bank holds every received row).
static int64_t ffn_bwd_bank_rows(const moe_dims &d, int64_t n_rows) {
  return ragged(d) ? n_rows : (int64_t)d.n_waves * experts_per_rank(d) * d.cap_recv;
}
// K extent of the bank-order transposes: fixed, every expert's own block of
// pad32(W * cap_recv) columns; ragged, one row holding every expert's packed
// range (kpack_len of its rows), at most this many columns.
static int64_t ffn_bwd_kcols(const moe_dims &d, int64_t nb) {
  if (!ragged(d)) return pad32((int64_t)d.n_waves * d.cap_recv);
  return pad32(nb + (int64_t)experts_per_rank(d) * (256 + 32));
}
static int64_t ffn_bwd_ws(const moe_dims &d, int64_t n_rows, char *base, FfnBwdWs &w) {
  const int64_t El = experts_per_rank(d), L = d.latent, F = d.d_ff;
  const int64_t nb = ffn_bwd_bank_rows(d, n_rows);
  const int64_t nr = ragged(d) ? n_rows : (int64_t)d.n_ranks * d.n_waves * d.cap_send;
  const int64_t Kp = ffn_bwd_kcols(d, nb), blocks = ragged(d) ? 1 : El;
  Carve c{base};
  w.WdT = c.take<uint16_t>(El * F * L);
  w.WguT = c.take<uint16_t>(El * L * 2 * F);
  w.dY = c.take<uint16_t>(nb * L);
  w.dH = c.take<uint16_t>(nb * F);
  w.Hb = c.take<uint16_t>(nb * F);
  w.dAB = c.take<uint16_t>(nb * 2 * F);
  w.dYT = c.take<uint16_t>(blocks * L * Kp);
  w.HT = c.take<uint16_t>(blocks * F * Kp);
  w.dABT = c.take<uint16_t>(blocks * 2 * F * Kp);
  w.UT = c.take<uint16_t>(blocks * L * Kp);
  w.iota = c.take<int32_t>(nb);
  w.flags = c.take<int32_t>(nr);
  w.queue = c.take<int32_t>(gemm_queue_bytes() / 4);
  w.part = c.take<float>(gemm_split_bytes() / 4);
  return c.off;
}

struct PackBwdWs {
  uint16_t *BldT, *BsT, *xT, *dzT, *dshT;
  float *part;
};
static int64_t pack_bwd_ws(const moe_dims &d, char *base, PackBwdWs &w) {
  const int64_t L = d.latent, D = d.d_model, SF = (int64_t)d.n_shared * d.d_ff_shared,
                Tp = pad32(d.T);
  Carve c{base};
  w.BldT = c.take<uint16_t>(D * L);
  w.BsT = c.take<uint16_t>(D * 2 * SF);
  w.xT = c.take<uint16_t>(D * Tp);
  w.dzT = c.take<uint16_t>(L * Tp);
  w.dshT = c.take<uint16_t>(2 * SF * Tp);
  w.part = c.take<float>(gemm_split_bytes() / 4);
  return c.off;
}

int64_t bwd_ws_bytes(const moe_dims &d, int call, int64_t n_rows) {
  if (call == MOE_CALL_COMBINE_BWD) {
    CombineBwdWs w;
    return combine_bwd_ws(d, nullptr, w);
  }
  if (call == MOE_CALL_FFN_BWD) {
    FfnBwdWs w;
    return ffn_bwd_ws(d, n_rows, nullptr, w);
  }
  PackBwdWs w;
  return pack_bwd_ws(d, nullptr, w);
}

static int check_bwd(const moe_dims *d, int call, const char *name, const void *ws,
                     int64_t ws_bytes, int64_t n_rows = 0) {
  MOE_TRY(check_dims(d));
  if (d->dedup) return fail(MOE_ERR_UNSUPPORTED, "%s: no dedup", name);
  MOE_TRY(check_ptr(ws, "ws"));
  const int64_t need = bwd_ws_bytes(*d, call, n_rows);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %lld < %lld bytes", name, (long long)ws_bytes,
                (long long)need);
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_combine_backward(const moe_dims *d, const moe_bf16 *returned,
                                    const int64_t *ret_offsets, int64_t n_ret_rows,
                                    const int32_t *topk, const int32_t *slot, const float *gates,
                                    const int32_t *fill, const moe_bf16 *x, const moe_bf16 *ylat,
                                    const moe_bf16 *w_lat_up, const moe_bf16 *ws_gate,
                                    const moe_bf16 *ws_up, const moe_bf16 *ws_down,
                                    const moe_bf16 *d_out, moe_bf16 *d_returned, float *d_gates,
                                    moe_bf16 *d_shared, moe_bf16 *dw_lat_up, moe_bf16 *dws_down,
                                    void *ws, int64_t ws_bytes, void *stream) {
  clear_error();
  MOE_TRY(check_bwd(d, MOE_CALL_COMBINE_BWD, "moe_combine_backward", ws, ws_bytes));
  const bool sh = d->n_shared > 0;
  const void *need[] = {returned, topk, slot, gates, fill, x, ylat, w_lat_up, d_out, d_returned,
                        d_gates, dw_lat_up};
  const char *names[] = {"returned", "topk", "slot", "gates", "fill", "x", "ylat", "w_lat_up",
                         "d_out", "d_returned", "d_gates", "dw_lat_up"};
  for (int i = 0; i < 12; ++i) MOE_TRY(check_ptr(need[i], names[i]));
  if (sh) {
    MOE_TRY(check_ptr(ws_gate, "ws_gate"));
    MOE_TRY(check_ptr(ws_up, "ws_up"));
    MOE_TRY(check_ptr(ws_down, "ws_down"));
    MOE_TRY(check_ptr(d_shared, "d_shared"));
    MOE_TRY(check_ptr(dws_down, "dws_down"));
  }
  const bool rg = ragged(*d);
  if (rg) {
    MOE_TRY(check_ptr(ret_offsets, "ret_offsets (ragged mode)"));
    if (n_ret_rows < 0 || n_ret_rows >= (1ll << 31))
      return fail(MOE_ERR_INVALID, "moe_combine_backward: n_ret_rows out of range");
  } else if (n_ret_rows != (int64_t)d->n_ranks * d->n_waves * d->cap_send) {
    return fail(MOE_ERR_INVALID, "moe_combine_backward: fixed mode needs n_ret_rows == n_ranks*n_waves*cap_send");
  }
  hipStream_t s = (hipStream_t)stream;
  const int T = d->T, L = d->latent, D = d->d_model, S = d->n_shared, Fs = d->d_ff_shared;
  const int SF = S * Fs, Tp = (int)pad32(T);
  CombineBwdWs w;
  combine_bwd_ws(*d, (char *)ws, w);

  // [d_ylat | d_h_s] = d_out . [W_lu^T ; W_sd,s^T]^T, one product
  const Tr trw[2] = {{w_lat_up, L, 0, w.Bt, D, 0, D, L, D, 1},
                     {ws_down, Fs, (int64_t)D * Fs, w.Bt + (int64_t)L * D, D, (int64_t)Fs * D, D,
                      Fs, D, S}};
  MOE_TRY(transposes("transpose_combine_weights", sh ? 2 : 1, trw, s));
  DenseSeg g1{d_out, D, w.Bt, D, D};
  MOE_TRY(gemm_nt("gemm_bwd_d_ylat", "gemm_bwd_d_ylat_tail", T, L + SF, 1, &g1, w.C1, L + SF,
                  w.part, s));
  // shared experts: recompute, SwiGLU gradient -> d_shared, h_s
  if (sh)
    MOE_TRY(gemm_shared_swiglu_bwd(T, x, D, D, ws_gate, ws_up, S, Fs, w.C1, L + SF, L, w.Hs,
                                   d_shared, w.part, s));
  // routed part: d_returned, d_gates
  const PoolKey pk = pool_key(*d);
  const int token_blocks = (int)cdiv(T, 4);
  const int64_t n_slots = n_ret_rows;
  const int n_seg = d->n_ranks * d->n_waves;
  MOE_TRY(by_chunks(L, [&](auto chv) {
    constexpr int CH = decltype(chv)::value;
    return launch("combine_backward", combine_backward_kernel<CH>,
                  dim3((unsigned)(token_blocks + cdiv(n_slots, 4))), dim3(256), 0, s, returned,
                  rg ? ret_offsets : nullptr, n_seg, w.C1, (int64_t)(L + SF), topk, slot, gates,
                  fill, d_returned, d_gates, T, d->top_k, L, experts_per_rank(*d), pk.Wk, pk.Tw,
                  pk.rows, d->cap_send, token_blocks, n_slots);
  }));
  // weight gradients, summed over tokens
  const Tr tra[3] = {{d_out, D, 0, w.doT, Tp, 0, T, D, Tp, 1},
                     {ylat, L, 0, w.ylT, Tp, 0, T, L, Tp, 1},
                     {w.Hs, SF, 0, w.HsT, Tp, 0, T, SF, Tp, 1}};
  MOE_TRY(transposes("transpose_combine_acts", sh ? 3 : 2, tra, s));
  // dW_lu and every dW_sd,s: one launch of 1 + S products over K = tokens
  NtProd pr[1 + 4];
  pr[0] = NtProd{w.doT, Tp, w.ylT, Tp, dw_lat_up, L, D, L};
  for (int i = 0; i < S; ++i)
    pr[1 + i] = NtProd{w.doT, Tp, w.HsT + (int64_t)i * Fs * Tp, Tp, dws_down + (int64_t)i * D * Fs,
                       Fs, D, Fs};
  return gemm_nt_multi("gemm_bwd_dw_combine", "gemm_bwd_dw_combine_tail", sh ? 1 + S : 1, pr, Tp,
                       w.part, s);
}

extern "C" int moe_expert_ffn_backward(const moe_dims *d, const moe_bf16 *bank,
                                       const int64_t *bank_offsets, int64_t n_bank_rows,
                                       const int32_t *bank_src, const int32_t *bfill,
                                       const moe_bf16 *w_gate, const moe_bf16 *w_up,
                                       const moe_bf16 *w_down, const moe_bf16 *d_ret,
                                       int64_t n_ret_rows, moe_bf16 *d_recv, moe_bf16 *dw_gate,
                                       moe_bf16 *dw_up, moe_bf16 *dw_down, void *ws,
                                       int64_t ws_bytes, void *stream) {
  clear_error();
  MOE_TRY(check_dims(d));
  const bool rg = ragged(*d);
  const int El = experts_per_rank(*d), L = d->latent, F = d->d_ff, Cr = d->cap_recv;
  if (rg) {
    MOE_TRY(check_ptr(bank_offsets, "bank_offsets (ragged mode)"));
    if (n_bank_rows < 0 || n_bank_rows >= (1ll << 31) || n_ret_rows != n_bank_rows)
      return fail(MOE_ERR_INVALID, "moe_expert_ffn_backward: ragged mode needs n_ret_rows == n_bank_rows < 2^31");
  } else {
    if (n_bank_rows != (int64_t)d->n_waves * El * Cr ||
        n_ret_rows != (int64_t)d->n_ranks * d->n_waves * d->cap_send)
      return fail(MOE_ERR_INVALID, "moe_expert_ffn_backward: fixed mode needs n_bank_rows == n_waves*E_l*cap_recv and n_ret_rows == n_ranks*n_waves*cap_send");
    if ((int64_t)d->n_waves * Cr >= (1ll << 30))
      return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn_backward: bank rows >= 2^30");
  }
  MOE_TRY(check_bwd(d, MOE_CALL_FFN_BWD, "moe_expert_ffn_backward", ws, ws_bytes, n_bank_rows));
  const void *need[] = {bank, bank_src, bfill, w_gate, w_up, w_down, d_ret, d_recv, dw_gate,
                        dw_up, dw_down};
  const char *names[] = {"bank", "bank_src", "bfill", "w_gate", "w_up", "w_down", "d_ret",
                         "d_recv", "dw_gate", "dw_up", "dw_down"};
  for (int i = 0; i < 11; ++i) MOE_TRY(check_ptr(need[i], names[i]));
  hipStream_t s = (hipStream_t)stream;
  const int64_t nb = n_bank_rows, nr = n_ret_rows;
  const int64_t Kp = ffn_bwd_kcols(*d, nb);
  if (Kp >= (1ll << 31) - 256)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn_backward: bank rows too many");
  const int64_t *boff = rg ? bank_offsets : nullptr;
  FfnBwdWs w;
  ffn_bwd_ws(*d, nb, (char *)ws, w);
  const int64_t WL = (int64_t)F * L;

  // operands with K contiguous: W_d^T [El][F][L], [W_g^T | W_u^T] [El][L][2F]
  const Tr trw[3] = {{w_down, F, WL, w.WdT, L, WL, L, F, L, El},
                     {w_gate, L, WL, w.WguT, 2 * F, 2 * WL, F, L, F, El},
                     {w_up, L, WL, w.WguT + F, 2 * F, 2 * WL, F, L, F, El}};
  MOE_TRY(transposes("transpose_expert_weights", 3, trw, s));
  // dy in bank order
  MOE_TRY(by_chunks(L, [&](auto chv) {
    constexpr int CH = decltype(chv)::value;
    return launch("gather_bank_grad", gather_rows_kernel<CH>, dim3((unsigned)cdiv(nb, 4)),
                  dim3(256), 0, s, d_ret, nr, bank_src, nb, w.dY, L);
  }));
  // (the iota kernel also zeroes the grouped products' queue counters)
  MOE_TRY(launch("iota", iota_kernel, dim3((unsigned)std::max<int64_t>(cdiv(nb, 256), 1)),
                 dim3(256), 0, s, w.iota, nb, w.queue));
  // d_h = dy . W_d (grouped, bank order)
  MOE_TRY(gemm_grouped_nt("gemm_bwd_d_h", "gemm_bwd_d_h_tail", *d, w.dY, L, boff, bfill, w.iota,
                          nb, w.WdT, F, w.dH, nb, w.part, w.queue, s));
  // a, b recomputed; d_a | d_b and h (h, and d_a | d_b once more, straight
  // into the transposed bank-order layout when the product groups allow it)
  bool transposed = false;
  MOE_TRY(gemm_expert_swiglu_bwd(*d, bank, boff, bfill, nb, w_gate, w_up, w.dH, w.Hb, w.dAB,
                                 w.part, s, w.HT, w.dABT, Kp, rg, &transposed));
  if (transposed)
    MOE_TRY(launch("zero_empty_k", zero_empty_k_kernel, dim3((unsigned)(El * (3 * F / 4))),
                   dim3(256), 0, s, w.HT, w.dABT, Kp, F, El, d->n_waves, bfill, (int)rg,
                   (int)std::min<int64_t>(256, Kp)));
  // d_u = d_a . W_g + d_b . W_u, scattered to the receive rows; others zero
  MOE_TRY(ret_rows_mark(bank_src, nb, w.flags, nr, w.queue, s));
  MOE_TRY(gemm_grouped_nt("gemm_bwd_d_u", "gemm_bwd_d_u_tail", *d, w.dAB, 2 * F, boff, bfill,
                          bank_src, nb, w.WguT, L, d_recv, nr, w.part, w.queue, s));
  MOE_TRY(ret_rows_zero_unmarked(w.flags, d_recv, L, nr, s));
  // weight gradients: per local expert, summed over its rows of every wave.
  // Fixed: expert e's rows packed into its own block of Kp columns; ragged:
  // every expert's rows packed into one row of Kp columns, expert after expert.
  const int W = d->n_waves;
  const int nw = rg ? (int)Kp : W * Cr;
  const int nbatch = rg ? 1 : El;
  const Tr trb[4] = {
      {w.dY, L, 0, w.dYT, Kp, (int64_t)L * Kp, nw, L, (int)Kp, nbatch, bfill, Cr, El, W, boff},
      {bank, L, 0, w.UT, Kp, (int64_t)L * Kp, nw, L, (int)Kp, nbatch, bfill, Cr, El, W, boff},
      {w.Hb, F, 0, w.HT, Kp, (int64_t)F * Kp, nw, F, (int)Kp, nbatch, bfill, Cr, El, W, boff},
      {w.dAB, 2 * F, 0, w.dABT, Kp, (int64_t)2 * F * Kp, nw, 2 * F, (int)Kp, nbatch, bfill, Cr, El,
       W, boff}};
  MOE_TRY(transposes("transpose_bank", transposed ? 2 : 4, trb, s));
  // expert e's operand blocks: its own (fixed), or the shared row (ragged)
  const int64_t blk = rg ? 0 : 1;
  if (3 * El <= 18) {  // all three weights of every local expert in one launch
    NtProd pr[18];
    for (int e = 0; e < El; ++e) {
      const uint16_t *ab = w.dABT + blk * e * 2 * F * Kp, *ut = w.UT + blk * e * L * Kp;
      pr[3 * e] = NtProd{w.dYT + blk * e * L * Kp, Kp, w.HT + blk * e * F * Kp, Kp,
                         dw_down + e * WL, F, L, F, e};
      pr[3 * e + 1] = NtProd{ab, Kp, ut, Kp, dw_gate + e * WL, L, F, L, e};
      pr[3 * e + 2] = NtProd{ab + (int64_t)F * Kp, Kp, ut, Kp, dw_up + e * WL, L, F, L, e};
    }
    // each expert's K: its filled bank rows (the transposes packed them first)
    return gemm_nt_multi("gemm_bwd_dw_experts", "gemm_bwd_dw_experts_tail", 3 * El, pr, (int)Kp,
                         w.part, s, bfill, d->n_waves, El, rg);
  }
  if (rg)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn_backward: ragged mode needs E_l <= 6");
  DenseSeg gd{w.dYT, Kp, w.HT, Kp, (int)Kp};
  MOE_TRY(gemm_nt_batched("gemm_bwd_dw_down", "gemm_bwd_dw_down_tail", L, F, gd, El,
                          (int64_t)L * Kp, (int64_t)F * Kp,
                          dw_down, F, WL, w.part, s));
  DenseSeg gg{w.dABT, Kp, w.UT, Kp, (int)Kp};
  MOE_TRY(gemm_nt_batched("gemm_bwd_dw_gate", "gemm_bwd_dw_gate_tail", F, L, gg, El,
                          (int64_t)2 * F * Kp, (int64_t)L * Kp,
                          dw_gate, L, WL, w.part, s));
  DenseSeg gu{w.dABT + (int64_t)F * Kp, Kp, w.UT, Kp, (int)Kp};
  return gemm_nt_batched("gemm_bwd_dw_up", "gemm_bwd_dw_up_tail", F, L, gu, El,
                         (int64_t)2 * F * Kp, (int64_t)L * Kp,
                         dw_up, L, WL, w.part, s);
}

extern "C" int moe_pack_backward(const moe_dims *d, const moe_bf16 *d_pools,
                                 const int64_t *pool_offsets, const int32_t *topk,
                                 const int32_t *slot, const moe_bf16 *x,
                                 const moe_bf16 *d_shared, const moe_bf16 *w_lat_down,
                                 const moe_bf16 *ws_gate, const moe_bf16 *ws_up, moe_bf16 *dz,
                                 moe_bf16 *dx, moe_bf16 *dw_lat_down, moe_bf16 *dws_gate,
                                 moe_bf16 *dws_up, void *ws, int64_t ws_bytes, void *stream) {
  clear_error();
  MOE_TRY(check_bwd(d, MOE_CALL_PACK_BWD, "moe_pack_backward", ws, ws_bytes));
  const bool sh = d->n_shared > 0;
  const void *need[] = {d_pools, topk, slot, x, w_lat_down, dz, dx, dw_lat_down};
  const char *names[] = {"d_pools", "topk", "slot", "x", "w_lat_down", "dz", "dx", "dw_lat_down"};
  for (int i = 0; i < 8; ++i) MOE_TRY(check_ptr(need[i], names[i]));
  if (sh) {
    MOE_TRY(check_ptr(d_shared, "d_shared"));
    MOE_TRY(check_ptr(ws_gate, "ws_gate"));
    MOE_TRY(check_ptr(ws_up, "ws_up"));
    MOE_TRY(check_ptr(dws_gate, "dws_gate"));
    MOE_TRY(check_ptr(dws_up, "dws_up"));
  }
  hipStream_t s = (hipStream_t)stream;
  const int T = d->T, L = d->latent, D = d->d_model, SF = d->n_shared * d->d_ff_shared;
  const int Tp = (int)pad32(T);
  PackBwdWs w;
  pack_bwd_ws(*d, (char *)ws, w);

  // dz[t] = sum over kept choices of the pool-row gradients (the pack copy's
  // adjoint); ragged: segments at pool_offsets, a slot past its segment adds 0
  const bool rg = ragged(*d);
  if (rg) MOE_TRY(check_ptr(pool_offsets, "pool_offsets (ragged mode)"));
  MOE_TRY(combine_gather_rows(*d, d_pools, rg ? pool_offsets : nullptr, topk, slot, nullptr, dz,
                              s));
  // dx = dz . W_ld + d_a . W_sg + d_b . W_su, one product with one rounding
  DenseSeg gx[2] = {{dz, L, w.BldT, L, L}, {d_shared, 2 * SF, w.BsT, 2 * SF, 2 * SF}};
  const Tr trw[3] = {{w_lat_down, D, 0, w.BldT, L, 0, L, D, L, 1},
                     {ws_gate, D, 0, w.BsT, 2 * SF, 0, SF, D, SF, 1},
                     {ws_up, D, 0, w.BsT + SF, 2 * SF, 0, SF, D, SF, 1}};
  MOE_TRY(transposes("transpose_pack_weights", sh ? 3 : 1, trw, s));
  MOE_TRY(gemm_nt("gemm_bwd_dx", "gemm_bwd_dx_tail", T, D, sh ? 2 : 1, gx, dx, D, w.part, s));
  // weight gradients, summed over tokens
  const Tr tra[3] = {{x, D, 0, w.xT, Tp, 0, T, D, Tp, 1},
                     {dz, L, 0, w.dzT, Tp, 0, T, L, Tp, 1},
                     {d_shared, 2 * SF, 0, w.dshT, Tp, 0, T, 2 * SF, Tp, 1}};
  MOE_TRY(transposes("transpose_pack_acts", sh ? 3 : 2, tra, s));
  // dW_ld, dW_sg, dW_su: one launch of three products over K = tokens
  NtProd pr[3] = {{w.dzT, Tp, w.xT, Tp, dw_lat_down, D, L, D},
                  {w.dshT, Tp, w.xT, Tp, dws_gate, D, SF, D},
                  {w.dshT + (int64_t)SF * Tp, Tp, w.xT, Tp, dws_up, D, SF, D}};
  return gemm_nt_multi("gemm_bwd_dw_pack", "gemm_bwd_dw_pack_tail", sh ? 3 : 1, pr, Tp, w.part, s);
}
