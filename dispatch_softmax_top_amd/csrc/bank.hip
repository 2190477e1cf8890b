// bank.hip -- receiver side: bank the rows received by this rank into its
// local experts, per wave.
//
// "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK), section 二
// (and its Japanese translation): a receiver capacity factor caps the rows
// assigned to one local expert, overflow is dropped and counted apart, and
// the three waves keep only part of the six-expert bank live at a time.
// "从玩具到前沿:训练一个真正的大模型,到底难在哪里" (devpress.csdn.net),
// section 四 and appendix A.3: each wave the receiver runs all local experts.
//
// Rows are taken in (source, row) order within each wave; the capacity
// applies per (wave, local expert).  The expert id in each row's tail is the
// only routing information used.
//
// Kernels, in stream order:
//   rank_count (also sets bank_src to -1) / rank_assign  bank positions
//   bank_rows   one wave per bank position: 16-byte copy of the payload
#include <type_traits>

#include "kernels.h"
#include "rank.h"

namespace moe {

template <bool RAGGED>
struct RecvSrc {
  const uint8_t *recv;
  const int64_t *offs;  // ragged: [R*W+1], segment (s, w) at s*W + w
  int64_t RB;
  int L, R, W, El, E, rank, cap_send;
  int dedup;  // items are (row, tail id index): four per row (fixed mode)
  const int64_t *vstart;  // ragged: first item of segment (w, s) in item order, in LDS
  __device__ void prepare(int64_t *sc) {
    if (!RAGGED) return;
    const int nseg = R * W;
    const int v = threadIdx.x;
    if (v < nseg) {
      const int s = v % R, w = v / R;
      sc[v] = offs[s * W + w + 1] - offs[s * W + w];
    }
    block_exscan_i64(sc, nseg, sc + RK_MAXK + 1);
    vstart = sc;
  }
  __device__ int32_t key(int64_t q, int32_t &aux) const {
    int64_t row;
    int w;
    const int idx = dedup ? (int)(q & 3) : 0;  // dedup: which of the row's four ids
    if (dedup) q >>= 2;
    if (!RAGGED) {
      const int64_t per = (int64_t)R * cap_send;
      w = (int)(q / per);
      const int64_t rem = q - (int64_t)w * per;
      const int s = (int)(rem / cap_send);
      const int i = (int)(rem - (int64_t)s * cap_send);
      row = ((int64_t)s * W + w) * cap_send + i;
    } else {
      int lo = 0, hi = R * W - 1;  // largest v with vstart[v] <= q
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (vstart[mid] <= q) lo = mid;
        else hi = mid - 1;
      }
      const int s = lo % R;
      w = lo / R;
      row = offs[s * W + w] + (q - vstart[lo]);
    }
    aux = (int32_t)(dedup ? row * 4 + idx : row);  // bank_src: receive row, or return slot
    const int h = *reinterpret_cast<const int32_t *>(recv + row * RB + 2 * (int64_t)L + 4 * idx);
    if (h == -1) return KEY_NONE;
    if (h < 0 || h >= E || h / El != rank) return KEY_BAD;
    return w * El + h % El;
  }
};

template <bool RAGGED>
struct BankEmit {
  static constexpr bool needs_offsets = RAGGED;
  int32_t *bank_src, *bfill, *bdemand, *bad_rows;
  int64_t *bank_offsets;
  int cap;
  __device__ void item(int64_t, int key, int32_t row, int rank, const int64_t *koff) const {
    if (key < 0) return;
    int64_t pos = -1;
    if (RAGGED) pos = koff[key] + rank;
    else if (rank < cap) pos = (int64_t)key * cap + rank;
    if (pos >= 0) bank_src[pos] = row;
  }
  __device__ void totals(int K, const int32_t *tot, const int64_t *koff, int32_t bad) const {
    for (int kk = threadIdx.x; kk < K; kk += blockDim.x) {
      bdemand[kk] = tot[kk];
      bfill[kk] = RAGGED ? tot[kk] : min(tot[kk], cap);
      if (RAGGED) bank_offsets[kk] = koff[kk];
    }
    if (threadIdx.x == 0) {
      if (RAGGED) bank_offsets[K] = koff[K];
      bad_rows[0] = bad;
    }
  }
};

// One wave per bank position; each lane loads all CH of its 16-byte chunks
// before storing any, so a wave keeps its whole row in flight.  The loads
// are non-temporal (each received row is read once); the stores are plain,
// since the expert GEMM reads the bank next (measured: non-temporal loads
// 69 us, plain 86 us, non-temporal loads and stores 74 us at 4096 tokens).
template <int CH>
__global__ __launch_bounds__(256) void bank_rows_kernel(const uint8_t *__restrict__ recv,
                                                        const int32_t *__restrict__ bank_src,
                                                        uint16_t *__restrict__ bank, int L,
                                                        int64_t n_pos, int src_shift) {
  const int64_t pos = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pos >= n_pos) return;
  const int src = bank_src[pos] >> src_shift;  // dedup: return slot -> receive row
  if (src < 0) return;
  const u32x4 *in = reinterpret_cast<const u32x4 *>(recv + (int64_t)src * (2 * (int64_t)L + 16));
  u32x4 *out = reinterpret_cast<u32x4 *>(bank + pos * L);
  const int nch = L / 8, lane = lane_id();
  // loads are never predicated (an index past the row is clamped to its last
  // chunk), so all CH issue back to back; only a partial row's stores are
  u32x4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = ld16<true>(in + min(lane + 64 * c, nch - 1));
  if (nch == 64 * CH) {
#pragma unroll
    for (int c = 0; c < CH; ++c) out[lane + 64 * c] = v[c];
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (lane + 64 * c < nch) out[lane + 64 * c] = v[c];
  }
}

template <int CH>
static int bank_copy(const moe_dims &d, const uint8_t *recv, const int32_t *bank_src,
                     uint16_t *bank, int64_t n_bank, hipStream_t s) {
  return launch("bank_rows", bank_rows_kernel<CH>, dim3((unsigned)cdiv(n_bank, 4)), dim3(256), 0,
                s, recv, bank_src, bank, d.latent, n_bank, d.dedup ? 2 : 0);
}

template <bool RAGGED>
static int bank_slots(const moe_dims &d, int rank, const uint8_t *recv,
                      const int64_t *recv_offsets, int64_t n_items, int64_t n_bank,
                      int32_t *bank_src, int32_t *bfill, int32_t *bdemand,
                      int64_t *bank_offsets, int32_t *bad_rows, int32_t *tc, hipStream_t s) {
  const int K = d.n_waves * experts_per_rank(d);
  const int tiles = (int)rank_tiles(n_items);
  RecvSrc<RAGGED> src{recv,      recv_offsets,  row_bytes(d), d.latent, d.n_ranks,
                      d.n_waves, experts_per_rank(d), d.n_experts, rank, d.cap_send,
                      RAGGED ? 0 : d.dedup, nullptr};
  BankEmit<RAGGED> em{bank_src, bfill, bdemand, bad_rows, bank_offsets, d.cap_recv};
  MOE_TRY(launch("rank_count_bank", rank_count<RecvSrc<RAGGED>>, dim3(tiles), dim3(RK_THREADS), 0,
                 s, src, n_items, K, tc, bank_src, n_bank));
  return launch("rank_assign_bank", rank_assign<RecvSrc<RAGGED>, BankEmit<RAGGED>>, dim3(tiles),
                dim3(RK_THREADS), 0, s, src, em, n_items, K, tiles, (const int32_t *)tc);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_bank(const moe_dims *d, int32_t rank, const uint8_t *recv,
                        const int64_t *recv_offsets, int64_t n_recv_rows, moe_bf16 *bank,
                        int64_t *bank_offsets, int32_t *bank_src, int32_t *bfill,
                        int32_t *bdemand, int32_t *bad_rows, void *ws, int64_t ws_bytes,
                        void *stream) {
  clear_error();
  MOE_TRY(check_dims(d));
  const bool rg = ragged(*d);
  if (rank < 0 || rank >= d->n_ranks) return fail(MOE_ERR_INVALID, "moe_bank: rank out of range");
  MOE_TRY(check_ptr(recv, "recv"));
  MOE_TRY(check_ptr(bank, "bank"));
  MOE_TRY(check_ptr(bank_src, "bank_src"));
  MOE_TRY(check_ptr(bfill, "bfill"));
  MOE_TRY(check_ptr(bdemand, "bdemand"));
  MOE_TRY(check_ptr(bad_rows, "bad_rows"));
  if (rg) {
    MOE_TRY(check_ptr(recv_offsets, "recv_offsets (ragged mode)"));
    MOE_TRY(check_ptr(bank_offsets, "bank_offsets (ragged mode)"));
    if (n_recv_rows < 0 || n_recv_rows >= (1ll << 31))
      return fail(MOE_ERR_INVALID, "moe_bank: n_recv_rows out of range");
  } else if (n_recv_rows != (int64_t)d->n_ranks * d->n_waves * d->cap_send) {
    return fail(MOE_ERR_INVALID, "moe_bank: fixed mode needs n_recv_rows == n_ranks*n_waves*cap_send");
  }
  const int64_t n_bank = rg ? n_recv_rows : (int64_t)d->n_waves * experts_per_rank(*d) * d->cap_recv;
  if (n_bank >= (1ll << 31)) return fail(MOE_ERR_UNSUPPORTED, "moe_bank: too many bank rows");
  const int64_t need = moe_workspace_bytes(d, MOE_CALL_BANK, n_recv_rows);
  if (need < 0) return (int)need;
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(MOE_ERR_WORKSPACE, "moe_bank: workspace %lld < %lld bytes", (long long)ws_bytes,
                (long long)need);
  if (ws) MOE_TRY(check_ptr(ws, "ws"));
  hipStream_t s = (hipStream_t)stream;
  int32_t *tc = (int32_t *)ws;
  MOE_TRY(rg ? bank_slots<true>(*d, rank, recv, recv_offsets, n_recv_rows, n_bank, bank_src, bfill,
                                bdemand, bank_offsets, bad_rows, tc, s)
             : bank_slots<false>(*d, rank, recv, nullptr, n_recv_rows * ret_slots(*d), n_bank,
                                 bank_src, bfill, bdemand, nullptr, bad_rows, tc, s));
  const int ch = (int)cdiv(d->latent / 8, 64);  // latent <= 8192 (check_dims)
  auto run = [&](auto kernel_ch) {
    constexpr int CH = decltype(kernel_ch)::value;
    return bank_copy<CH>(*d, recv, bank_src, bank, n_bank, s);
  };
  if (ch <= 1) return run(std::integral_constant<int, 1>());
  if (ch <= 2) return run(std::integral_constant<int, 2>());
  if (ch <= 4) return run(std::integral_constant<int, 4>());
  if (ch <= 6) return run(std::integral_constant<int, 6>());
  if (ch <= 8) return run(std::integral_constant<int, 8>());
  return run(std::integral_constant<int, 16>());
}
