// rank.h -- ordered slot assignment: for a sequence of items, each with a
// small integer key (or none), give every keyed item its position among the
// earlier items with the same key.  Deterministic: no order-dependent
// atomics decide a position.
//
// Items are split into tiles of RK_TILE; wave w of a tile owns one
// contiguous run of 64*RK_IPT items, read in RK_IPT rounds of 64 (all loads
// issued before any use, so one wave has its whole run in flight).
//   rank_count   per tile: how many items carry each key (LDS atomics only
//                add, so the totals are order-independent) -> ws
//   rank_assign  per tile: position = (items of that key in earlier tiles)
//                + (in earlier waves of this tile) + (in earlier rounds of
//                this wave) + (in lower lanes of this round), the last from
//                a wave ballot; block 0 also writes the per-key totals.
#pragma once
#include "common.h"

namespace moe {

constexpr int RK_THREADS = 1024;
constexpr int RK_WAVES = RK_THREADS / 64;
constexpr int RK_IPT = 2;
constexpr int RK_TILE = RK_THREADS * RK_IPT;
constexpr int RK_MAXK = 1024;

enum : int32_t { KEY_NONE = -1, KEY_BAD = -2 };

inline int64_t rank_tiles(int64_t n) { return cdiv(n, RK_TILE) > 0 ? cdiv(n, RK_TILE) : 1; }
inline int64_t rank_ws_bytes(int64_t n, int K) { return align_up(rank_tiles(n) * (K + 1) * 4, 256); }

__device__ __forceinline__ int64_t rk_item(int r) {
  return (int64_t)blockIdx.x * RK_TILE + (threadIdx.x >> 6) * (64 * RK_IPT) + r * 64 + lane_id();
}

// Exclusive scan of v[0..n) (n <= RK_THREADS) in place, int64, whole block.
// out[n] receives the total.  Uses tmp[RK_THREADS].
__device__ inline void block_exscan_i64(int64_t *v, int n, int64_t *tmp) {
  const int t = threadIdx.x;
  int64_t x = t < n ? v[t] : 0;
  tmp[t] = x;
  __syncthreads();
  for (int off = 1; off < RK_THREADS; off <<= 1) {
    int64_t y = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += y;
    __syncthreads();
  }
  if (t < n) v[t] = tmp[t] - x;
  if (t == RK_THREADS - 1) v[n] = tmp[t];
  __syncthreads();
}

// Src:  __device__ void prepare(int64_t* lds_scratch)  (block-wide setup)
//       __device__ int32_t key(int64_t item, int32_t& aux)
// Fill: bank_src style array set to -1 by the count kernel (may be null).
template <class Src>
__global__ __launch_bounds__(RK_THREADS) void rank_count(Src src, int64_t n, int K,
                                                         int32_t *__restrict__ tile_counts,
                                                         int32_t *__restrict__ clear,
                                                         int64_t n_clear) {
  __shared__ int32_t cnt[RK_MAXK + 1];
  __shared__ int64_t scratch[2 * RK_THREADS + 2];
  const int t = threadIdx.x;
  for (int i = t; i <= K; i += RK_THREADS) cnt[i] = 0;
  src.prepare(scratch);
  __syncthreads();
  int32_t key[RK_IPT], aux[RK_IPT];
#pragma unroll
  for (int r = 0; r < RK_IPT; ++r) {
    int64_t it = rk_item(r);
    key[r] = it < n ? src.key(it, aux[r]) : KEY_NONE;
  }
#pragma unroll
  for (int r = 0; r < RK_IPT; ++r) {
    if (key[r] >= 0) atomicAdd(&cnt[key[r]], 1);
    else if (key[r] == KEY_BAD) atomicAdd(&cnt[K], 1);
  }
  __syncthreads();
  for (int i = t; i <= K; i += RK_THREADS) tile_counts[(int64_t)blockIdx.x * (K + 1) + i] = cnt[i];
  if (clear)
    for (int64_t p = (int64_t)blockIdx.x * RK_THREADS + t; p < n_clear;
         p += (int64_t)gridDim.x * RK_THREADS)
      clear[p] = -1;
}

// Emit: __device__ void item(int64_t item, int key, int32_t aux, int rank, const int64_t* koff)
//         (called for every item < n; rank is meaningful only when key >= 0)
//       __device__ void totals(int K, const int32_t* ktot, const int64_t* koff, int32_t bad)
//       static constexpr bool needs_offsets
template <class Src, class Emit>
__global__ __launch_bounds__(RK_THREADS) void rank_assign(Src src, Emit emit, int64_t n, int K,
                                                          int n_tiles,
                                                          const int32_t *__restrict__ tile_counts) {
  __shared__ int32_t wcnt[RK_WAVES][RK_MAXK];
  __shared__ int32_t ktot[RK_MAXK];
  __shared__ int64_t koff[RK_MAXK + 1];
  __shared__ int64_t scratch[2 * RK_THREADS + 2];
  __shared__ int32_t bad_total;
  const int t = threadIdx.x, w = t >> 6, lane = lane_id();
  for (int i = t; i < RK_WAVES * RK_MAXK; i += RK_THREADS) (&wcnt[0][0])[i] = 0;
  src.prepare(scratch);
  __syncthreads();

  int32_t key[RK_IPT], aux[RK_IPT];
#pragma unroll
  for (int r = 0; r < RK_IPT; ++r) {
    int64_t it = rk_item(r);
    key[r] = it < n ? src.key(it, aux[r]) : KEY_NONE;
  }
#pragma unroll
  for (int r = 0; r < RK_IPT; ++r)
    if (key[r] >= 0) atomicAdd(&wcnt[w][key[r]], 1);
  __syncthreads();

  // per key: items in earlier tiles, total, then running base per wave
  for (int kk = t; kk < K; kk += RK_THREADS) {
    int32_t before = 0, total = 0;
    for (int tt = 0; tt < n_tiles; ++tt) {
      int32_t c = tile_counts[(int64_t)tt * (K + 1) + kk];
      before += tt < (int)blockIdx.x ? c : 0;
      total += c;
    }
    int32_t run = before;
    for (int ww = 0; ww < RK_WAVES; ++ww) {
      int32_t c = wcnt[ww][kk];
      wcnt[ww][kk] = run;
      run += c;
    }
    ktot[kk] = total;
    koff[kk] = total;
  }
  if (t == 0) {
    int32_t b = 0;
    for (int tt = 0; tt < n_tiles; ++tt) b += tile_counts[(int64_t)tt * (K + 1) + K];
    bad_total = b;
  }
  __syncthreads();
  if (Emit::needs_offsets) block_exscan_i64(koff, K, scratch);
  if (blockIdx.x == 0) emit.totals(K, ktot, koff, bad_total);

  // bits to tell apart keys -2 .. K-1
  int bits = 1;
  while ((1 << bits) < K + 2) ++bits;
#pragma unroll
  for (int r = 0; r < RK_IPT; ++r) {
    const int k = key[r];
    const uint64_t peers = match_key((uint32_t)(k + 2), bits);
    int base = 0;
    if (k >= 0) base = wcnt[w][k];
    const bool leader = (peers & ~((2ull << lane) - 1ull)) == 0;
    if (k >= 0 && leader) wcnt[w][k] = base + __popcll(peers);
    const int64_t it = rk_item(r);
    if (it < n) emit.item(it, k, aux[r], base + __popcll(peers & lanemask_lt()), koff);
  }
}

}  // namespace moe
