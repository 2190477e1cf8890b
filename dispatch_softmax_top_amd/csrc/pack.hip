// pack.hip -- sender side: latent down-projection, slot assignment into one
// fixed pool per (destination rank, wave), and the row scatter.
//
// "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK), section 二
// (same in the Japanese translation, section 二): activations are projected
// to the latent width before the exchange; the sender keeps one fixed pool
// per destination GPU (not per expert), sends in three waves of one array
// shape, puts the expert id inside the payload so no counts or metadata are
// exchanged, caps each (source, destination) pool with the sender capacity
// factor, and drops and counts the overflow.
//
// Kernels, in stream order:
//   rank_count / rank_assign  positions of (token, choice) assignments in
//                             their pool, in (token, choice) order
//
// Pools are keyed by (dest, wave(t)) when waves split the tokens, and by
// dest alone when they cut each destination's pool of W*C_s rows into W
// chunks; both cases share the kernels through (pool key, rows per key):
// key = dest * Wk + t / Tw with Wk = W (or 1, and Tw past T), and a kept
// row lands at key * pool_rows + slot with pool_rows = C_s (or W * C_s).
//   gemm_latent_down          z = x . W_ld (bf16 MFMA)
//   pack_rows                 one wave per token: z[t] read once, written to
//                             each kept destination row with 16-byte stores;
//                             extra blocks stamp id -1 on unfilled slots
#include <mutex>
#include <type_traits>

#include "gemm.h"
#include "kernels.h"
#include "rank.h"

namespace moe {

// Index of choice j among the token's earlier choices on the same
// destination (the dedup variant groups them four to a row).
__device__ __forceinline__ int dedup_rank(const int32_t *tk, int j, int El) {
  const int dj = tk[j] / El;
  int c = 0;
  for (int i = 0; i < j; ++i) c += tk[i] / El == dj;
  return c;
}

struct SenderSrc {
  const int32_t *topk;
  int k, E, El, W, Tw, dedup;
  __device__ void prepare(int64_t *) {}
  __device__ int32_t key(int64_t item, int32_t &aux) const {
    aux = 0;
    const int e = topk[item];
    if ((unsigned)e >= (unsigned)E) return KEY_BAD;  // not a valid choice: never kept
    const int t = (int)(item / k);
    // dedup: only a row's first choice takes a position; the others join it
    if (dedup && dedup_rank(topk + (int64_t)t * k, (int)(item - (int64_t)t * k), El) % 4)
      return KEY_NONE;
    return (e / El) * W + t / Tw;
  }
};

// dedup: every choice that joined a row takes the slot of the row's first
// choice (assigned by rank_assign before).  One thread per choice.
__global__ __launch_bounds__(256) void dedup_follow_kernel(const int32_t *__restrict__ topk,
                                                           int32_t *__restrict__ slot, int64_t n,
                                                           int k, int El) {
  const int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (it >= n) return;
  const int64_t t0 = it - it % k;
  const int j = (int)(it - t0);
  const int32_t *tk = topk + t0;
  const int c = dedup_rank(tk, j, El);
  if (c % 4 == 0) return;
  const int dj = tk[j] / El, lead = c - c % 4;
  for (int i = 0, r = 0; i < j; ++i)
    if (tk[i] / El == dj) {
      if (r == lead) {
        slot[it] = slot[t0 + i];
        return;
      }
      ++r;
    }
}

// chunks = W when the key is the destination alone (its pool holds W chunks
// of cap rows), 0 when the key already names the wave.
template <bool RAGGED>
struct SenderEmit {
  static constexpr bool needs_offsets = RAGGED;
  int32_t *slot, *fill, *demand;
  int64_t *pool_offsets;
  int cap, chunks;
  __device__ void item(int64_t it, int key, int32_t, int rank, const int64_t *) const {
    const int limit = chunks ? chunks * cap : cap;  // W * cap < 2^31 (checked on the host)
    slot[it] = (key >= 0 && (RAGGED || rank < limit)) ? rank : -1;
  }
  __device__ void totals(int K, const int32_t *tot, const int64_t *koff, int32_t) const {
    if (chunks) {  // fill / demand per (dest, chunk); the overflow is the last chunk's
      for (int q = threadIdx.x; q < K * chunks; q += blockDim.x) {
        const int w = q % chunks;
        const int left = max(tot[q / chunks] - w * cap, 0);
        fill[q] = min(left, cap);
        demand[q] = w + 1 < chunks ? min(left, cap) : left;
      }
      return;
    }
    for (int kk = threadIdx.x; kk < K; kk += blockDim.x) {
      demand[kk] = tot[kk];
      fill[kk] = RAGGED ? tot[kk] : min(tot[kk], cap);
      if (RAGGED) pool_offsets[kk] = koff[kk];
    }
    if (RAGGED && threadIdx.x == 0) pool_offsets[K] = koff[K];
  }
};


// One wave per token: each lane loads all CH of its 16-byte chunks of z[t]
// first (the whole row in flight), then writes them to every kept row.
template <int CH>
__global__ __launch_bounds__(256) void pack_rows_kernel(
    const uint16_t *__restrict__ z, const int32_t *__restrict__ topk,
    const int32_t *__restrict__ slot, const int32_t *__restrict__ fill,
    const int64_t *__restrict__ pool_offsets, uint8_t *__restrict__ pools, int T, int k, int L,
    int El, int Wk, int Tw, int pool_rows, int cap, int token_blocks, int64_t n_slots,
    int dedup) {
  const int64_t RB = 2 * (int64_t)L + 16;
  const int lane = lane_id();
  if ((int)blockIdx.x < token_blocks) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int nch = L / 8;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(z + (int64_t)t * L);
    u32x4 v[CH];  // unpredicated loads (clamped index): all CH in flight at once
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = src[min(lane + 64 * c, nch - 1)];
    int my_row = -1, my_e = -1;
    int s = -1, e = -1;
    if (lane < k) {
      s = slot[(int64_t)t * k + lane];
      e = topk[(int64_t)t * k + lane];  // independent of s: same round trip
      if (s >= 0) {
        const int p = (e / El) * Wk + t / Tw;
        my_row = cap ? p * pool_rows + s : (int)pool_offsets[p] + s;
        my_e = e;
      }
    }
    u32x4 hdr = {(uint32_t)my_e, 0u, 0u, 0u};
    if (dedup) {
      // this lane's index among same-destination choices; a row's first
      // choice writes the row with the ids of its group (up to four, in
      // choice order), the others write nothing
      const int dst = lane < k ? e / El : -1;
      int c = 0;
      for (int j = 0; j < k; ++j) {
        const int dj = __shfl(dst, j);
        if (dj == dst && j < lane) ++c;
      }
      // a leader (c % 4 == 0) collects the choices ranked c .. c + 3 on its
      // destination: id number cj - c of its row
      int id0 = -1, id1 = -1, id2 = -1, id3 = -1;
      for (int j = 0; j < k; ++j) {
        const int dj = __shfl(dst, j), ej = __shfl(e, j), cj = __shfl(c, j);
        if (dj != dst || (c & 3)) continue;
        const int q = cj - c;
        if (q == 0) id0 = ej;
        if (q == 1) id1 = ej;
        if (q == 2) id2 = ej;
        if (q == 3) id3 = ej;
      }
      if (c & 3) my_row = -1;
      hdr = u32x4{(uint32_t)id0, (uint32_t)id1, (uint32_t)id2, (uint32_t)id3};
    }
    for (int j = 0; j < k; ++j) {
      const int row = __shfl(my_row, j);
      if (row < 0) continue;
      u32x4 *dst = reinterpret_cast<u32x4 *>(pools + row * RB);
      if (nch == 64 * CH) {
#pragma unroll
        for (int c = 0; c < CH; ++c) dst[lane + 64 * c] = v[c];
      } else {
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (lane + 64 * c < nch) dst[lane + 64 * c] = v[c];
      }
    }
    if (my_row >= 0) *reinterpret_cast<u32x4 *>(pools + my_row * RB + 2 * (int64_t)L) = hdr;
  } else {
    const int64_t idx = (int64_t)(blockIdx.x - token_blocks) * 256 + threadIdx.x;
    if (idx >= n_slots) return;
    const int p = (int)(idx / cap), i = (int)(idx - (int64_t)p * cap);
    if (i >= fill[p]) {
      const uint32_t more = dedup ? 0xffffffffu : 0u;  // dedup: four empty ids
      u32x4 h = {0xffffffffu, more, more, more};
      *reinterpret_cast<u32x4 *>(pools + idx * RB + 2 * (int64_t)L) = h;
    }
  }
}

template <int CH>
static int pack_copy(const moe_dims &d, const uint16_t *z, const int32_t *topk,
                     const int32_t *slot, const int32_t *fill, const int64_t *pool_offsets,
                     uint8_t *pools, int token_blocks, int64_t n_slots, hipStream_t s) {
  const int64_t blocks = token_blocks + cdiv(n_slots, 256);
  const PoolKey pk = pool_key(d);
  return launch("pack_rows", pack_rows_kernel<CH>, dim3((unsigned)blocks), dim3(256), 0, s, z,
                topk, slot, fill, pool_offsets, pools, d.T, d.top_k, d.latent,
                experts_per_rank(d), pk.Wk, pk.Tw, pk.rows, d.cap_send, token_blocks, n_slots,
                d.dedup);
}

template <bool RAGGED>
static int sender_slots(const moe_dims &d, const int32_t *topk, int32_t *slot, int32_t *fill,
                        int32_t *demand, int64_t *pool_offsets, int32_t *tile_counts,
                        hipStream_t s) {
  const int64_t n = (int64_t)d.T * d.top_k;
  const PoolKey pk = pool_key(d);
  const int K = d.n_ranks * pk.Wk;
  const int tiles = (int)rank_tiles(n);
  SenderSrc src{topk, d.top_k, d.n_experts, experts_per_rank(d), pk.Wk, pk.Tw, d.dedup};
  SenderEmit<RAGGED> em{slot, fill, demand, pool_offsets, d.cap_send,
                        d.wave_mode == MOE_WAVES_CHUNKS ? d.n_waves : 0};
  MOE_TRY(launch("rank_count_sender", rank_count<SenderSrc>, dim3(tiles), dim3(RK_THREADS), 0, s,
                 src, n, K, tile_counts, (int32_t *)nullptr, (int64_t)0));
  MOE_TRY(launch("rank_assign_sender", rank_assign<SenderSrc, SenderEmit<RAGGED>>, dim3(tiles),
                 dim3(RK_THREADS), 0, s, src, em, n, K, tiles, (const int32_t *)tile_counts));
  if (!d.dedup) return MOE_OK;
  return launch("dedup_follow", dedup_follow_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s,
                topk, slot, n, d.top_k, experts_per_rank(d));
}

// Scratch of moe_pack_waves_noalloc: the per-tile key counts of the
// sender's slot assignment, in a fixed device array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  rank_count writes every entry rank_assign reads, so nothing
// needs clearing between calls.
static __device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / 4];

// Device address of `scratch` on each device, taken once per device with it
// current.  In host code the array's name is only a stand-in symbol: kernels
// get this address, never the name.
constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[SCRATCH_MAX_DEVICES];

static int noalloc_scratch(void **out) {
  int dev = -1;
  MOE_TRY(hip_status(hipGetDevice(&dev), "moe_pack_waves_noalloc: hipGetDevice"));
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_waves_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    MOE_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                       "moe_pack_waves_noalloc: hipGetSymbolAddress"));
    if (!p) return fail(MOE_ERR_HIP, "moe_pack_waves_noalloc: scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Both entry points: checks on the host, then the launches.  fixed_scratch:
// the slot assignment's counts go to `scratch` (ws and ws_bytes unused).
static int pack_waves(const moe_dims *d, const moe_bf16 *x, const moe_bf16 *w_lat_down,
                      const int32_t *topk, moe_bf16 *z, uint8_t *pools, int64_t *pool_offsets,
                      int32_t *slot, int32_t *fill, int32_t *demand, void *ws, int64_t ws_bytes,
                      bool fixed_scratch, void *stream) {
  clear_error();
  MOE_TRY(check_dims(d));
  const bool rg = ragged(*d);
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(w_lat_down, "w_lat_down"));
  MOE_TRY(check_ptr(topk, "topk"));
  MOE_TRY(check_ptr(z, "z"));
  MOE_TRY(check_ptr(pools, "pools"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(fill, "fill"));
  MOE_TRY(check_ptr(demand, "demand"));
  if (rg) MOE_TRY(check_ptr(pool_offsets, "pool_offsets (ragged mode)"));
  const int64_t need = moe_workspace_bytes(d, MOE_CALL_PACK, 0);
  if (need < 0) return (int)need;
  if (fixed_scratch) {
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_ERR_UNSUPPORTED,
                  "moe_pack_waves_noalloc: needs %lld scratch bytes, the fixed scratch holds "
                  "%lld (use moe_pack_waves with a workspace)",
                  (long long)need, (long long)MOE_NOALLOC_SCRATCH_BYTES);
  } else {
    if (ws_bytes < need || (need > 0 && !ws))
      return fail(MOE_ERR_WORKSPACE, "moe_pack_waves: workspace %lld < %lld bytes",
                  (long long)ws_bytes, (long long)need);
    if (ws) MOE_TRY(check_ptr(ws, "ws"));
  }
  if ((int64_t)d->n_ranks * d->n_waves * d->cap_send >= (1ll << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_waves: pool rows must fit in int32");
  if (fixed_scratch) MOE_TRY(noalloc_scratch(&ws));
  hipStream_t s = (hipStream_t)stream;
  int32_t *tc = (int32_t *)ws;

  MOE_TRY(rg ? sender_slots<true>(*d, topk, slot, fill, demand, pool_offsets, tc, s)
             : sender_slots<false>(*d, topk, slot, fill, demand, pool_offsets, tc, s));
  DenseSeg seg{x, d->d_model, w_lat_down, d->d_model, d->d_model};
  MOE_TRY(gemm_latent_down(d->T, d->latent, seg, z, d->latent, s));
  const int token_blocks = (int)cdiv(d->T, 4);
  const int64_t n_slots = rg ? 0 : (int64_t)d->n_ranks * d->n_waves * d->cap_send;
  const int ch = (int)cdiv(d->latent / 8, 64);  // latent <= 8192 (check_dims)
  auto run = [&](auto kernel_ch) {
    constexpr int CH = decltype(kernel_ch)::value;
    return pack_copy<CH>(*d, z, topk, slot, fill, pool_offsets, pools, token_blocks, n_slots, s);
  };
  if (ch <= 1) return run(std::integral_constant<int, 1>());
  if (ch <= 2) return run(std::integral_constant<int, 2>());
  if (ch <= 4) return run(std::integral_constant<int, 4>());
  if (ch <= 6) return run(std::integral_constant<int, 6>());
  if (ch <= 8) return run(std::integral_constant<int, 8>());
  return run(std::integral_constant<int, 16>());
}

}  // namespace moe

using namespace moe;

extern "C" int moe_pack_waves(const moe_dims *d, const moe_bf16 *x, const moe_bf16 *w_lat_down,
                              const int32_t *topk, moe_bf16 *z, uint8_t *pools,
                              int64_t *pool_offsets, int32_t *slot, int32_t *fill,
                              int32_t *demand, void *ws, int64_t ws_bytes, void *stream) {
  return pack_waves(d, x, w_lat_down, topk, z, pools, pool_offsets, slot, fill, demand, ws,
                    ws_bytes, false, stream);
}

extern "C" int moe_pack_waves_noalloc(const moe_dims *d, const moe_bf16 *x,
                                      const moe_bf16 *w_lat_down, const int32_t *topk,
                                      moe_bf16 *z, uint8_t *pools, int64_t *pool_offsets,
                                      int32_t *slot, int32_t *fill, int32_t *demand,
                                      void *stream) {
  return pack_waves(d, x, w_lat_down, topk, z, pools, pool_offsets, slot, fill, demand, nullptr,
                    0, true, stream);
}
