// combine.hip -- gate-weighted combine of the returned rows, latent
// up-projection, and the shared experts.
//
// "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK), section 二
// (and the Japanese translation): the routed outputs are projected back to
// the model width and then joined with the shared-expert path; the two shared
// experts process every token independently of routing.  Section 四: an
// assignment dropped for capacity only loses its routed contribution.
//
// Kernels, in stream order:
//   combine_gather      one wave per token: ylat = bf16(sum_j g_j * row_j),
//                       fp32 accumulation, 16-byte row reads
//   gemm_shared_swiglu  h_s = bf16(silu(x.W_sg,s) * (x.W_su,s)) -> ws
//   gemm_up_shared      out = bf16(ylat.W_lu + sum_s h_s.W_sd,s): one product
//                       over the concatenated K = latent + n_shared*d_ff_shared
#include <algorithm>

#include "kernels.h"

namespace moe {

// One wave per (token, row part): a token's row of nch 16-byte chunks is cut
// into `parts` runs of 64 * CH chunks, so that many short-lived waves (and
// few registers per wave) keep the memory system busy.  A wave reads its
// part of every kept returned row of the token, one row at a time in choice
// order (the summation order), with non-temporal loads: each returned row is
// read exactly once.  Dropped choices are skipped (ballot of the valid ones).
constexpr int CMB_MAX_CH = 3;  // measured at latent 3072: 3 -> 42 us, 1 -> 44, 6 -> 43

template <int CH>
__global__ __launch_bounds__(256) void combine_gather_kernel(
    const uint16_t *__restrict__ returned, const int64_t *__restrict__ ret_offsets,
    const int32_t *__restrict__ topk, const int32_t *__restrict__ slot,
    const float *__restrict__ gates, uint16_t *__restrict__ ylat, int T, int k, int L, int El,
    int Wk, int Tw, int pool_rows, int cap, int parts, int dedup) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);  // < 2^31: T <= 2^27, parts <= 16
  const int t = wv / parts;
  if (t >= T) return;
  const int lane = lane_id();
  const int nch = L / 8, c0 = (wv - t * parts) * 64 * CH + lane;  // this lane's first chunk
  int64_t my_row = -1;
  float my_g = 0.f;
  int my_c = 0;  // dedup: index among the token's same-destination choices
  if (dedup) {
    const int dst = lane < k ? topk[(int64_t)t * k + lane] / El : -1;
    for (int j = 0; j < k; ++j) {
      const int dj = __shfl(dst, j);
      if (dj == dst && j < lane) ++my_c;
    }
  }
  if (lane < k) {
    // the three loads are independent: issued together, one round trip
    const int s = slot[(int64_t)t * k + lane];
    const int e = topk[(int64_t)t * k + lane];
    const float g = gates ? gates[(int64_t)t * k + lane] : 1.f;
    if (s >= 0) {
      const int p = (e / El) * Wk + t / Tw;
      if (cap) {
        my_row = (int64_t)p * pool_rows + s;
        if (dedup) my_row = my_row * 4 + (my_c & 3);  // the choice's return slot
      } else if (s < ret_offsets[p + 1] - ret_offsets[p]) {
        my_row = ret_offsets[p] + s;
      }
      my_g = g;
    }
  }
  float acc[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
  const u32x4 *ret16 = reinterpret_cast<const u32x4 *>(returned);
  uint64_t valid = ballot(my_row >= 0);  // wave-uniform
  while (valid) {
    const int j = (int)__builtin_ctzll(valid);
    valid &= valid - 1;
    const int64_t row = ((int64_t)__shfl((int)(my_row >> 32), j) << 32) |
                        (uint32_t)__shfl((int)my_row, j);
    const float g = __shfl(my_g, j);
    const u32x4 *src = ret16 + row * nch;
    // unpredicated (clamped) loads: all CH in flight together
    u32x4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = ld16<true>(src + min(c0 + 64 * c, nch - 1));
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc[c][2 * h] = fmaf(g, __uint_as_float(v[c][h] << 16), acc[c][2 * h]);
        acc[c][2 * h + 1] = fmaf(g, __uint_as_float(v[c][h] & 0xffff0000u), acc[c][2 * h + 1]);
      }
  }
  u32x4 *dst = reinterpret_cast<u32x4 *>(ylat + (int64_t)t * L);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ci = c0 + 64 * c;
    if (ci < nch) {
      u32x4 o;
#pragma unroll
      for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(acc[c][2 * h], acc[c][2 * h + 1]);
      dst[ci] = o;
    }
  }
}

template <int CH>
static int gather(const moe_dims &d, const uint16_t *returned, const int64_t *ret_offsets,
                  const int32_t *topk, const int32_t *slot, const float *gates, uint16_t *ylat,
                  hipStream_t s) {
  const int parts = (int)cdiv(cdiv(d.latent / 8, 64), CH);
  const PoolKey pk = pool_key(d);
  return launch("combine_gather", combine_gather_kernel<CH>,
                dim3((unsigned)cdiv((int64_t)d.T * parts, 4)), dim3(256), 0, s, returned,
                ret_offsets, topk, slot, gates, ylat, d.T, d.top_k, d.latent,
                experts_per_rank(d), pk.Wk, pk.Tw, pk.rows, d.cap_send, parts, d.dedup);
}

int combine_gather_rows(const moe_dims &d, const uint16_t *rows, const int64_t *offsets,
                        const int32_t *topk, const int32_t *slot, const float *gates,
                        uint16_t *out, hipStream_t s) {
  // chunks per lane: the row's 64-chunk rounds, at most CMB_MAX_CH per wave
  const int ch = (int)std::min<int64_t>(cdiv(d.latent / 8, 64), CMB_MAX_CH);
  return ch <= 1   ? gather<1>(d, rows, offsets, topk, slot, gates, out, s)
         : ch <= 2 ? gather<2>(d, rows, offsets, topk, slot, gates, out, s)
                   : gather<3>(d, rows, offsets, topk, slot, gates, out, s);
}

// gather + up-projection with the shared experts' intermediate H [T, S*Fs]
static int combine_rest(const moe_dims *d, const uint16_t *returned, const int64_t *ret_offsets,
                        const int32_t *topk, const int32_t *slot, const float *gates,
                        const uint16_t *w_lat_up, const uint16_t *H, const uint16_t *ws_down,
                        uint16_t *ylat, uint16_t *out, float *part, hipStream_t s) {
  MOE_TRY(combine_gather_rows(*d, returned, ret_offsets, topk, slot, gates, ylat, s));
  const int S = d->n_shared, Fs = d->d_ff_shared;
  DenseSeg segs[1 + 4];
  segs[0] = DenseSeg{ylat, d->latent, w_lat_up, d->latent, d->latent};
  for (int i = 0; i < S; ++i)
    segs[1 + i] = DenseSeg{H + (int64_t)i * Fs, (int64_t)S * Fs,
                           ws_down + (int64_t)i * d->d_model * Fs, Fs, Fs};
  return gemm_up_shared(d->T, d->d_model, 1 + S, segs, out, d->d_model, part, s);
}

static int check_rest(const moe_dims *d, const moe_bf16 *returned, const int64_t *ret_offsets,
                      const int32_t *topk, const int32_t *slot, const float *gates,
                      const moe_bf16 *w_lat_up, const moe_bf16 *ws_down, moe_bf16 *ylat,
                      moe_bf16 *out) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(returned, "returned"));
  MOE_TRY(check_ptr(topk, "topk"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(gates, "gates"));
  MOE_TRY(check_ptr(w_lat_up, "w_lat_up"));
  MOE_TRY(check_ptr(ylat, "ylat"));
  MOE_TRY(check_ptr(out, "out"));
  if (d->n_shared > 0) MOE_TRY(check_ptr(ws_down, "ws_down"));
  if (ragged(*d)) MOE_TRY(check_ptr(ret_offsets, "ret_offsets (ragged mode)"));
  return MOE_OK;
}

static int check_shared(const moe_dims *d, const moe_bf16 *x, const moe_bf16 *ws_gate,
                        const moe_bf16 *ws_up) {
  MOE_TRY(check_ptr(x, "x"));
  if (d->n_shared > 0) {
    MOE_TRY(check_ptr(ws_gate, "ws_gate"));
    MOE_TRY(check_ptr(ws_up, "ws_up"));
  }
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_shared_swiglu(const moe_dims *d, const moe_bf16 *x, const moe_bf16 *ws_gate,
                                 const moe_bf16 *ws_up, moe_bf16 *h_shared, void *stream) {
  clear_error();
  MOE_TRY(check_dims(d));
  MOE_TRY(check_shared(d, x, ws_gate, ws_up));
  if (d->n_shared > 0) MOE_TRY(check_ptr(h_shared, "h_shared"));
  return gemm_shared_swiglu(d->T, x, d->d_model, d->d_model, ws_gate, ws_up, d->n_shared,
                            d->d_ff_shared, h_shared, nullptr, (hipStream_t)stream);
}

extern "C" int moe_combine_shared(const moe_dims *d, const moe_bf16 *returned,
                                  const int64_t *ret_offsets, const int32_t *topk,
                                  const int32_t *slot, const float *gates,
                                  const moe_bf16 *w_lat_up, const moe_bf16 *h_shared,
                                  const moe_bf16 *ws_down, moe_bf16 *ylat, moe_bf16 *out,
                                  void *ws, int64_t ws_bytes, void *stream) {
  clear_error();
  MOE_TRY(check_rest(d, returned, ret_offsets, topk, slot, gates, w_lat_up, ws_down, ylat, out));
  if (d->n_shared > 0) MOE_TRY(check_ptr(h_shared, "h_shared"));
  // the workspace only holds the partial tiles of a split last round
  if (ws || ws_bytes) {
    const int64_t need = moe_workspace_bytes(d, MOE_CALL_COMBINE_SHARED, 0);
    if (need < 0) return (int)need;
    if (ws_bytes < need || !ws)
      return fail(MOE_ERR_WORKSPACE, "moe_combine_shared: workspace %lld < %lld bytes",
                  (long long)ws_bytes, (long long)need);
    MOE_TRY(check_ptr(ws, "ws"));
  }
  return combine_rest(d, returned, ret_offsets, topk, slot, gates, w_lat_up, h_shared, ws_down,
                      ylat, out, (float *)ws, (hipStream_t)stream);
}

extern "C" int moe_combine(const moe_dims *d, const moe_bf16 *returned, const int64_t *ret_offsets,
                           const int32_t *topk, const int32_t *slot, const float *gates,
                           const moe_bf16 *x, const moe_bf16 *w_lat_up, const moe_bf16 *ws_gate,
                           const moe_bf16 *ws_up, const moe_bf16 *ws_down, moe_bf16 *ylat,
                           moe_bf16 *out, void *ws, int64_t ws_bytes, void *stream) {
  clear_error();
  MOE_TRY(check_rest(d, returned, ret_offsets, topk, slot, gates, w_lat_up, ws_down, ylat, out));
  MOE_TRY(check_shared(d, x, ws_gate, ws_up));
  const int64_t need = moe_workspace_bytes(d, MOE_CALL_COMBINE, 0);
  if (need < 0) return (int)need;
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(MOE_ERR_WORKSPACE, "moe_combine: workspace %lld < %lld bytes",
                (long long)ws_bytes, (long long)need);
  if (ws) MOE_TRY(check_ptr(ws, "ws"));
  hipStream_t s = (hipStream_t)stream;
  // workspace: the shared experts' intermediate, then the partial tiles of
  // the up-projection's split last round (the shared experts run whole, as
  // in moe_shared_swiglu)
  uint16_t *H = (uint16_t *)ws;
  float *part = (float *)((char *)ws + shared_h_bytes(*d));
  MOE_TRY(gemm_shared_swiglu(d->T, x, d->d_model, d->d_model, ws_gate, ws_up, d->n_shared,
                             d->d_ff_shared, H, nullptr, s));
  return combine_rest(d, returned, ret_offsets, topk, slot, gates, w_lat_up, H, ws_down, ylat,
                      out, part, s);
}
