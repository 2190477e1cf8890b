// route.hip -- router: softmax over all experts, then the top k.
//
// "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK), section 二,
// and "从玩具到前沿:训练一个真正的大模型,到底难在哪里" (devpress.csdn.net),
// section 四: every token is routed to 8 of 384 experts.
//
// One wave64 per token.  Lane l holds the logits of experts l*V .. l*V+V-1
// (V = ceil(E / 64)).  The choice order is (logit descending, index
// ascending).  Each candidate's order-preserving 32-bit image of its fp32
// logit is its key; each lane keeps its candidates sorted by (key
// descending, index ascending).  k rounds take the wave-wide largest head
// (DPP maxima inside 16-lane rows, two row broadcasts, one lane read: a
// wave-uniform value); if several lanes hold that key (equal logits), a
// second reduction takes the lowest index among them.  The winner's lane
// pops its head, and choice j is written into lane j.  The first choice is
// the largest logit m; gates are exp(l - m) / sum exp(l - m) over all E
// logits, in fp32 (exp by the hardware exp2).
//
// Quantile balancing ("从玩具到前沿:训练一个真正的大模型,到底难在哪里",
// section 四 and appendix A.2): a per-expert bias is added to the logits
// before routing (fp32 sum; it only changes the next choices), from a count
// of each expert's selections over the past batches:
//   expert_counts   per-block LDS histogram of topk, added to counts[E]
//   balance_bias    b_i = -alpha (H_i / sum H - 1/E) over a window of counts
#include <math.h>

#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t ord_f32(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal logits compare equal
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // negative: ~u, else u | sign
}

__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __uint_as_float(o ^ ((uint32_t)((int32_t)~o >> 31) | 0x80000000u));
}

// Reductions over the wave with a wave-uniform result: DPP inside each
// 16-lane row (swaps within quads, then rotations by 4 and 8; every lane
// reads a valid lane, so the DPP folds into the operation itself and every
// lane ends with its row's result), then row 0's lane 15 is folded into row
// 1 and row 2's into row 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31); lane 63 then holds ((r3 op r2) op (r1 op r0)) and is read
// once.  `id` is the operation's identity (what the rows left out of a
// broadcast fold in).  The order of the operations is fixed, so a sum is the
// same on every call.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));   // [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true));  // row_ror:4
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true));  // row_ror:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xA, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// v with lane j set to the wave-uniform x: one v_writelane, whose lane
// select has to be M0 when the value is an SGPR.
__device__ __forceinline__ int write_lane(int v, int x, int j) {
  asm("s_mov_b32 m0, %2\n\ts_nop 0\n\tv_writelane_b32 %0, %1, m0"
      : "+v"(v) : "s"(x), "s"(j) : "m0");
  return v;
}

// k rounds over each lane's sorted candidates kc[0 .. N-1] (image
// descending, index ascending; image 0: none): the largest head is the next
// choice (equal images: the lowest index among the lanes holding it), and
// its owner pops its head.  Choice j's index and image go to lane j of
// my_idx and my_key; m_key is the image of the first choice (the largest
// logit).  CHECK: the lanes kept only their N best candidates; returns false
// if some lane ran out of them before the last round (its next one might
// still have been chosen).
template <int VPL, int N, int K, bool CHECK>
__device__ __forceinline__ bool route_rounds(uint32_t (&kc)[N], int (&ic)[N], int k, int lane,
                                             int &my_idx, uint32_t &my_key, uint32_t &m_key) {
  const uint64_t empty0 = CHECK ? ballot(kc[0] == 0u) : 0;  // lanes that never held one
  int owner = 0;
#pragma unroll
  for (int j = 0; j < (K > 0 ? K : k); ++j) {
    const uint32_t best = wave_max_u32(kc[0]);
    const uint64_t holders = ballot(kc[0] == best);
    int e;
    if (__popcll(holders) == 1) {
      owner = (int)__builtin_ctzll(holders);
      e = __builtin_amdgcn_readlane(ic[0], owner);
    } else {
      e = (int)wave_min_u32(kc[0] == best ? (uint32_t)ic[0] : 0xffffffffu);
      owner = e / VPL;
    }
    if (owner == lane) {
#pragma unroll
      for (int i = 0; i + 1 < N; ++i) {
        kc[i] = kc[i + 1];
        ic[i] = ic[i + 1];
      }
      kc[N - 1] = 0u;
    }
    if (j == 0) m_key = best;
    my_idx = write_lane(my_idx, e, j);
    my_key = (uint32_t)write_lane((int)my_key, (int)best, j);
  }
  if constexpr (CHECK) {
    // a lane out of candidates is fine only if it ran out in the last round
    const uint64_t out = ballot(kc[0] == 0u) & ~empty0 & ~(1ull << owner);
    return out == 0;
  }
  return true;
}

// One wave per token; lane l holds experts l*VPL .. l*VPL + VPL - 1 (one run
// of the logit row, so the loads are 8-byte pairs where E allows).  Experts
// past E are -inf logits: their image ties the lowest real one, and a tie
// goes to the lower index, so they are never chosen (k <= E), and their
// exp(-inf - m) adds nothing to the softmax sum.
// bias: NULL, or [E] fp32 added to every token's logits (one fp32 rounding).
// renorm: gates divided by their sum over the k chosen.
// K > 0: k == K, the rounds unrolled; K == 0: any k.
// With more than three candidates per lane the rounds first run on each
// lane's best three; in the rare case that a lane runs out of them with
// rounds left, they run again on every candidate.
template <int VPL, int K>
__global__ __launch_bounds__(256) void route_topk_softmax(const float *__restrict__ logits,
                                                          const float *__restrict__ bias,
                                                          int T, int E, int k, int renorm,
                                                          int32_t *__restrict__ topk,
                                                          float *__restrict__ gates) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const int lane = lane_id(), e0 = lane * VPL;
  const float *l = logits + (int64_t)t * E;

  // candidates of this lane: order-preserving image of the fp32 logit and
  // the expert index, sorted by (image descending, index ascending)
  float v[VPL];
  bool pairs = false;
  if constexpr (VPL % 2 == 0) pairs = (E % 2) == 0 && e0 + VPL <= E;  // 8-byte aligned pairs
  if (pairs) {
    const float2 *lp = reinterpret_cast<const float2 *>(l + e0);
#pragma unroll
    for (int i = 0; i < VPL / 2; ++i) {
      const float2 x = lp[i];
      v[2 * i] = x.x;
      v[2 * i + 1] = x.y;
    }
    if (bias) {
      const float2 *bp = reinterpret_cast<const float2 *>(bias + e0);
#pragma unroll
      for (int i = 0; i < VPL / 2; ++i) {
        const float2 x = bp[i];
        v[2 * i] += x.x;
        v[2 * i + 1] += x.y;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = e0 + i;
      v[i] = e < E ? (bias ? l[e] + bias[e] : l[e]) : -INFINITY;
    }
  }
  uint32_t key[VPL];
  int idx[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    key[i] = ord_f32(v[i]);
    idx[i] = e0 + i;
  }
#pragma unroll
  for (int i = 1; i < VPL; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {  // stable: equal images keep index order
      const bool sw = key[j] > key[j - 1];
      const uint32_t ka = key[j - 1], kb = key[j];
      const int ia = idx[j - 1], ib = idx[j];
      key[j - 1] = sw ? kb : ka;
      key[j] = sw ? ka : kb;
      idx[j - 1] = sw ? ib : ia;
      idx[j] = sw ? ia : ib;
    }

  int my_idx = 0;
  uint32_t my_key = 0u, m_key = 0u;
  if constexpr (K > 0) k = K;
  if constexpr (VPL > 3) {
    uint32_t hk[3] = {key[0], key[1], key[2]};
    int hi[3] = {idx[0], idx[1], idx[2]};
    if (!route_rounds<VPL, 3, K, true>(hk, hi, k, lane, my_idx, my_key, m_key))
      route_rounds<VPL, VPL, K, false>(key, idx, k, lane, my_idx, my_key, m_key);
  } else {
    route_rounds<VPL, VPL, K, false>(key, idx, k, lane, my_idx, my_key, m_key);
  }
  // softmax denominator over all E logits, then the gates of the k chosen
  const float m = unord_f32(m_key);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) s += __expf(v[i] - m);
  s = wave_sum_dpp(s);
  const float ej = __expf(unord_f32(my_key) - m);
  // renorm: the k chosen probabilities over their sum, i.e. the softmax over
  // the chosen logits, from exp(l - the first choice's logit), in fp32
  const float g = renorm ? ej / wave_sum_dpp(lane < k ? ej : 0.f) : ej / s;
  if (lane < k) {
    topk[(int64_t)t * k + lane] = my_idx;
    gates[(int64_t)t * k + lane] = g;
  }
}

template <int VPL>
static int launch_route(const float *logits, const float *bias, int T, int E, int k,
                        int renorm, int32_t *topk, float *gates, hipStream_t s) {
  return launch("route_topk_softmax", k == 8 ? route_topk_softmax<VPL, 8> : route_topk_softmax<VPL, 0>,
                dim3((unsigned)cdiv(T, 4)), dim3(256), 0, s, logits, bias, T, E, k, renorm, topk,
                gates);
}

static int route(const float *logits, const float *bias, int32_t T, int32_t E, int32_t k,
                 int renorm, int32_t *topk, float *gates, hipStream_t s) {
  if (T < 1 || E < 1 || k < 1 || k > E)
    return fail(MOE_ERR_INVALID, "moe_route: need T >= 1 and 1 <= k <= E");
  if (E > 1024 || k > 32) return fail(MOE_ERR_UNSUPPORTED, "moe_route: E <= 1024, k <= 32");
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk, "topk"));
  MOE_TRY(check_ptr(gates, "gates"));
  const int vpl = (int)cdiv(E, 64);
  if (vpl <= 1) return launch_route<1>(logits, bias, T, E, k, renorm, topk, gates, s);
  if (vpl <= 2) return launch_route<2>(logits, bias, T, E, k, renorm, topk, gates, s);
  if (vpl <= 4) return launch_route<4>(logits, bias, T, E, k, renorm, topk, gates, s);
  if (vpl <= 6) return launch_route<6>(logits, bias, T, E, k, renorm, topk, gates, s);
  if (vpl <= 8) return launch_route<8>(logits, bias, T, E, k, renorm, topk, gates, s);
  if (vpl <= 12) return launch_route<12>(logits, bias, T, E, k, renorm, topk, gates, s);
  return launch_route<16>(logits, bias, T, E, k, renorm, topk, gates, s);
}

// ---------------------------------------------------------------------------
// quantile balancing
// ---------------------------------------------------------------------------

constexpr int CNT_THREADS = 256, CNT_ITEMS = 16;  // items per thread

__global__ __launch_bounds__(256) void counts_clear(int32_t *counts, int E) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = 0;
}

// Choices (t, j) of one block's items counted in LDS (integer adds: the
// totals do not depend on the order), then added to counts.
__global__ __launch_bounds__(CNT_THREADS) void expert_counts(const int32_t *__restrict__ topk,
                                                             int64_t n, int E,
                                                             int32_t *__restrict__ counts) {
  __shared__ int32_t hist[1024];
  for (int e = threadIdx.x; e < E; e += CNT_THREADS) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * CNT_THREADS * CNT_ITEMS + threadIdx.x;
  int32_t v[CNT_ITEMS];
#pragma unroll
  for (int i = 0; i < CNT_ITEMS; ++i) {
    const int64_t it = base + (int64_t)i * CNT_THREADS;
    v[i] = it < n ? topk[it] : -1;
  }
#pragma unroll
  for (int i = 0; i < CNT_ITEMS; ++i)
    if ((unsigned)v[i] < (unsigned)E) atomicAdd(&hist[v[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += CNT_THREADS)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// Backward of the router, one wave per token.  With p = softmax(l) over all
// E (l = fp32(logit + bias), recomputed) and gate j = p[e_j]:
//   d_l[e] = sum_j d_gates[j] p[e_j] ([e == e_j] - p[e]);
// renormalised gates q = softmax over the k chosen logits:
//   d_l[e_j] = q_j (d_gates[j] - sum_i d_gates[i] q_i), 0 elsewhere.
template <int VPL>
__global__ __launch_bounds__(256) void route_backward_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int T, int E, int k,
    int renorm, const int32_t *__restrict__ topk, const float *__restrict__ d_gates,
    float *__restrict__ d_logits) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const float *l = logits + (int64_t)t * E;
  int my_e = -1;
  float my_dg = 0.f, my_l = -INFINITY;
  if (lane < k) {
    const int e = topk[(int64_t)t * k + lane];
    my_dg = d_gates[(int64_t)t * k + lane];
    if ((unsigned)e < (unsigned)E) {
      my_e = e;
      my_l = bias ? l[e] + bias[e] : l[e];
    }
  }
  float out[VPL];
  float add;  // this lane's chosen expert's own term
  if (!renorm) {
    float v[VPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? (bias ? l[e] + bias[e] : l[e]) : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = wave_max_f32(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) z += (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
    z = wave_sum_f32(z);
    const float pj = my_e >= 0 ? expf(my_l - m) / z : 0.f;
    add = my_dg * pj;
    const float s = wave_sum_f32(add);
#pragma unroll
    for (int i = 0; i < VPL; ++i) out[i] = -(expf(v[i] - m) / z) * s;
  } else {
    const float mk = wave_max_f32(my_l);
    const float ej = my_e >= 0 ? expf(my_l - mk) : 0.f;
    const float q = ej / wave_sum_f32(ej);
    const float s = wave_sum_f32(my_dg * q);
    add = my_e >= 0 ? q * (my_dg - s) : 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) out[i] = 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int ej = __shfl(my_e, j);
    const float aj = __shfl(add, j);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i == ej) out[i] += aj;
  }
  float *o = d_logits + (int64_t)t * E;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (lane + 64 * i < E) o[lane + 64 * i] = out[i];
}

template <int VPL>
static int launch_route_bwd(const float *logits, const float *bias, int T, int E, int k,
                            int renorm, const int32_t *topk, const float *d_gates,
                            float *d_logits, hipStream_t s) {
  return launch("route_backward", route_backward_kernel<VPL>, dim3((unsigned)cdiv(T, 4)),
                dim3(256), 0, s, logits, bias, T, E, k, renorm, topk, d_gates, d_logits);
}

// One block: H_i = sum over the window's batches, f_i = H_i / sum H (1/E when
// nothing was chosen), b_i = -alpha (f_i - 1/E), in double, rounded to fp32.
__global__ __launch_bounds__(1024) void balance_bias(const int32_t *__restrict__ window, int nb,
                                                     int E, double alpha,
                                                     float *__restrict__ bias) {
  __shared__ int64_t part[1024 / 64];
  const int i = threadIdx.x;
  int64_t h = 0;
  if (i < E)
    for (int b = 0; b < nb; ++b) h += window[(int64_t)b * E + i];
  int64_t w = h;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)w, m), hi = __shfl_xor((uint32_t)((uint64_t)w >> 32), m);
    w += (int64_t)(((uint64_t)hi << 32) | lo);
  }
  if (lane_id() == 0) part[i >> 6] = w;
  __syncthreads();
  int64_t total = 0;
  for (int q = 0; q < (int)(blockDim.x >> 6); ++q) total += part[q];
  if (i < E) {
    const double f = total > 0 ? (double)h / (double)total : 1.0 / (double)E;
    bias[i] = (float)(-alpha * (f - 1.0 / (double)E));
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk,
                         float *gates, void *stream) {
  clear_error();
  return route(logits, nullptr, T, E, k, 0, topk, gates, (hipStream_t)stream);
}

extern "C" int moe_route_biased(const float *logits, const float *bias, int32_t T, int32_t E,
                                int32_t k, int32_t flags, int32_t *topk, float *gates,
                                void *stream) {
  clear_error();
  MOE_TRY(check_ptr(bias, "bias", true));
  if (flags & ~MOE_ROUTE_RENORM) return fail(MOE_ERR_INVALID, "moe_route_biased: unknown flags");
  return route(logits, bias, T, E, k, (flags & MOE_ROUTE_RENORM) != 0, topk, gates,
               (hipStream_t)stream);
}

extern "C" int moe_expert_counts(const int32_t *topk, int32_t T, int32_t k, int32_t E,
                                 int32_t *counts, void *stream) {
  clear_error();
  if (T < 1 || k < 1 || E < 1) return fail(MOE_ERR_INVALID, "moe_expert_counts: sizes must be >= 1");
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_expert_counts: E <= 1024");
  if ((int64_t)T * k >= (1ll << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_counts: T * k must fit in int32");
  MOE_TRY(check_ptr(topk, "topk"));
  MOE_TRY(check_ptr(counts, "counts"));
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)T * k;
  MOE_TRY(launch("counts_clear", counts_clear, dim3(1), dim3(256), 0, s, counts, E));
  return launch("expert_counts", expert_counts,
                dim3((unsigned)cdiv(n, (int64_t)CNT_THREADS * CNT_ITEMS)), dim3(CNT_THREADS), 0,
                s, topk, n, E, counts);
}

extern "C" int moe_balance_bias(const int32_t *window, int32_t n_batches, int32_t E,
                                double alpha, float *bias, void *stream) {
  clear_error();
  if (n_batches < 1 || E < 1) return fail(MOE_ERR_INVALID, "moe_balance_bias: sizes must be >= 1");
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_balance_bias: E <= 1024");
  if (!(alpha == alpha)) return fail(MOE_ERR_INVALID, "moe_balance_bias: alpha is NaN");
  MOE_TRY(check_ptr(window, "window"));
  MOE_TRY(check_ptr(bias, "bias"));
  return launch("balance_bias", balance_bias, dim3(1), dim3(1024), 0, (hipStream_t)stream,
                window, n_batches, E, alpha, bias);
}

extern "C" int moe_route_backward(const float *logits, const float *bias, int32_t T, int32_t E,
                                  int32_t k, int32_t flags, const int32_t *topk,
                                  const float *d_gates, float *d_logits, void *stream) {
  clear_error();
  if (T < 1 || E < 1 || k < 1 || k > E)
    return fail(MOE_ERR_INVALID, "moe_route_backward: need T >= 1 and 1 <= k <= E");
  if (E > 1024 || k > 32) return fail(MOE_ERR_UNSUPPORTED, "moe_route_backward: E <= 1024, k <= 32");
  if (flags & ~MOE_ROUTE_RENORM) return fail(MOE_ERR_INVALID, "moe_route_backward: unknown flags");
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(bias, "bias", true));
  MOE_TRY(check_ptr(topk, "topk"));
  MOE_TRY(check_ptr(d_gates, "d_gates"));
  MOE_TRY(check_ptr(d_logits, "d_logits"));
  const int rn = (flags & MOE_ROUTE_RENORM) != 0;
  hipStream_t s = (hipStream_t)stream;
  const int vpl = (int)cdiv(E, 64);
  if (vpl <= 1) return launch_route_bwd<1>(logits, bias, T, E, k, rn, topk, d_gates, d_logits, s);
  if (vpl <= 2) return launch_route_bwd<2>(logits, bias, T, E, k, rn, topk, d_gates, d_logits, s);
  if (vpl <= 4) return launch_route_bwd<4>(logits, bias, T, E, k, rn, topk, d_gates, d_logits, s);
  if (vpl <= 6) return launch_route_bwd<6>(logits, bias, T, E, k, rn, topk, d_gates, d_logits, s);
  if (vpl <= 8) return launch_route_bwd<8>(logits, bias, T, E, k, rn, topk, d_gates, d_logits, s);
  if (vpl <= 12)
    return launch_route_bwd<12>(logits, bias, T, E, k, rn, topk, d_gates, d_logits, s);
  return launch_route_bwd<16>(logits, bias, T, E, k, rn, topk, d_gates, d_logits, s);
}
