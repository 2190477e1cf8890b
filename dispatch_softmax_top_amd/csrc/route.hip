// route.hip -- router: softmax over all experts, then the top k.
//
// "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK), section 二,
// and "从玩具到前沿:训练一个真正的大模型,到底难在哪里" (devpress.csdn.net),
// section 四: every token is routed to 8 of 384 experts.
//
// One wave64 per token.  Lane l holds logits l, l+64, l+128, ... .  The
// choice order is (logit descending, index ascending): each candidate is
// encoded as a 64-bit key (order-preserving image of the fp32 value, then
// the complement of the index) so one unsigned max picks the next expert.
// Each lane keeps its candidates sorted; k rounds of a wave-wide max take
// the head of the winning lane.  Gates are exp(l - max) / sum exp(l - max)
// over all E logits, in fp32.
#include <math.h>

#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal logits compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_topk_softmax(const float *__restrict__ logits,
                                                          int T, int E, int k,
                                                          int32_t *__restrict__ topk,
                                                          float *__restrict__ gates) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const int lane = lane_id();
  const float *l = logits + (int64_t)t * E;

  float v[VPL];
  uint64_t key[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? l[e] : -INFINITY;
    m = fmaxf(m, v[i]);
    key[i] = e < E ? (((uint64_t)ord_f32(v[i]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e)) : 0ull;
  }
  m = wave_max_f32(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) s += (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
  s = wave_sum_f32(s);

  // sort this lane's keys, largest first (insertion sort, unrolled)
#pragma unroll
  for (int i = 1; i < VPL; ++i) {
#pragma unroll
    for (int j = i; j > 0; --j) {
      uint64_t a = key[j - 1], b = key[j];
      key[j - 1] = a > b ? a : b;
      key[j] = a > b ? b : a;
    }
  }

  int my_idx = 0;
  float my_gate = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = wave_max_u64(key[0]);
    uint32_t e = 0xffffffffu - (uint32_t)best;
    if ((int)(e & 63u) == lane) {  // owner pops its head
#pragma unroll
      for (int i = 0; i + 1 < VPL; ++i) key[i] = key[i + 1];
      key[VPL - 1] = 0ull;
    }
    if (lane == j) {
      my_idx = (int)e;
      my_gate = expf(unord_f32((uint32_t)(best >> 32)) - m) / s;
    }
  }
  if (lane < k) {
    topk[(int64_t)t * k + lane] = my_idx;
    gates[(int64_t)t * k + lane] = my_gate;
  }
}

template <int VPL>
static int launch_route(const float *logits, int T, int E, int k, int32_t *topk, float *gates,
                        hipStream_t s) {
  return launch("route_topk_softmax", route_topk_softmax<VPL>, dim3((unsigned)cdiv(T, 4)),
                dim3(256), 0, s, logits, T, E, k, topk, gates);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk,
                         float *gates, void *stream) {
  clear_error();
  if (T < 1 || E < 1 || k < 1 || k > E)
    return fail(MOE_ERR_INVALID, "moe_route: need T >= 1 and 1 <= k <= E");
  if (E > 1024 || k > 32) return fail(MOE_ERR_UNSUPPORTED, "moe_route: E <= 1024, k <= 32");
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk, "topk"));
  MOE_TRY(check_ptr(gates, "gates"));
  hipStream_t s = (hipStream_t)stream;
  int vpl = (int)cdiv(E, 64);
  if (vpl <= 1) return launch_route<1>(logits, T, E, k, topk, gates, s);
  if (vpl <= 2) return launch_route<2>(logits, T, E, k, topk, gates, s);
  if (vpl <= 4) return launch_route<4>(logits, T, E, k, topk, gates, s);
  if (vpl <= 6) return launch_route<6>(logits, T, E, k, topk, gates, s);
  if (vpl <= 8) return launch_route<8>(logits, T, E, k, topk, gates, s);
  if (vpl <= 12) return launch_route<12>(logits, T, E, k, topk, gates, s);
  return launch_route<16>(logits, T, E, k, topk, gates, s);
}
