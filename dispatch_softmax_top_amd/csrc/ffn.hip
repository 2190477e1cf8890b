// ffn.hip -- routed experts: every local expert runs on its bank rows, each
// wave ("从玩具到前沿:训练一个真正的大模型,到底难在哪里", devpress.csdn.net,
// section 四 and appendix A.3).  The expert's form is not fixed by the pages;
// a SwiGLU is used: y = bf16( bf16(silu(u.W_g) * (u.W_u)) . W_d ).
//
// Kernels, in stream order:
//   ffn_flags_clear / ffn_flags_mark  which return rows will receive a result
//                        (the clear also zeroes the GEMMs' queue counters)
//   gemm_expert_swiglu   grouped over (wave, expert) bank groups -> h (ws)
//   gemm_expert_down     grouped, rows scattered to their receive position
//   ffn_zero_rows        every other return row set to zero
#include <algorithm>

#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void ffn_flags_clear(int32_t *flags, int64_t n, int32_t *zero16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) flags[i] = 0;
  if (zero16 && i < 16) zero16[i] = 0;
}

__global__ __launch_bounds__(256) void ffn_flags_mark(const int32_t *__restrict__ bank_src,
                                                      int64_t n_bank, int32_t *flags,
                                                      int64_t n_ret) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_bank) return;
  const int r = bank_src[i];
  if (r >= 0 && r < n_ret) flags[r] = 1;
}

__global__ __launch_bounds__(256) void ffn_zero_rows(const int32_t *__restrict__ flags,
                                                     uint16_t *__restrict__ ret, int L,
                                                     int64_t n_ret) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_ret || flags[row]) return;
  u32x4 *out = reinterpret_cast<u32x4 *>(ret + row * L);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int c = lane_id(); c < L / 8; c += 64) out[c] = zero;
}

int ret_rows_mark(const int32_t *bank_src, int64_t n_bank, int32_t *flags, int64_t n_ret,
                  int32_t *zero16, hipStream_t s) {
  const int64_t blocks = std::max<int64_t>(cdiv(n_ret, 256), zero16 ? 1 : 0);
  MOE_TRY(launch("ffn_flags_clear", ffn_flags_clear, dim3((unsigned)blocks), dim3(256), 0, s,
                 flags, n_ret, zero16));
  return launch("ffn_flags_mark", ffn_flags_mark, dim3((unsigned)cdiv(n_bank, 256)), dim3(256), 0,
                s, bank_src, n_bank, flags, n_ret);
}

int ret_rows_zero_unmarked(const int32_t *flags, uint16_t *ret, int L, int64_t n_ret,
                           hipStream_t s) {
  return launch("ffn_zero_rows", ffn_zero_rows, dim3((unsigned)cdiv(n_ret, 4)), dim3(256), 0, s,
                flags, ret, L, n_ret);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_expert_ffn(const moe_dims *d, const moe_bf16 *bank, const int64_t *bank_offsets,
                              const int32_t *bank_src, const int32_t *bfill, int64_t n_bank_rows,
                              const moe_bf16 *w_gate, const moe_bf16 *w_up,
                              const moe_bf16 *w_down, moe_bf16 *ret, int64_t n_ret_rows,
                              void *ws, int64_t ws_bytes, void *stream) {
  clear_error();
  MOE_TRY(check_dims(d));
  const bool rg = ragged(*d);
  MOE_TRY(check_ptr(bank, "bank"));
  MOE_TRY(check_ptr(bank_src, "bank_src"));
  MOE_TRY(check_ptr(bfill, "bfill"));
  MOE_TRY(check_ptr(w_gate, "w_gate"));
  MOE_TRY(check_ptr(w_up, "w_up"));
  MOE_TRY(check_ptr(w_down, "w_down"));
  MOE_TRY(check_ptr(ret, "ret"));
  MOE_TRY(check_ptr(ws, "ws"));
  if (rg) {
    MOE_TRY(check_ptr(bank_offsets, "bank_offsets (ragged mode)"));
    if (n_bank_rows < 0 || n_bank_rows >= (1ll << 31) || n_ret_rows < 0 ||
        n_ret_rows >= (1ll << 31))
      return fail(MOE_ERR_INVALID, "moe_expert_ffn: row counts out of range");
  } else {
    if (n_bank_rows != (int64_t)d->n_waves * experts_per_rank(*d) * d->cap_recv)
      return fail(MOE_ERR_INVALID, "moe_expert_ffn: fixed mode needs n_bank_rows == n_waves*E_l*cap_recv");
    if (n_ret_rows != (int64_t)d->n_ranks * d->n_waves * d->cap_send * ret_slots(*d))
      return fail(MOE_ERR_INVALID, "moe_expert_ffn: fixed mode needs n_ret_rows == n_ranks*n_waves*cap_send (*4 with dedup)");
  }
  const int64_t need = moe_workspace_bytes(d, MOE_CALL_FFN, n_bank_rows);
  if (need < 0) return (int)need;
  if (rg && n_ret_rows > n_bank_rows)
    return fail(MOE_ERR_INVALID, "moe_expert_ffn: ragged mode needs n_ret_rows <= n_bank_rows");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace %lld < %lld bytes",
                (long long)ws_bytes, (long long)need);
  hipStream_t s = (hipStream_t)stream;
  // workspace: intermediate h, return-row flags, the GEMMs' work queue,
  // partial tiles of their split last rounds (shared by both: stream order)
  const int64_t ret_rows = rg ? n_bank_rows : n_ret_rows;
  uint16_t *H = (uint16_t *)ws;
  int32_t *flags = (int32_t *)((char *)ws + ffn_h_bytes(*d, n_bank_rows));
  int32_t *queue = (int32_t *)((char *)flags + ffn_flag_bytes(ret_rows));
  float *part = (float *)((char *)queue + gemm_queue_bytes());

  MOE_TRY(ret_rows_mark(bank_src, n_bank_rows, flags, n_ret_rows, queue, s));
  MOE_TRY(gemm_expert_swiglu(*d, bank, bank_offsets, bfill, n_bank_rows, w_gate, w_up, H, part,
                             queue, s));
  MOE_TRY(gemm_expert_down(*d, H, bank_offsets, bfill, bank_src, n_bank_rows, w_down, ret,
                           n_ret_rows, part, queue, s));
  return ret_rows_zero_unmarked(flags, ret, d->latent, n_ret_rows, s);
}
