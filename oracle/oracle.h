/*
 * oracle.h -- plain single-threaded CPU reference of one GPU's share of the
 * pooled-wave MoE dispatch path.
 *
 * TEST INFRASTRUCTURE ONLY.  It is called from tests, from the smoke check
 * and from the CPU-baseline leg of the benchmark, never from the product
 * path.  It shares no code, header or table with the HIP library.
 *
 * Sources, cited by page title and section:
 *   [P2] "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK)
 *   [P3] "Marin、535BパラメータMoEモデルのオープントレーニングを開始"
 *        (lamjinlab.com, ja) -- a paragraph-by-paragraph translation of [P2]
 *   [P1] "从玩具到前沿:训练一个真正的大模型,到底难在哪里" (devpress.csdn.net)
 *
 * Layouts (row-major, element units unless stated):
 *   bf16 values are passed as uint16_t bit patterns.
 *   Weights are stored output-major ("out x in"): a weight W of the product
 *   y = x.W with W of shape [in, out] is stored as W^T, shape [out, in].
 *   A pool / receive row is `latent` bf16 values followed by a 16-byte tail
 *   {int32 global expert id (-1 = empty slot), 0, 0, 0}.
 *   Fixed mode (cap_send, cap_recv > 0):
 *     pools [R][W][cap_send] rows, recv [R_src][W][cap_send] rows,
 *     bank [W][E_l][cap_recv][latent], ret [R][W][cap_send][latent].
 *   Ragged mode (cap_send == cap_recv == 0): segments at int64 offsets,
 *     pools in (dest, wave) order, recv/ret in (source, wave) order,
 *     bank in (wave, local expert) order; each offsets array has one entry
 *     per segment plus a final total.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* wave_mode 0: wave(t) = t / T_w, one pool of cap_send rows per (dest,
 * wave).  wave_mode 1 (the other reading of the waves, fixed mode only): one
 * pool of n_waves*cap_send rows per dest, filled in (token, choice) order and
 * cut into n_waves chunks of cap_send rows; chunk w is wave w.  The layout
 * [R][W][cap_send] is the same; slot is then the position in the dest's pool.
 * dedup 1 (a variant, fixed mode only): a token sends one row per group of up
 * to four of its choices on one destination; the row's tail holds their ids
 * in choice order (-1 for unused), every member's slot is the row's position,
 * and returns come back in four slots per receive row ([rows][4][latent]). */
typedef struct {
  int32_t T, d_model, latent, n_experts, n_ranks, top_k, n_waves, d_ff,
      n_shared, d_ff_shared, cap_send, cap_recv, wave_mode, dedup;
} orc_dims;

/* bf16 <-> double, round to nearest even, straight from double. */
uint16_t orc_bf16_from_double(double v);
double orc_bf16_to_double(uint16_t b);

int32_t orc_tokens_per_wave(int32_t T, int32_t n_waves);
/* ceil(cf * tokens_per_wave * top_k / groups) in exact integer arithmetic,
 * cf = cf_num / cf_den.  groups = n_ranks (sender) or E_l (receiver). */
int64_t orc_capacity(int64_t tokens_per_wave, int32_t top_k, int32_t groups,
                     int64_t cf_num, int64_t cf_den);

void orc_route(const float *logits, int64_t T, int32_t E, int32_t k,
               int32_t *topk, float *gates);

void orc_route_biased(const float *logits, const float *bias, int64_t T,
                      int32_t E, int32_t k, int32_t *topk, float *gates);
void orc_route_ex(const float *logits, const float *bias, int64_t T,
                  int32_t E, int32_t k, int32_t renorm, int32_t *topk,
                  float *gates);
void orc_expert_counts(const int32_t *topk, int64_t n, int32_t E,
                       int32_t *counts);
void orc_balance_bias(const int32_t *window, int32_t n_batches, int32_t E,
                      double alpha, float *bias);

void orc_latent_rows(const uint16_t *x, int32_t D, const uint16_t *w_ld_t,
                     int32_t L, const int64_t *rows, int64_t n, uint16_t *z);

int64_t orc_sender(const orc_dims *d, const int32_t *topk, int32_t *slot,
                   int32_t *fill, int32_t *demand, int64_t *pool_offsets);

void orc_pack_rows(const orc_dims *d, const uint16_t *z, const int32_t *topk,
                   const int32_t *slot, const int64_t *pool_offsets,
                   uint8_t *pools, int64_t n_pool_rows);

/* hdr: one tail id per receive row, or with dedup the four ids of each row
 * ([n_recv_rows][4]); with dedup bank_src holds return slots (row * 4 + id
 * index). */
int64_t orc_bank_slots(const orc_dims *d, int32_t rank, const int32_t *hdr,
                       const int64_t *recv_offsets, int64_t n_recv_rows,
                       int64_t *bank_offsets, int32_t *bank_src,
                       int32_t *bfill, int32_t *bdemand, int32_t *bad_rows);

/* Tail id of one pool / receive row; all four tail ids. */
int32_t orc_row_header(const uint8_t *row, int32_t L);
void orc_row_ids(const uint8_t *row, int32_t L, int32_t *ids);

void orc_bank_rows(const orc_dims *d, const uint8_t *recv,
                   const int64_t *bank_offsets, const int32_t *bank_src,
                   const int32_t *bfill, uint16_t *bank);

void orc_ffn_row(int32_t L, int32_t F, const uint16_t *u, const uint16_t *wg_t,
                 const uint16_t *wu_t, const uint16_t *wd_t, uint16_t *y);

void orc_expert_ffn(const orc_dims *d, const uint16_t *bank,
                    const int64_t *bank_offsets, const int32_t *bank_src,
                    const int32_t *bfill, const uint16_t *w_gate,
                    const uint16_t *w_up, const uint16_t *w_down,
                    uint16_t *ret, int64_t n_ret_rows);

void orc_combine_tokens(const orc_dims *d, const uint16_t *returned,
                        const int64_t *ret_offsets, const int32_t *topk,
                        const int32_t *slot, const float *gates,
                        const uint16_t *x, const uint16_t *w_lu_t,
                        const uint16_t *ws_gate, const uint16_t *ws_up,
                        const uint16_t *ws_down, const int64_t *tokens,
                        int64_t n, uint16_t *ylat, uint16_t *out);

/* Backward of the branch.  Layouts as in the forward calls; d_shared is
 * [T][2][n_shared][d_ff_shared]: the gradients of the shared experts' gate
 * products, then of their up products.  Ragged mode (cap_send == 0):
 * returned / d_returned and d_pools have segments (destination, wave) at
 * ret_offsets / pool_offsets [n_ranks*n_waves + 1], and a slot at or past
 * its segment's length has no row (the forward read it as zero: its gate
 * gradient is 0 and nothing is written); the bank's groups start at
 * bank_offsets.  The offsets are ignored (may be NULL) in fixed mode.
 * n_ret_rows: rows of returned and d_returned. */
void orc_route_backward(const float *logits, const float *bias, int64_t T,
                        int32_t E, int32_t k, int32_t renorm,
                        const int32_t *topk, const float *d_gates,
                        float *d_logits);
void orc_combine_backward(const orc_dims *d, const uint16_t *returned,
                          const int64_t *ret_offsets, int64_t n_ret_rows,
                          const int32_t *topk, const int32_t *slot,
                          const float *gates, const uint16_t *x,
                          const uint16_t *ylat, const uint16_t *w_lu_t,
                          const uint16_t *ws_gate, const uint16_t *ws_up,
                          const uint16_t *ws_down, const uint16_t *d_out,
                          uint16_t *d_returned, float *d_gates,
                          uint16_t *d_shared, uint16_t *dw_lat_up,
                          uint16_t *dws_down);
void orc_expert_ffn_backward(const orc_dims *d, const uint16_t *bank,
                             const int64_t *bank_offsets,
                             const int32_t *bank_src, const int32_t *bfill,
                             const uint16_t *w_gate, const uint16_t *w_up,
                             const uint16_t *w_down, const uint16_t *d_ret,
                             int64_t n_ret_rows, uint16_t *d_recv,
                             uint16_t *dw_gate, uint16_t *dw_up,
                             uint16_t *dw_down);
void orc_pack_backward(const orc_dims *d, const uint16_t *d_pools,
                       const int64_t *pool_offsets,
                       const int32_t *topk, const int32_t *slot,
                       const uint16_t *x, const uint16_t *d_shared,
                       const uint16_t *w_ld_t, const uint16_t *ws_gate,
                       const uint16_t *ws_up, uint16_t *dz, uint16_t *dx,
                       uint16_t *dw_lat_down, uint16_t *dws_gate,
                       uint16_t *dws_up);

/* Backward on sampled outputs: the same values as the full functions for
 * listed tokens, bank positions or weight entries (full-size checks). */
void orc_combine_backward_tokens(const orc_dims *d, const uint16_t *returned,
                                 const int64_t *ret_offsets,
                                 const int32_t *topk, const int32_t *slot,
                                 const float *gates, const uint16_t *x,
                                 const uint16_t *w_lu_t, const uint16_t *ws_gate,
                                 const uint16_t *ws_up, const uint16_t *ws_down,
                                 const uint16_t *d_out, const int64_t *tokens,
                                 int64_t n, uint16_t *d_ret_rows,
                                 float *d_gates, uint16_t *d_shared);
void orc_combine_wgrad_entries(const orc_dims *d, const uint16_t *x,
                               const uint16_t *ylat, const uint16_t *ws_gate,
                               const uint16_t *ws_up, const uint16_t *d_out,
                               int32_t which, const int32_t *sh_idx,
                               const int32_t *ra, const int32_t *cb, int64_t n,
                               uint16_t *out);
void orc_expert_ffn_backward_rows(const orc_dims *d, const uint16_t *bank,
                                  const int64_t *bank_offsets,
                                  const int32_t *bank_src,
                                  const uint16_t *w_gate, const uint16_t *w_up,
                                  const uint16_t *w_down, const uint16_t *d_ret,
                                  const int64_t *pos, int64_t n, uint16_t *d_u);
void orc_expert_wgrad_entries(const orc_dims *d, const uint16_t *bank,
                              const int64_t *bank_offsets,
                              const int32_t *bank_src, const int32_t *bfill,
                              const uint16_t *w_gate, const uint16_t *w_up,
                              const uint16_t *w_down, const uint16_t *d_ret,
                              int32_t j, int32_t which, const int32_t *ra,
                              const int32_t *cb, int64_t n, uint16_t *out);
void orc_pack_backward_tokens(const orc_dims *d, const uint16_t *d_pools,
                              const int64_t *pool_offsets,
                              const int32_t *topk, const int32_t *slot,
                              const uint16_t *d_shared, const uint16_t *w_ld_t,
                              const uint16_t *ws_gate, const uint16_t *ws_up,
                              const int64_t *tokens, int64_t n, uint16_t *dz,
                              uint16_t *dx);
void orc_pack_wgrad_entries(const orc_dims *d, const uint16_t *d_pools,
                            const int64_t *pool_offsets,
                            const int32_t *topk, const int32_t *slot,
                            const uint16_t *x, const uint16_t *d_shared,
                            int32_t which, const int32_t *sh_idx,
                            const int32_t *ra, const int32_t *cb, int64_t n,
                            uint16_t *out);

#ifdef __cplusplus
}
#endif
#endif
