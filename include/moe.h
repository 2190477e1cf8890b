/*
 * moe.h -- C ABI of libmoe.so: one GPU's share of a pooled-wave
 * mixture-of-experts dispatch path, hand-written HIP for gfx950 (MI355X).
 *
 * Sources, cited by page title and section:
 *   [P2] "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK)
 *   [P3] "Marin、535BパラメータMoEモデルのオープントレーニングを開始"
 *        (lamjinlab.com, ja) -- translation of [P2]
 *   [P1] "从玩具到前沿:训练一个真正的大模型,到底难在哪里" (devpress.csdn.net)
 *
 * The path, per source shard of T tokens ([P2]/[P3] section 二):
 *   moe_route       softmax over E routed experts, top-k choice and gates
 *   moe_pack_waves  latent down-projection, then one fixed pool per
 *                   destination rank and wave, expert id inside each row,
 *                   sender capacity, overflow dropped and counted
 *   (exchange)      outside this library: the caller moves pools to the
 *                   destination ranks' receive buffers
 *   moe_bank        rows received for this rank banked per wave and local
 *                   expert, receiver capacity, overflow dropped and counted
 *   moe_expert_ffn  every local expert run on its bank rows, each wave
 *   (return)        outside this library
 *   moe_combine     gate-weighted sum of each token's returned rows, latent
 *                   up-projection, plus the shared experts
 * and, for training, the same stages backward: moe_combine_backward,
 * moe_route_backward, moe_expert_ffn_backward, moe_pack_backward.
 * Quantile balancing of the routing: moe_route_biased, moe_expert_counts,
 * moe_balance_bias.
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers, 16-byte aligned, owned by the
 *     caller.  The library never allocates, frees or synchronises inside a
 *     hot-path call; scratch comes only through (ws, ws_bytes).
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = null stream)
 *     and return at once.  Calls on distinct buffers are re-entrant.
 *   - bf16 tensors are passed as uint16_t bit patterns (moe_bf16).
 *   - Weights are output-major: the weight W of y = x.W (W of shape
 *     [in, out]) is stored as W^T, shape [out, in], row-major.
 *   - A pool / receive row is `latent` bf16 values followed by a 16-byte
 *     tail {int32 global expert id, 0, 0, 0}; id -1 marks an empty slot
 *     (its payload bytes are unspecified).  Row stride = 2*latent + 16.
 *     With moe_dims.dedup the tail holds four ids (see moe_dims).
 *   - Fixed mode (cap_send > 0 and cap_recv > 0):
 *       pools  [n_ranks][n_waves][cap_send] rows   (destination, wave, slot)
 *       recv   [n_ranks][n_waves][cap_send] rows   (source, wave, slot)
 *       bank   [n_waves][E_l][cap_recv][latent]    (wave, local expert, pos)
 *       ret    [n_ranks][n_waves][cap_send][latent] (recv layout, no tail)
 *     Ragged / dropless mode (cap_send == cap_recv == 0): the same orders,
 *     but each (outer, wave) segment has its own length and starts at an
 *     int64 offset; an offsets array has one entry per segment plus the
 *     total at the end.
 *   - Waves (wave_mode MOE_WAVES_TOKENS) split a shard's tokens into
 *     contiguous runs: wave(t) = floor(t / T_w), T_w = ceil(T / n_waves).
 *     With MOE_WAVES_CHUNKS (fixed mode only) the waves instead cut one
 *     pool of n_waves*cap_send rows per destination into n_waves chunks:
 *     an assignment's slot is its position in the destination's pool and
 *     its wave is slot / cap_send.  The buffer layouts above are the same
 *     in both modes (pool (dest, w) is chunk w).  Expert e lives on rank
 *     floor(e / E_l) as local expert e mod E_l, E_l = n_experts / n_ranks.
 *   - Every output is fully written except where stated unspecified.
 *   - Errors: arguments are checked on the host before any launch; a
 *     negative moe_status is returned and moe_last_error() (per thread)
 *     says why.  Nothing is enqueued when a call returns an error.
 *     Data-dependent faults found on the device (a receive row whose id is
 *     neither -1 nor hosted by `rank`) are counted, never trapped.
 *   - Environment: MOE_GEMM_CUS, if set, is the number of compute units the
 *     GEMM launchers plan for when it is below the device's (a multiple of
 *     8, at least 8; anything else makes every call that takes moe_dims
 *     return MOE_ERR_INVALID).  It sets the persistent GEMMs' grids (one
 *     block per planned CU, so a caller can leave CUs to kernels on other
 *     streams) and which last rounds are split along K.  Outputs of GEMM
 *     tiles that are not split do not depend on it; a split tile's fp32
 *     partial sums are added in a fixed order, but in another grouping than
 *     the unsplit tile's, so its bf16 results may differ in the last bit.
 */
#ifndef MOE_H
#define MOE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7

typedef uint16_t moe_bf16;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* bad pointer, size or layout */
  MOE_ERR_UNSUPPORTED = -2, /* valid, but outside what the kernels handle */
  MOE_ERR_HIP = -3,         /* the HIP runtime reported an error */
  MOE_ERR_WORKSPACE = -4    /* ws too small */
} moe_status;

/* Sizes of one layer share.  cap_send / cap_recv: rows per
 * (destination, wave) pool and per (wave, local expert) bank; both 0 selects
 * ragged / dropless mode.  Supported: n_experts % n_ranks == 0,
 * n_experts <= 1024, 1 <= top_k <= min(32, n_experts), latent % 64 == 0,
 * latent <= 8192, T <= 2^27, T * top_k < 2^31,
 * d_model % 64 == 0, d_ff % 128 == 0, d_ff_shared % 128 == 0,
 * n_ranks * n_waves <= 1024, n_waves * E_l <= 1024, n_shared <= 4.
 * wave_mode: MOE_WAVES_TOKENS (0) or MOE_WAVES_CHUNKS (1, needs fixed
 * mode); the two readings of how a shard is sent in waves.
 * dedup: 0, or 1 for the variant where a token's choices on one destination
 * share rows: one row per group of up to four of them (in choice order),
 * whose tail holds their four global ids {e0, e1, e2, e3} (-1 unused; an
 * empty row is all -1).  Every member's slot is its row's position; pool
 * capacities count rows.  The bank takes one item per id, in (source, row,
 * id index) order; bank_src then holds return slots (receive row * 4 + id
 * index) and the return buffer has four latent rows per receive row
 * ([n_recv_rows * 4][latent]); the combine reads slot row * 4 + (the
 * choice's index among the token's same-destination choices) % 4.  Fixed
 * mode only; the backward calls do not take it. */
typedef struct {
  int32_t T, d_model, latent, n_experts, n_ranks, top_k, n_waves, d_ff,
      n_shared, d_ff_shared, cap_send, cap_recv, wave_mode, dedup;
} moe_dims;

enum { MOE_WAVES_TOKENS = 0, MOE_WAVES_CHUNKS = 1 };

int moe_abi_version(void);

/* Text of the last error raised on the calling thread ("" if none). */
const char *moe_last_error(void);

/* Capacities from rational capacity factors cf = num/den ([P2]/[P3]
 * section 二: the sender factor caps rows from one source to one destination,
 * the receiver factor caps rows of one local expert).  Each factor multiplies
 * the mean load of its buffer for one wave -- T_w*k/n_ranks rows per pool and
 * T_w*k/E_l rows per local expert -- and the product is rounded up, in exact
 * integer arithmetic.  Reads T, n_waves, top_k, n_ranks, n_experts from d. */
int moe_capacity(const moe_dims *d, int64_t cf_send_num, int64_t cf_send_den,
                 int64_t cf_recv_num, int64_t cf_recv_den, int32_t *cap_send,
                 int32_t *cap_recv);

enum { MOE_CALL_ROUTE = 0, MOE_CALL_PACK = 1, MOE_CALL_BANK = 2,
       MOE_CALL_FFN = 3, MOE_CALL_COMBINE = 4, MOE_CALL_COMBINE_SHARED = 5,
       MOE_CALL_COMBINE_BWD = 6, MOE_CALL_FFN_BWD = 7, MOE_CALL_PACK_BWD = 8 };

/* Bytes of scratch a call needs.  n_rows: bank rows allocated (FFN, ragged
 * mode); ignored otherwise.  Returns a negative moe_status on bad dims. */
int64_t moe_workspace_bytes(const moe_dims *d, int call, int64_t n_rows);

/* Router ([P2]/[P3] section 二, [P1] section 四: k of E routed experts per
 * token).  logits [T, E] fp32 (any routing bias already added).  Choice by
 * decreasing logit, equal logits to the lower index; topk [T, k] int32 in
 * that order; gates [T, k] fp32 = the chosen experts' probabilities under the
 * softmax over all E logits (not renormalised).  NaN logits unsupported. */
int moe_route(const float *logits, int32_t T, int32_t E, int32_t k,
              int32_t *topk, float *gates, void *stream);

/* Quantile balancing ([P1] section 四 and appendix A.2): a per-expert bias,
 * computed from how often each expert was chosen over the past batches, is
 * added to the router logits; it changes only the next routing decisions.
 *   moe_route_biased   moe_route on fp32(logits[t, e] + bias[e]) (selection
 *                      and softmax both); bias [E] fp32, NULL = no bias.
 *                      flags: MOE_ROUTE_RENORM divides each token's k gates
 *                      by their sum (= softmax over the k chosen logits; the
 *                      pages leave renormalisation open), 0 = moe_route's
 *                      gates; other bits are rejected
 *   moe_expert_counts  counts[e] = number of choices (t, j) with
 *                      topk[t, j] == e (entries outside [0, E) not counted);
 *                      topk [T, k] int32, counts [E] int32 out, fully written
 *   moe_balance_bias   H_i = sum over the n_batches rows of window [n_batches,
 *                      E] int32 (one row of counts per past batch; the caller
 *                      keeps the rows), f_i = H_i / sum(H) (1/E if sum(H) is
 *                      0), bias_i = -alpha * (f_i - 1/E) computed in double
 *                      and rounded to fp32; bias [E] out.  The bias is set
 *                      from the window, not accumulated.
 * Supported: E <= 1024, k <= 32.  Errors as for moe_route. */
enum { MOE_ROUTE_RENORM = 1 };
int moe_route_biased(const float *logits, const float *bias, int32_t T, int32_t E,
                     int32_t k, int32_t flags, int32_t *topk, float *gates, void *stream);
int moe_expert_counts(const int32_t *topk, int32_t T, int32_t k, int32_t E,
                      int32_t *counts, void *stream);
int moe_balance_bias(const int32_t *window, int32_t n_batches, int32_t E,
                     double alpha, float *bias, void *stream);

/* Sender ([P2]/[P3] section 二; [P1] appendix A.3): latent projection
 * z = x . W_ld, then every assignment (t, j) in (token, choice) order takes
 * the next position of pool (dest(e), wave(t)); kept iff the position is
 * below cap_send (always in ragged mode).  MOE_WAVES_CHUNKS: the next
 * position of dest(e)'s pool of n_waves*cap_send rows, kept iff below that;
 * row dest*n_waves*cap_send + slot; fill[p] / demand[p] are then chunk w's
 * rows, clamp(n - w*cap_send, 0, cap_send), with the rows past the last
 * chunk added to the last chunk's demand.
 *   x           [T, d_model] bf16
 *   w_lat_down  [latent, d_model] bf16 (W_ld^T)
 *   topk        [T, k] int32 from moe_route
 *   z           [T, latent] bf16 out
 *   pools       fixed: [n_ranks*n_waves*cap_send] rows out (kept rows carry
 *               z[t] and id e; the rest only the id -1);
 *               ragged: [T*k] rows out, pool p at pool_offsets[p]
 *   pool_offsets ragged: [n_ranks*n_waves + 1] int64 out; NULL if fixed
 *   slot        [T, k] int32 out: position in its pool, or -1 if dropped
 *   fill        [n_ranks*n_waves] int32 out: kept rows per pool
 *   demand      [n_ranks*n_waves] int32 out: rows asked of each pool
 *   Pool index p = dest * n_waves + wave.  Sender drops = sum(demand-fill). */
int moe_pack_waves(const moe_dims *d, const moe_bf16 *x,
                   const moe_bf16 *w_lat_down, const int32_t *topk,
                   moe_bf16 *z, uint8_t *pools, int64_t *pool_offsets,
                   int32_t *slot, int32_t *fill, int32_t *demand, void *ws,
                   int64_t ws_bytes, void *stream);

/* moe_pack_waves without a workspace, for callers that cannot allocate
 * device memory (code under stream capture, serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs and kernels as moe_pack_waves,
 * bit for bit; the slot assignment's per-tile counts go to a fixed device
 * array of MOE_NOALLOC_SCRATCH_BYTES inside the library instead of ws.  The
 * call allocates nothing.  Each GPU holds one such array (taken on the first
 * call made with that device current, kept until the process ends), shared
 * by every call on that GPU: calls that overlap on one GPU (two streams, or
 * two threads) race on it and must be ordered by the caller.  The stream
 * must belong to the current device.  Limit: moe_workspace_bytes(d,
 * MOE_CALL_PACK, 0) <= MOE_NOALLOC_SCRATCH_BYTES, where that size is
 * ceil(T*top_k/2048) * (n_ranks*n_waves + 1) * 4 bytes rounded up to 256;
 * with 64 ranks and 3 waves that is T*top_k <= 2,781,184.  Larger shapes
 * return MOE_ERR_UNSUPPORTED before any launch. */
#define MOE_NOALLOC_SCRATCH_BYTES (1 << 20)
int moe_pack_waves_noalloc(const moe_dims *d, const moe_bf16 *x,
                           const moe_bf16 *w_lat_down, const int32_t *topk,
                           moe_bf16 *z, uint8_t *pools, int64_t *pool_offsets,
                           int32_t *slot, int32_t *fill, int32_t *demand,
                           void *stream);

/* Receiver ([P2]/[P3] section 二; [P1] section 四 and appendix A.3): rows
 * received by `rank` are banked per (wave, local expert) in (source, row)
 * order within each wave; kept iff the position is below cap_recv.
 *   recv         fixed: [n_ranks*n_waves*cap_send] rows;
 *                ragged: n_recv_rows rows, segment (s, w) at
 *                recv_offsets[s*n_waves + w]
 *   recv_offsets ragged: [n_ranks*n_waves + 1] int64; NULL if fixed
 *   n_recv_rows  rows in recv (must equal n_ranks*n_waves*cap_send if fixed)
 *   bank         fixed: [n_waves*E_l*cap_recv, latent] bf16 out;
 *                ragged: [n_recv_rows, latent], group g at bank_offsets[g];
 *                rows past each group's fill are unspecified
 *   bank_offsets ragged: [n_waves*E_l + 1] int64 out; NULL if fixed
 *   bank_src     [bank rows] int32 out: receive row of each bank row, -1
 *                where unused
 *   bfill        [n_waves*E_l] int32 out: kept rows per group
 *   bdemand      [n_waves*E_l] int32 out: rows that asked for each group
 *   bad_rows     [1] int32 out: rows whose id is not -1 and not on `rank`
 *   Group g = wave * E_l + local expert.  Receiver drops = sum(bdemand-bfill). */
int moe_bank(const moe_dims *d, int32_t rank, const uint8_t *recv,
             const int64_t *recv_offsets, int64_t n_recv_rows, moe_bf16 *bank,
             int64_t *bank_offsets, int32_t *bank_src, int32_t *bfill,
             int32_t *bdemand, int32_t *bad_rows, void *ws, int64_t ws_bytes,
             void *stream);

/* Expert FFN ([P1] section 四 and appendix A.3: each wave the receiver runs
 * all of its local experts).  For every kept bank row u of group (w, j):
 * y = bf16( bf16(silu(u.W_g,j) * (u.W_u,j)) . W_d,j ), silu(a) = a/(1+e^-a)
 * (SwiGLU: the pages leave the expert's form open), written to ret at row
 * bank_src; every other ret row is zero.
 *   bank, bank_offsets, bank_src, bfill  from moe_bank
 *   n_bank_rows  rows allocated in bank (bounds the launch)
 *   w_gate, w_up [E_l, d_ff, latent] bf16; w_down [E_l, latent, d_ff] bf16
 *   ret          [n_ret_rows, latent] bf16 out, recv layout
 *   ws           scratch of moe_workspace_bytes(d, MOE_CALL_FFN, n_bank_rows) */
int moe_expert_ffn(const moe_dims *d, const moe_bf16 *bank,
                   const int64_t *bank_offsets, const int32_t *bank_src,
                   const int32_t *bfill, int64_t n_bank_rows,
                   const moe_bf16 *w_gate, const moe_bf16 *w_up,
                   const moe_bf16 *w_down, moe_bf16 *ret, int64_t n_ret_rows,
                   void *ws, int64_t ws_bytes, void *stream);

/* Combine ([P2]/[P3] section 二: routed outputs go back to model width and
 * join the shared-expert path; section 四: a dropped assignment only loses its
 * routed contribution, the two shared experts see every token).
 *   ylat[t] = bf16( sum_j [slot>=0] gates[t,j] * returned[dest(e), wave(t), slot] )
 *   out[t]  = bf16( ylat[t].W_lu + sum_s bf16(silu(x.W_sg,s)*(x.W_su,s)).W_sd,s )
 *   returned     rows of the pools' layout (destination, wave, slot), latent
 *                wide, no tail; ragged: segment p at ret_offsets[p], a slot
 *                at or past its segment's length reads as zero
 *   ret_offsets  ragged: [n_ranks*n_waves + 1] int64; NULL if fixed
 *   topk, slot, gates  from moe_route / moe_pack_waves
 *   x            [T, d_model] bf16
 *   w_lat_up     [d_model, latent] bf16 (W_lu^T)
 *   ws_gate, ws_up [n_shared, d_ff_shared, d_model]; ws_down
 *                [n_shared, d_model, d_ff_shared] bf16
 *   ylat         [T, latent] bf16 out; out [T, d_model] bf16 out
 *   ws           scratch of moe_workspace_bytes(d, MOE_CALL_COMBINE, 0) */
int moe_combine(const moe_dims *d, const moe_bf16 *returned,
                const int64_t *ret_offsets, const int32_t *topk,
                const int32_t *slot, const float *gates, const moe_bf16 *x,
                const moe_bf16 *w_lat_up, const moe_bf16 *ws_gate,
                const moe_bf16 *ws_up, const moe_bf16 *ws_down, moe_bf16 *ylat,
                moe_bf16 *out, void *ws, int64_t ws_bytes, void *stream);

/* The same combine as two calls.  The shared experts read only x, so a
 * caller can run them on another stream while the routed experts run.
 *   moe_shared_swiglu   h_shared[t, s*d_ff_shared + f] =
 *                       bf16(silu(x.W_sg,s) * (x.W_su,s))[t, f]
 *     x, ws_gate, ws_up  as in moe_combine
 *     h_shared     [T, n_shared*d_ff_shared] bf16 out (n_shared == 0: no-op)
 *   moe_combine_shared  ylat and out exactly as moe_combine, with the shared
 *                       experts' intermediate read from h_shared.
 *     ws           scratch of moe_workspace_bytes(d, MOE_CALL_COMBINE_SHARED, 0)
 *                  for the partial tiles of the up-projection's last round
 *                  (cut along K when it would fill at most half the CUs);
 *                  NULL with ws_bytes 0 runs that round whole (results
 *                  then differ in fp32 summation order only)
 *     Other arguments as in moe_combine.
 * moe_combine equals moe_shared_swiglu into its workspace followed by
 * moe_combine_shared with a workspace, bit for bit.  Errors as for
 * moe_combine. */
int moe_shared_swiglu(const moe_dims *d, const moe_bf16 *x, const moe_bf16 *ws_gate,
                      const moe_bf16 *ws_up, moe_bf16 *h_shared, void *stream);
int moe_combine_shared(const moe_dims *d, const moe_bf16 *returned,
                       const int64_t *ret_offsets, const int32_t *topk,
                       const int32_t *slot, const float *gates,
                       const moe_bf16 *w_lat_up, const moe_bf16 *h_shared,
                       const moe_bf16 *ws_down, moe_bf16 *ylat, moe_bf16 *out,
                       void *ws, int64_t ws_bytes, void *stream);

/* Kernel timing.  While enabled, every kernel the library launches is
 * bracketed by two hipEvents on its stream.  moe_profile_collect()
 * waits for the recorded events and folds them into per-kernel totals;
 * moe_profile_get(i, ...) reads entry i (returns MOE_ERR_INVALID past the
 * end); moe_profile_reset() clears the totals.  Not for concurrent use from
 * several threads. */
int moe_profile_enable(int on);
int moe_profile_collect(void);
int moe_profile_get(int i, char *name, int name_len, double *total_ms,
                    int64_t *launches);
void moe_profile_reset(void);

/* ------------------------------------------------------------------------
 * Backward of the branch (training; fixed capacities or ragged / dropless,
 * not dedup).  [P2]/[P3] describe a model in open training and give its
 * forward pass; each call below is the chain rule through the forward call
 * of the same stage, for a loss whose gradient with respect to `out` is
 * d_out.  Gradients are stored like their values: bf16 activations and
 * weight gradients (written, not accumulated), fp32 gate and logit
 * gradients.  The intermediates a = u.W_g and b = u.W_u are recomputed.
 * Order on one rank: moe_combine_backward -> (return exchange reversed) ->
 * moe_expert_ffn_backward -> (forward exchange reversed) ->
 * moe_pack_backward, and moe_route_backward with the gate gradients.
 * The router's own product (logits = x . W_r) is outside the boundary: its
 * input gradient is the caller's.  Workspaces: moe_workspace_bytes(d,
 * MOE_CALL_*_BWD, n_rows), n_rows = the bank rows of the expert call in
 * ragged mode (0 otherwise).  Ragged mode: every buffer in the pools' layout
 * (returned, d_returned, d_pools) has segments (destination, wave) at the
 * offsets passed with it, and a choice whose slot lies at or past its
 * segment's length has no row there (as in moe_combine, where such a
 * returned row reads as zero): its gate gradient is 0, it adds nothing to
 * dz, and nothing is written for it.
 * ------------------------------------------------------------------------ */

/* Router: d_logits [T, E] fp32 from d_gates [T, k].  With p the softmax of
 * l = fp32(logit + bias) over all E and gate j = p[e_j]:
 * d_l[e] = sum_j d_gates[j] p[e_j] ([e == e_j] - p[e]).  flags
 * MOE_ROUTE_RENORM (gates = softmax over the k chosen, q):
 * d_l[e_j] = q_j (d_gates[j] - sum_i d_gates[i] q_i), 0 elsewhere.  The
 * bias (NULL = none) is stop-gradient.  topk as returned by the router. */
int moe_route_backward(const float *logits, const float *bias, int32_t T,
                       int32_t E, int32_t k, int32_t flags, const int32_t *topk,
                       const float *d_gates, float *d_logits, void *stream);

/* Combine side, on the sender.  Inputs as given to / produced by
 * moe_combine (returned rows in the pools' layout, the sender's topk, slot,
 * gates, fill, x, the forward's ylat) plus d_out [T, d_model] bf16.
 *   ret_offsets ragged: [n_ranks*n_waves + 1] int64, the segments of
 *              returned and d_returned; NULL if fixed
 *   n_ret_rows rows of returned and d_returned (fixed mode: must equal
 *              n_ranks*n_waves*cap_send)
 *   d_returned [n_ret_rows, latent] out: bf16(g d_ylat[t]) in each kept
 *              choice's row, 0 in every other row; d_ylat =
 *              d_out . W_lu^T (rounded to bf16, not returned)
 *   d_gates    [T, k] fp32 out: returned row . d_ylat[t], 0 if dropped
 *   d_shared   [T, 2, n_shared, d_ff_shared] bf16 out: d_a, then d_b, of
 *              every shared expert (input of moe_pack_backward)
 *   dw_lat_up  [d_model, latent] bf16 out (W_lu's layout)
 *   dws_down   [n_shared, d_model, d_ff_shared] bf16 out
 * ws_gate / ws_up / ws_down / d_shared / dws_down may be NULL if n_shared = 0. */
int moe_combine_backward(const moe_dims *d, const moe_bf16 *returned,
                         const int64_t *ret_offsets, int64_t n_ret_rows,
                         const int32_t *topk, const int32_t *slot,
                         const float *gates, const int32_t *fill,
                         const moe_bf16 *x, const moe_bf16 *ylat,
                         const moe_bf16 *w_lat_up, const moe_bf16 *ws_gate,
                         const moe_bf16 *ws_up, const moe_bf16 *ws_down,
                         const moe_bf16 *d_out, moe_bf16 *d_returned,
                         float *d_gates, moe_bf16 *d_shared,
                         moe_bf16 *dw_lat_up, moe_bf16 *dws_down, void *ws,
                         int64_t ws_bytes, void *stream);

/* Receiver side.  bank, bank_offsets, bank_src, bfill as produced by
 * moe_bank; weights as given to moe_expert_ffn; d_ret [n_ret_rows, latent]:
 * the gradients of this rank's return rows (receive layout).
 *   n_bank_rows  rows of bank (fixed: n_waves*E_l*cap_recv; ragged: the
 *                receive rows, n_ret_rows)
 *   n_ret_rows   rows of d_ret and d_recv (fixed: n_ranks*n_waves*cap_send)
 *   d_recv   [n_ret_rows, latent] out: gradient of each kept receive row's
 *            payload (d_a . W_g + d_b . W_u), 0 elsewhere
 *   dw_gate, dw_up [E_l, d_ff, latent], dw_down [E_l, latent, d_ff] out,
 *            each local expert's sum over its kept rows of every wave.
 * Ragged mode needs E_l <= 6. */
int moe_expert_ffn_backward(const moe_dims *d, const moe_bf16 *bank,
                            const int64_t *bank_offsets, int64_t n_bank_rows,
                            const int32_t *bank_src, const int32_t *bfill,
                            const moe_bf16 *w_gate, const moe_bf16 *w_up,
                            const moe_bf16 *w_down, const moe_bf16 *d_ret,
                            int64_t n_ret_rows, moe_bf16 *d_recv, moe_bf16 *dw_gate,
                            moe_bf16 *dw_up, moe_bf16 *dw_down, void *ws,
                            int64_t ws_bytes, void *stream);

/* Sender side.  d_pools [pool rows, latent]: gradients of this shard's pool
 * payloads (the pools' layout; ragged: segments at pool_offsets, [n_ranks*
 * n_waves + 1] int64, NULL if fixed); topk, slot, x as in the forward pass;
 * d_shared from moe_combine_backward.
 *   dz          [T, latent] bf16 out: sum over kept choices of their rows
 *   dx          [T, d_model] bf16 out: dz . W_ld^T + the shared experts'
 *               input gradient, one sum, one rounding
 *   dw_lat_down [latent, d_model], dws_gate, dws_up [n_shared, d_ff_shared,
 *               d_model] bf16 out.
 * d_shared, ws_gate, ws_up, dws_gate, dws_up may be NULL if n_shared = 0. */
int moe_pack_backward(const moe_dims *d, const moe_bf16 *d_pools,
                      const int64_t *pool_offsets, const int32_t *topk,
                      const int32_t *slot,
                      const moe_bf16 *x, const moe_bf16 *d_shared,
                      const moe_bf16 *w_lat_down, const moe_bf16 *ws_gate,
                      const moe_bf16 *ws_up, moe_bf16 *dz, moe_bf16 *dx,
                      moe_bf16 *dw_lat_down, moe_bf16 *dws_gate,
                      moe_bf16 *dws_up, void *ws, int64_t ws_bytes,
                      void *stream);

#ifdef __cplusplus
}
#endif
#endif
