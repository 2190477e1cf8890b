/*
 * oracle.c -- plain, slow, single-threaded CPU reference of the pooled-wave
 * MoE dispatch share.  TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Every floating-point sum runs in double, in the written loop order, and is
 * rounded once to the stored type (bf16 with round-to-nearest-even, or fp32).
 * There is no blocking, fusion or reordering beyond the definitions below.
 *
 * Sources, cited by page title and section:
 *   [P2] "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK)
 *   [P3] "Marin、535BパラメータMoEモデルのオープントレーニングを開始"
 *        (lamjinlab.com, ja), translation of [P2]
 *   [P1] "从玩具到前沿:训练一个真正的大模型,到底难在哪里" (devpress.csdn.net)
 *
 * Readings of points the pages leave open are marked READING below.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 conversion                                                          */
/* ------------------------------------------------------------------------ */

double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Nearest bf16 to v (ties to even), computed from the double directly so
 * there is exactly one rounding.  bf16 has 8 significant bits and the fp32
 * exponent range; below 2^-126 the spacing stays 2^-133 (subnormals). */
uint16_t orc_bf16_from_double(double v) {
  if (v != v) return 0x7fc0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int q = (e - 1 >= -126) ? (e - 1) - 7 : -133;
  double r = nearbyint(ldexp(a, -q)); /* default rounding mode: ties to even */
  double res = ldexp(r, q);
  if (res > 3.3895313892515355e38) return sign | 0x7f80; /* beyond max bf16 */
  float f = (float)res;                                     /* exact */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7fff);
}

static double bf(uint16_t b) { return orc_bf16_to_double(b); }
static uint16_t to_bf(double v) { return orc_bf16_from_double(v); }

/* ------------------------------------------------------------------------ */
/* Sizes                                                                    */
/* ------------------------------------------------------------------------ */

/* READING: the three waves of [P2] section 二 split each shard's tokens into
 * contiguous thirds: wave(t) = floor(t / T_w) with T_w = ceil(T / W). */
int32_t orc_tokens_per_wave(int32_t T, int32_t n_waves) {
  return (T + n_waves - 1) / n_waves;
}

/* Capacity of one fixed buffer ([P2]/[P3] section 二: a sender factor caps the
 * rows one source sends to one destination, a receiver factor caps the rows
 * one local expert takes).  READING: the factor multiplies the mean load of
 * the buffer for one wave -- T_w*k/R rows per (source, destination) pool and
 * T_w*k/E_l rows per local expert (R sources times T_w*k/R rows spread over
 * E_l experts) -- and the product is rounded up.  Exact integers throughout. */
int64_t orc_capacity(int64_t tokens_per_wave, int32_t top_k, int32_t groups,
                     int64_t cf_num, int64_t cf_den) {
  int64_t a = cf_num * tokens_per_wave * (int64_t)top_k;
  int64_t b = cf_den * (int64_t)groups;
  return (a + b - 1) / b;
}

/* ------------------------------------------------------------------------ */
/* Router: softmax over all experts, then the top k                         */
/* ------------------------------------------------------------------------ */

/* [P2]/[P3] section 二 and [P1] section 四: the router picks 8 of the 384
 * routed experts per token.  READING: the gate of a chosen expert is its
 * probability under the softmax over all E logits (no renormalisation over
 * the k chosen).  Selection runs on the fp32 logits themselves (softmax is
 * monotone, so this is the same choice) in order of decreasing logit; equal
 * logits go to the lower expert index.  topk[t, j] is the j-th choice. */
void orc_route(const float *logits, int64_t T, int32_t E, int32_t k,
               int32_t *topk, float *gates) {
  char *taken = (char *)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    const float *l = logits + t * E;
    double m = l[0];
    for (int32_t e = 1; e < E; ++e)
      if (l[e] > m) m = l[e];
    double Z = 0.0;
    for (int32_t e = 0; e < E; ++e) Z += exp((double)l[e] - m);
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: lower index wins ties */
      }
      taken[best] = 1;
      topk[t * k + j] = best;
      gates[t * k + j] = (float)(exp((double)l[best] - m) / Z);
    }
  }
  free(taken);
}

/* ------------------------------------------------------------------------ */
/* Quantile balancing                                                       */
/* ------------------------------------------------------------------------ */

/* [P1] section 四 and appendix A.2: a routing bias is added to the router
 * logits (stop-gradient: it changes only which experts are chosen next).
 * The biased logit is rounded to fp32 -- the precision the routing decision
 * is taken in -- and the router above then runs on it unchanged. */
void orc_route_biased(const float *logits, const float *bias, int64_t T,
                      int32_t E, int32_t k, int32_t *topk, float *gates) {
  float *lb = (float *)malloc(sizeof(float) * (size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) lb[e] = logits[t * E + e] + bias[e];
    orc_route(lb, 1, E, k, topk + t * k, gates + t * k);
  }
  free(lb);
}

/* Variant of the gates (the pages leave it open whether the chosen experts'
 * weights are renormalised): with renorm, gate j of token t is the chosen
 * expert's probability divided by the sum over the k chosen, which is the
 * softmax over the k chosen logits.  In double, rounded once to fp32. */
void orc_route_ex(const float *logits, const float *bias, int64_t T,
                  int32_t E, int32_t k, int32_t renorm, int32_t *topk,
                  float *gates) {
  float *lb = (float *)malloc(sizeof(float) * (size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e)
      lb[e] = bias ? logits[t * E + e] + bias[e] : logits[t * E + e];
    orc_route(lb, 1, E, k, topk + t * k, gates + t * k);
    if (renorm) {
      double m = lb[topk[t * k]], z = 0.0; /* the first choice holds the largest logit */
      for (int32_t j = 0; j < k; ++j) z += exp((double)lb[topk[t * k + j]] - m);
      for (int32_t j = 0; j < k; ++j)
        gates[t * k + j] = (float)(exp((double)lb[topk[t * k + j]] - m) / z);
    }
  }
  free(lb);
}

/* [P1] appendix A.2: H counts how often each expert was chosen.  One batch's
 * counts: counts[e] = number of choices (t, j) with topk[t, j] == e; entries
 * outside [0, E) are not choices of an expert and are not counted. */
void orc_expert_counts(const int32_t *topk, int64_t n, int32_t E,
                       int32_t *counts) {
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < n; ++i)
    if (topk[i] >= 0 && topk[i] < E) counts[topk[i]] += 1;
}

/* [P1] appendix A.2: with H[i] the selections of expert i over the past N
 * batches, f_i = H[i] / sum(H) and the bias is b_i = -alpha * (f_i - 1/E).
 * window[b * E + i] holds batch b's counts.  READING: the formula sets the
 * bias (it does not add to the previous one); with no selections at all
 * (sum(H) == 0) the frequencies are taken as uniform, so every bias is 0.
 * Computed in double, rounded once to fp32. */
void orc_balance_bias(const int32_t *window, int32_t n_batches, int32_t E,
                      double alpha, float *bias) {
  int64_t total = 0;
  for (int32_t b = 0; b < n_batches; ++b)
    for (int32_t i = 0; i < E; ++i) total += window[(int64_t)b * E + i];
  for (int32_t i = 0; i < E; ++i) {
    int64_t h = 0;
    for (int32_t b = 0; b < n_batches; ++b) h += window[(int64_t)b * E + i];
    double f = total > 0 ? (double)h / (double)total : 1.0 / (double)E;
    bias[i] = (float)(-alpha * (f - 1.0 / (double)E));
  }
}

/* ------------------------------------------------------------------------ */
/* Latent down-projection                                                   */
/* ------------------------------------------------------------------------ */

/* [P2]/[P3] section 二: the routed activations are projected from the model
 * width to the latent width before they cross GPUs.  z[t] = x[t] . W_ld,
 * one rounding to bf16.  rows == NULL means rows 0 .. n-1. */
void orc_latent_rows(const uint16_t *x, int32_t D, const uint16_t *w_ld_t,
                     int32_t L, const int64_t *rows, int64_t n, uint16_t *z) {
  double *xr = (double *)malloc(sizeof(double) * (size_t)D);
  for (int64_t r = 0; r < n; ++r) {
    int64_t t = rows ? rows[r] : r;
    for (int32_t i = 0; i < D; ++i) xr[i] = bf(x[t * D + i]);
    for (int32_t c = 0; c < L; ++c) {
      const uint16_t *w = w_ld_t + (int64_t)c * D;
      double acc = 0.0;
      for (int32_t i = 0; i < D; ++i) acc += xr[i] * bf(w[i]);
      z[r * L + c] = to_bf(acc);
    }
  }
  free(xr);
}

/* ------------------------------------------------------------------------ */
/* Sender: fixed pool per destination and wave                              */
/* ------------------------------------------------------------------------ */

static int32_t dest_of(const orc_dims *d, int32_t e) {
  /* READING: experts are placed contiguously, E_l = E / R per rank. */
  return e / (d->n_experts / d->n_ranks);
}

/* Variant (dedup): a token's choices on one destination travel as groups
 * of up to four in one row.  Group position of choice j = the number of the
 * token's earlier choices on the same destination; positions 0, 4 lead a
 * row, the others belong to the row of the choice 4 * floor(c / 4). */
static int32_t dedup_rank(const orc_dims *d, const int32_t *tk, int32_t j) {
  int32_t c = 0, dj = dest_of(d, tk[j]);
  for (int32_t i = 0; i < j; ++i) c += dest_of(d, tk[i]) == dj;
  return c;
}

/* True for a choice that joins an earlier choice's row; its slot is then
 * set to that row's (already assigned) slot. */
static int dedup_follower(const orc_dims *d, const int32_t *tk, int32_t j,
                          int32_t *slot_row) {
  int32_t c = dedup_rank(d, tk, j);
  if (c % 4 == 0) return 0;
  int32_t dj = dest_of(d, tk[j]), lead = c - c % 4;
  for (int32_t i = 0; i < j; ++i)
    if (dest_of(d, tk[i]) == dj && dedup_rank(d, tk, i) == lead) {
      slot_row[j] = slot_row[i];
      return 1;
    }
  return 0; /* not reached */
}

/* READING (other wave reading, wave_mode 1): one pool of W*cap_send rows
 * per destination, filled in (token, choice) order; position i lies in chunk
 * (wave) i / cap_send.  fill and demand are reported per chunk: chunk w holds
 * min(max(n - w*cap, 0), cap) rows, and the rows past the last chunk count as
 * that chunk's unmet demand. */
static int64_t orc_sender_chunks(const orc_dims *d, const int32_t *topk,
                                 int32_t *slot, int32_t *fill,
                                 int32_t *demand) {
  const int32_t W = d->n_waves, R = d->n_ranks, k = d->top_k;
  const int64_t cap = d->cap_send, pool = (int64_t)W * cap;
  int64_t drops = 0;
  int64_t *n = (int64_t *)calloc((size_t)R, sizeof(int64_t));
  for (int32_t t = 0; t < d->T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      if (d->dedup && dedup_follower(d, topk + (int64_t)t * k, j, slot + (int64_t)t * k)) {
        drops += slot[(int64_t)t * k + j] < 0;
        continue;
      }
      int32_t e = topk[(int64_t)t * k + j];
      int64_t pos = n[dest_of(d, e)]++;
      if (pos < pool) {
        slot[(int64_t)t * k + j] = (int32_t)pos;
      } else {
        slot[(int64_t)t * k + j] = -1;
        ++drops;
      }
    }
  }
  for (int32_t r = 0; r < R; ++r)
    for (int32_t w = 0; w < W; ++w) {
      int64_t left = n[r] - w * cap;
      if (left < 0) left = 0;
      fill[r * W + w] = (int32_t)(left < cap ? left : cap);
      demand[r * W + w] = (int32_t)(w + 1 < W ? fill[r * W + w] : left);
    }
  free(n);
  return drops;
}

/* [P2]/[P3] section 二: one fixed pool per destination GPU (not per expert),
 * three waves of equal shape, overflow beyond the sender capacity dropped and
 * counted apart.  [P1] appendix A.3 describes the same fixed per-destination
 * pools sent in three waves.
 * Walk the assignments in (token, choice) order; an assignment takes the next
 * free position of pool (dest(e), wave(t)); it is kept when that position is
 * below the capacity (always, in ragged mode).  slot[t,j] = position or -1.
 * fill = kept rows per pool, demand = all rows asked of the pool; pool index
 * is dest * W + wave.  Ragged mode also writes pool_offsets (exclusive prefix
 * of demand, plus the total).  Returns the number of dropped assignments. */
int64_t orc_sender(const orc_dims *d, const int32_t *topk, int32_t *slot,
                   int32_t *fill, int32_t *demand, int64_t *pool_offsets) {
  const int32_t W = d->n_waves, R = d->n_ranks, k = d->top_k;
  const int32_t Tw = orc_tokens_per_wave(d->T, W);
  const int32_t cap = d->cap_send;
  if (d->wave_mode == 1) return orc_sender_chunks(d, topk, slot, fill, demand);
  int64_t drops = 0;
  int32_t *n = (int32_t *)calloc((size_t)R * W, sizeof(int32_t));
  for (int32_t t = 0; t < d->T; ++t) {
    int32_t w = t / Tw;
    for (int32_t j = 0; j < k; ++j) {
      if (d->dedup && dedup_follower(d, topk + (int64_t)t * k, j, slot + (int64_t)t * k)) {
        drops += slot[(int64_t)t * k + j] < 0;
        continue;
      }
      int32_t e = topk[(int64_t)t * k + j];
      int32_t p = dest_of(d, e) * W + w;
      int32_t pos = n[p]++;
      if (cap == 0 || pos < cap) {
        slot[(int64_t)t * k + j] = pos;
      } else {
        slot[(int64_t)t * k + j] = -1;
        ++drops;
      }
    }
  }
  for (int32_t p = 0; p < R * W; ++p) {
    demand[p] = n[p];
    fill[p] = (cap == 0 || n[p] < cap) ? n[p] : cap;
  }
  if (cap == 0 && pool_offsets) {
    pool_offsets[0] = 0;
    for (int32_t p = 0; p < R * W; ++p) pool_offsets[p + 1] = pool_offsets[p] + n[p];
  }
  free(n);
  return drops;
}

/* Row record: latent bf16 values then {expert id, 0, 0, 0}.  [P2]/[P3]
 * section 二: the expert id travels inside the payload, so no counts or
 * routing metadata are exchanged.  READING: one row per kept assignment, so a
 * token with several experts on one rank is sent once per such expert. */
static void put_header(uint8_t *row, int32_t L, int32_t id) {
  int32_t h[4] = {id, 0, 0, 0};
  memcpy(row + (size_t)L * 2, h, 16);
}

static int32_t get_header(const uint8_t *row, int32_t L) {
  int32_t id;
  memcpy(&id, row + (size_t)L * 2, 4);
  return id;
}

void orc_row_ids(const uint8_t *row, int32_t L, int32_t *ids) {
  memcpy(ids, row + (size_t)L * 2, 16);
}

void orc_pack_rows(const orc_dims *d, const uint16_t *z, const int32_t *topk,
                   const int32_t *slot, const int64_t *pool_offsets,
                   uint8_t *pools, int64_t n_pool_rows) {
  const int32_t L = d->latent, W = d->n_waves, k = d->top_k;
  const size_t rb = (size_t)L * 2 + 16;
  const int32_t Tw = orc_tokens_per_wave(d->T, W);
  for (int64_t r = 0; r < n_pool_rows; ++r) {
    memset(pools + r * rb, 0, rb - 16);
    put_header(pools + r * rb, L, -1);
    if (d->dedup) memset(pools + r * rb + (size_t)L * 2, 0xff, 16); /* four empty ids */
  }
  for (int32_t t = 0; t < d->T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      int32_t s = slot[(int64_t)t * k + j];
      if (s < 0) continue;
      int32_t e = topk[(int64_t)t * k + j];
      int32_t p = dest_of(d, e) * W + t / Tw;
      int64_t row = d->cap_send ? (int64_t)p * d->cap_send + s : pool_offsets[p] + s;
      if (d->wave_mode == 1) row = (int64_t)dest_of(d, e) * W * d->cap_send + s;
      if (d->dedup) {
        const int32_t *tk = topk + (int64_t)t * k;
        int32_t c = dedup_rank(d, tk, j);
        if (c % 4) continue; /* written with its row's leader */
        int32_t ids[4] = {-1, -1, -1, -1}, m = 0;
        for (int32_t i = j; i < k && m < 4; ++i)
          if (dest_of(d, tk[i]) == dest_of(d, e) && dedup_rank(d, tk, i) >= c) ids[m++] = tk[i];
        memcpy(pools + row * rb, z + (int64_t)t * L, (size_t)L * 2);
        memcpy(pools + row * rb + (size_t)L * 2, ids, 16);
        continue;
      }
      memcpy(pools + row * rb, z + (int64_t)t * L, (size_t)L * 2);
      put_header(pools + row * rb, L, e);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Receiver: bank rows into the local experts                               */
/* ------------------------------------------------------------------------ */

/* [P2]/[P3] section 二: a receiver factor caps the rows of each local expert;
 * overflow is dropped and counted apart; the bank holds six local experts
 * and the three waves keep only part of it live at a time.  [P1] section 四
 * and appendix A.3: every wave runs all local experts.
 * READING: the receiver capacity applies per wave and local expert; rows are
 * taken in (source, row) order within each wave.  hdr[row] is the tail id
 * of each receive row: -1 = empty (skipped); an id that is not hosted by
 * `rank` is counted in bad_rows and skipped.  bank_src[pos] = receive row of
 * bank position pos (-1 where unused).  Returns dropped rows. */
int64_t orc_bank_slots(const orc_dims *d, int32_t rank, const int32_t *hdr,
                       const int64_t *recv_offsets, int64_t n_recv_rows,
                       int64_t *bank_offsets, int32_t *bank_src,
                       int32_t *bfill, int32_t *bdemand, int32_t *bad_rows) {
  const int32_t R = d->n_ranks, W = d->n_waves;
  const int32_t El = d->n_experts / d->n_ranks;
  const int32_t cap = d->cap_recv;
  const int ragged = d->cap_send == 0;
  const int32_t G = W * El;
  int32_t *c = (int32_t *)calloc((size_t)G, sizeof(int32_t));
  int32_t bad = 0;
  /* items: one per receive row, or with dedup one per tail id of each row
   * (row, id index), in that order */
  const int32_t per = d->dedup ? 4 : 1;
  /* pass 1: counts */
  for (int32_t w = 0; w < W; ++w) {
    for (int32_t s = 0; s < R; ++s) {
      int64_t a = ragged ? recv_offsets[s * W + w] : ((int64_t)s * W + w) * d->cap_send;
      int64_t b = ragged ? recv_offsets[s * W + w + 1] : a + d->cap_send;
      for (int64_t q = a * per; q < b * per; ++q) {
        int32_t h = hdr[q];
        if (h == -1) continue;
        if (h < 0 || h >= d->n_experts || h / El != rank) {
          ++bad;
          continue;
        }
        c[w * El + h % El]++;
      }
    }
  }
  int64_t drops = 0;
  for (int32_t g = 0; g < G; ++g) {
    bdemand[g] = c[g];
    bfill[g] = (ragged || c[g] < cap) ? c[g] : cap;
    drops += c[g] - bfill[g];
  }
  int64_t n_bank = ragged ? n_recv_rows : (int64_t)G * cap;
  if (ragged) {
    bank_offsets[0] = 0;
    for (int32_t g = 0; g < G; ++g) bank_offsets[g + 1] = bank_offsets[g] + c[g];
  }
  for (int64_t i = 0; i < n_bank; ++i) bank_src[i] = -1;
  /* pass 2: positions in (source, row) order within each wave */
  memset(c, 0, sizeof(int32_t) * (size_t)G);
  for (int32_t w = 0; w < W; ++w) {
    for (int32_t s = 0; s < R; ++s) {
      int64_t a = ragged ? recv_offsets[s * W + w] : ((int64_t)s * W + w) * d->cap_send;
      int64_t b = ragged ? recv_offsets[s * W + w + 1] : a + d->cap_send;
      for (int64_t q = a * per; q < b * per; ++q) {
        int32_t h = hdr[q];
        if (h < 0 || h >= d->n_experts || h / El != rank) continue;
        int32_t g = w * El + h % El;
        int32_t p = c[g]++;
        if (ragged) bank_src[bank_offsets[g] + p] = (int32_t)q;
        else if (p < cap) bank_src[(int64_t)g * cap + p] = (int32_t)q;
      }
    }
  }
  *bad_rows = bad;
  free(c);
  return drops;
}

/* Copy each kept receive row's payload into its bank position. */
void orc_bank_rows(const orc_dims *d, const uint8_t *recv,
                   const int64_t *bank_offsets, const int32_t *bank_src,
                   const int32_t *bfill, uint16_t *bank) {
  const int32_t L = d->latent;
  const int32_t G = d->n_waves * (d->n_experts / d->n_ranks);
  const size_t rb = (size_t)L * 2 + 16;
  for (int32_t g = 0; g < G; ++g) {
    int64_t start = d->cap_send ? (int64_t)g * d->cap_recv : bank_offsets[g];
    for (int32_t p = 0; p < bfill[g]; ++p) {
      int64_t pos = start + p;
      int64_t row = d->dedup ? bank_src[pos] / 4 : bank_src[pos];
      memcpy(bank + pos * L, recv + row * rb, (size_t)L * 2);
    }
  }
}

/* Helper for tests that only have receive headers. */
int32_t orc_row_header(const uint8_t *row, int32_t L) { return get_header(row, L); }

/* ------------------------------------------------------------------------ */
/* Expert FFN                                                               */
/* ------------------------------------------------------------------------ */

static double silu(double a) { return a / (1.0 + exp(-a)); }

/* READING: the pages do not fix the routed expert's form or size; a SwiGLU
 * is used: h = bf16(silu(u.W_g) * (u.W_u)), y = bf16(h.W_d), silu(a) =
 * a / (1 + e^-a).  wg_t, wu_t are [F][L] and wd_t is [L][F]. */
void orc_ffn_row(int32_t L, int32_t F, const uint16_t *u, const uint16_t *wg_t,
                 const uint16_t *wu_t, const uint16_t *wd_t, uint16_t *y) {
  double *ud = (double *)malloc(sizeof(double) * (size_t)L);
  double *h = (double *)malloc(sizeof(double) * (size_t)F);
  for (int32_t i = 0; i < L; ++i) ud[i] = bf(u[i]);
  for (int32_t f = 0; f < F; ++f) {
    double a = 0.0, b = 0.0;
    const uint16_t *g = wg_t + (int64_t)f * L, *v = wu_t + (int64_t)f * L;
    for (int32_t i = 0; i < L; ++i) a += ud[i] * bf(g[i]);
    for (int32_t i = 0; i < L; ++i) b += ud[i] * bf(v[i]);
    h[f] = bf(to_bf(silu(a) * b));
  }
  for (int32_t c = 0; c < L; ++c) {
    const uint16_t *w = wd_t + (int64_t)c * F;
    double acc = 0.0;
    for (int32_t f = 0; f < F; ++f) acc += h[f] * bf(w[f]);
    y[c] = to_bf(acc);
  }
  free(ud);
  free(h);
}

/* [P1] section 四 and appendix A.3: each wave the receiver runs all of its
 * local experts.  Every kept bank row of group (wave, j) goes through local
 * expert j; the result is written to the return buffer at the row's receive
 * position (bank_src); every other return row is zero. */
void orc_expert_ffn(const orc_dims *d, const uint16_t *bank,
                    const int64_t *bank_offsets, const int32_t *bank_src,
                    const int32_t *bfill, const uint16_t *w_gate,
                    const uint16_t *w_up, const uint16_t *w_down,
                    uint16_t *ret, int64_t n_ret_rows) {
  const int32_t L = d->latent, F = d->d_ff;
  const int32_t El = d->n_experts / d->n_ranks;
  const int32_t G = d->n_waves * El;
  memset(ret, 0, sizeof(uint16_t) * (size_t)n_ret_rows * (size_t)L);
  for (int32_t g = 0; g < G; ++g) {
    int32_t j = g % El;
    int64_t start = d->cap_send ? (int64_t)g * d->cap_recv : bank_offsets[g];
    for (int32_t p = 0; p < bfill[g]; ++p) {
      int64_t pos = start + p;
      orc_ffn_row(L, F, bank + pos * L, w_gate + (int64_t)j * F * L,
                  w_up + (int64_t)j * F * L, w_down + (int64_t)j * L * F,
                  ret + (int64_t)bank_src[pos] * L);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Combine, latent up-projection and shared experts                         */
/* ------------------------------------------------------------------------ */

/* [P2]/[P3] section 二: the routed outputs are projected back to the model
 * width and then joined with the shared-expert path; the two shared experts
 * see every token regardless of routing.  [P2]/[P3] section 四: a dropped
 * assignment only loses its routed contribution.
 *   ylat[t] = bf16( sum_j [slot >= 0] g[t,j] * returned[dest(e), wave(t), slot] )
 *   out[t]  = bf16( ylat[t].W_lu + sum_s h_s(x[t]).W_sd,s ),
 *   h_s(x)  = bf16( silu(x.W_sg,s) * (x.W_su,s) ),
 * with the final sum in one double accumulator (W_lu terms, then shared
 * expert 0, then 1), rounded once.  returned is indexed like the sender's
 * pools (destination, wave, row).  Ragged mode: ret_offsets holds the segment
 * offsets in (destination, wave) order; a slot at or past its segment's
 * length reads as zero.  tokens == NULL means tokens 0 .. n-1; ylat and out
 * receive n rows. */
void orc_combine_tokens(const orc_dims *d, const uint16_t *returned,
                        const int64_t *ret_offsets, const int32_t *topk,
                        const int32_t *slot, const float *gates,
                        const uint16_t *x, const uint16_t *w_lu_t,
                        const uint16_t *ws_gate, const uint16_t *ws_up,
                        const uint16_t *ws_down, const int64_t *tokens,
                        int64_t n, uint16_t *ylat, uint16_t *out) {
  const int32_t L = d->latent, D = d->d_model, k = d->top_k, W = d->n_waves;
  const int32_t S = d->n_shared, Fs = d->d_ff_shared;
  const int32_t Tw = orc_tokens_per_wave(d->T, W);
  double *acc = (double *)malloc(sizeof(double) * (size_t)L);
  double *yl = (double *)malloc(sizeof(double) * (size_t)L);
  double *xr = (double *)malloc(sizeof(double) * (size_t)D);
  double *h = (double *)malloc(sizeof(double) * (size_t)S * Fs);
  for (int64_t r = 0; r < n; ++r) {
    int64_t t = tokens ? tokens[r] : r;
    int32_t w = (int32_t)(t / Tw);
    for (int32_t c = 0; c < L; ++c) acc[c] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t s = slot[t * k + j];
      if (s < 0) continue;
      int32_t e = topk[t * k + j];
      int32_t seg = dest_of(d, e) * W + w;
      int64_t row;
      if (d->wave_mode == 1) {
        row = (int64_t)dest_of(d, e) * W * d->cap_send + s; /* slot: position in the dest's pool */
      } else if (d->cap_send) {
        row = (int64_t)seg * d->cap_send + s;
      } else {
        if (s >= ret_offsets[seg + 1] - ret_offsets[seg]) continue;
        row = ret_offsets[seg] + s;
      }
      if (d->dedup) row = row * 4 + dedup_rank(d, topk + t * k, j) % 4; /* return slot */
      double g = gates[t * k + j];
      for (int32_t c = 0; c < L; ++c) acc[c] += g * bf(returned[row * L + c]);
    }
    for (int32_t c = 0; c < L; ++c) {
      ylat[r * L + c] = to_bf(acc[c]);
      yl[c] = bf(ylat[r * L + c]);
    }
    for (int32_t i = 0; i < D; ++i) xr[i] = bf(x[t * D + i]);
    for (int32_t sh = 0; sh < S; ++sh) {
      for (int32_t f = 0; f < Fs; ++f) {
        const uint16_t *g = ws_gate + ((int64_t)sh * Fs + f) * D;
        const uint16_t *v = ws_up + ((int64_t)sh * Fs + f) * D;
        double a = 0.0, b = 0.0;
        for (int32_t i = 0; i < D; ++i) a += xr[i] * bf(g[i]);
        for (int32_t i = 0; i < D; ++i) b += xr[i] * bf(v[i]);
        h[sh * Fs + f] = bf(to_bf(silu(a) * b));
      }
    }
    for (int32_t c = 0; c < D; ++c) {
      double o = 0.0;
      const uint16_t *wl = w_lu_t + (int64_t)c * L;
      for (int32_t i = 0; i < L; ++i) o += yl[i] * bf(wl[i]);
      for (int32_t sh = 0; sh < S; ++sh) {
        const uint16_t *wd = ws_down + ((int64_t)sh * D + c) * Fs;
        for (int32_t f = 0; f < Fs; ++f) o += h[sh * Fs + f] * bf(wd[f]);
      }
      out[r * D + c] = to_bf(o);
    }
  }
  free(acc);
  free(yl);
  free(xr);
  free(h);
}

/* ------------------------------------------------------------------------ */
/* Backward of the branch                                                   */
/* ------------------------------------------------------------------------ */

/* [P2]/[P3] (the model is being trained) give the forward pass only; the
 * gradients below follow from the forward definitions above by the chain
 * rule, for a loss whose gradient with respect to out is d_out.
 * READING (rounding points): every gradient tensor is stored like the value
 * it belongs to -- activation and weight gradients in bf16 (a parameter's
 * gradient has the parameter's type), gate and logit gradients in fp32 --
 * and each is one double sum rounded once.  The intermediates a = u.W_g and
 * b = u.W_u are recomputed from the forward inputs in double.  Fixed
 * capacities only. */

/* d silu / da = s (1 + a (1 - s)), s = 1 / (1 + e^-a) */
static double silu_grad(double a) {
  double s = 1.0 / (1.0 + exp(-a));
  return s * (1.0 + a * (1.0 - s));
}

/* Row of assignment (t, e, slot s) in a buffer of the pools' layout, or -1.
 * Fixed mode: (destination, wave, slot) with cap_send rows per pool.  Ragged
 * mode (waves by token): segment (destination, wave) starts at offsets[seg],
 * and a slot at or past the segment's length has no row (as in the forward
 * combine, where such a returned row reads as zero). */
static int64_t pool_row(const orc_dims *d, const int64_t *offsets, int64_t t, int32_t e,
                        int32_t s) {
  const int32_t W = d->n_waves;
  if (d->wave_mode == 1) return (int64_t)dest_of(d, e) * W * d->cap_send + s;
  const int64_t seg = (int64_t)dest_of(d, e) * W + t / orc_tokens_per_wave(d->T, W);
  if (d->cap_send) return seg * d->cap_send + s;
  if (s >= offsets[seg + 1] - offsets[seg]) return -1;
  return offsets[seg] + s;
}

/* First bank row of bank group g (fixed: g * cap_recv; ragged: offsets). */
static int64_t group_start(const orc_dims *d, const int64_t *bank_offsets, int32_t g) {
  return d->cap_send ? (int64_t)g * d->cap_recv : bank_offsets[g];
}

/* Router: with p = softmax(l) over all E (l = fp32(logit + bias)) and gate
 * g_j = p[e_j], dL/dl[e] = sum_j d_gates[j] * g_j * ([e == e_j] - p[e]).
 * Renormalised gates (q = softmax over the k chosen logits):
 * dL/dl[e_j] = q_j (d_gates[j] - sum_i d_gates[i] q_i), 0 for the others.
 * The bias is stop-gradient.  p and q are recomputed in double. */
void orc_route_backward(const float *logits, const float *bias, int64_t T,
                        int32_t E, int32_t k, int32_t renorm,
                        const int32_t *topk, const float *d_gates,
                        float *d_logits) {
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  double *dl = (double *)malloc(sizeof(double) * (size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      float lb = bias ? logits[t * E + e] + bias[e] : logits[t * E + e];
      p[e] = lb;
      dl[e] = 0.0;
    }
    const int32_t *tk = topk + t * k;
    const float *dg = d_gates + t * k;
    if (!renorm) {
      double m = p[0], Z = 0.0, s = 0.0;
      for (int32_t e = 1; e < E; ++e)
        if (p[e] > m) m = p[e];
      for (int32_t e = 0; e < E; ++e) Z += exp(p[e] - m);
      for (int32_t e = 0; e < E; ++e) p[e] = exp(p[e] - m) / Z;
      for (int32_t j = 0; j < k; ++j) s += (double)dg[j] * p[tk[j]];
      for (int32_t e = 0; e < E; ++e) dl[e] = -p[e] * s;
      for (int32_t j = 0; j < k; ++j) dl[tk[j]] += (double)dg[j] * p[tk[j]];
    } else {
      double m = p[tk[0]], z = 0.0, s = 0.0;
      for (int32_t j = 1; j < k; ++j)
        if (p[tk[j]] > m) m = p[tk[j]];
      for (int32_t j = 0; j < k; ++j) z += exp(p[tk[j]] - m);
      for (int32_t j = 0; j < k; ++j) s += (double)dg[j] * exp(p[tk[j]] - m) / z;
      for (int32_t j = 0; j < k; ++j) {
        double q = exp(p[tk[j]] - m) / z;
        dl[tk[j]] = q * ((double)dg[j] - s);
      }
    }
    for (int32_t e = 0; e < E; ++e) d_logits[t * E + e] = (float)dl[e];
  }
  free(p);
  free(dl);
}

/* Combine side.  From out = ylat.W_lu + sum_s h_s.W_sd,s and
 * ylat[t] = sum_j g[t,j] returned[row(t,j)]:
 *   d_ylat[t]          = bf16(d_out[t] . W_lu^T)        (used, not stored)
 *   d_h_s[t]           = bf16(d_out[t] . W_sd,s^T)
 *   d_returned[row]    = bf16(g[t,j] d_ylat[t]) for kept (t, j); other rows 0
 *   d_gates[t,j]       = fp32(returned[row] . d_ylat[t]); 0 if dropped
 *   d_shared[t][0][s]  = bf16(d_h_s * b * silu'(a)),  a = x.W_sg,s, b = x.W_su,s
 *   d_shared[t][1][s]  = bf16(d_h_s * silu(a))
 *   dw_lat_up[c][i]    = bf16(sum_t d_out[t][c] ylat[t][i])      ([D][L])
 *   dws_down[s][c][f]  = bf16(sum_t d_out[t][c] h_s[t][f])       ([S][D][Fs])
 * with h_s = bf16(silu(a) b) as in the forward pass. */
void orc_combine_backward(const orc_dims *d, const uint16_t *returned,
                          const int64_t *ret_offsets, int64_t n_ret_rows,
                          const int32_t *topk, const int32_t *slot,
                          const float *gates, const uint16_t *x,
                          const uint16_t *ylat, const uint16_t *w_lu_t,
                          const uint16_t *ws_gate, const uint16_t *ws_up,
                          const uint16_t *ws_down, const uint16_t *d_out,
                          uint16_t *d_returned, float *d_gates,
                          uint16_t *d_shared, uint16_t *dw_lat_up,
                          uint16_t *dws_down) {
  const int64_t T = d->T;
  const int32_t L = d->latent, D = d->d_model, k = d->top_k;
  const int32_t S = d->n_shared, Fs = d->d_ff_shared;
  double *dyl = (double *)malloc(sizeof(double) * (size_t)L);
  uint16_t *hs = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T * S * Fs + 1));
  memset(d_returned, 0, sizeof(uint16_t) * (size_t)(n_ret_rows * L));
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t *go = d_out + t * D;
    for (int32_t i = 0; i < L; ++i) {
      double acc = 0.0;
      for (int32_t c = 0; c < D; ++c) acc += bf(go[c]) * bf(w_lu_t[(int64_t)c * L + i]);
      dyl[i] = bf(to_bf(acc));
    }
    for (int32_t j = 0; j < k; ++j) {
      int32_t s = slot[t * k + j];
      int64_t row = s < 0 ? -1 : pool_row(d, ret_offsets, t, topk[t * k + j], s);
      if (row < 0) { /* dropped, or (ragged) a row the forward read as zero */
        d_gates[t * k + j] = 0.0f;
        continue;
      }
      double g = gates[t * k + j], dot = 0.0;
      for (int32_t i = 0; i < L; ++i) {
        d_returned[row * L + i] = to_bf(g * dyl[i]);
        dot += bf(returned[row * L + i]) * dyl[i];
      }
      d_gates[t * k + j] = (float)dot;
    }
    for (int32_t sh = 0; sh < S; ++sh)
      for (int32_t f = 0; f < Fs; ++f) {
        double dh = 0.0, a = 0.0, b = 0.0;
        for (int32_t c = 0; c < D; ++c)
          dh += bf(go[c]) * bf(ws_down[((int64_t)sh * D + c) * Fs + f]);
        dh = bf(to_bf(dh));
        const uint16_t *wg = ws_gate + ((int64_t)sh * Fs + f) * D;
        const uint16_t *wu = ws_up + ((int64_t)sh * Fs + f) * D;
        for (int32_t i = 0; i < D; ++i) a += bf(x[t * D + i]) * bf(wg[i]);
        for (int32_t i = 0; i < D; ++i) b += bf(x[t * D + i]) * bf(wu[i]);
        hs[(t * S + sh) * Fs + f] = to_bf(silu(a) * b);
        d_shared[(t * 2 * S + sh) * Fs + f] = to_bf(dh * b * silu_grad(a));
        d_shared[(t * 2 * S + S + sh) * Fs + f] = to_bf(dh * silu(a));
      }
  }
  for (int32_t c = 0; c < D; ++c) {
    for (int32_t i = 0; i < L; ++i) {
      double acc = 0.0;
      for (int64_t t = 0; t < T; ++t) acc += bf(d_out[t * D + c]) * bf(ylat[t * L + i]);
      dw_lat_up[(int64_t)c * L + i] = to_bf(acc);
    }
    for (int32_t sh = 0; sh < S; ++sh)
      for (int32_t f = 0; f < Fs; ++f) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t)
          acc += bf(d_out[t * D + c]) * bf(hs[(t * S + sh) * Fs + f]);
        dws_down[((int64_t)sh * D + c) * Fs + f] = to_bf(acc);
      }
  }
  free(dyl);
  free(hs);
}

/* Receiver side.  For every kept bank row u of group (wave, j) with
 * dy = d_ret[bank_src] (the gradient of its expert output):
 *   d_h[f] = bf16(sum_l dy[l] W_d,j[l][f])
 *   a, b = u.W_g,j, u.W_u,j;  h = bf16(silu(a) b)
 *   d_a = bf16(d_h b silu'(a)),  d_b = bf16(d_h silu(a))
 *   d_recv[bank_src] = bf16(sum_f d_a[f] W_g[f] + d_b[f] W_u[f]); other rows 0
 *   dw_down[j][l][f] = bf16(sum over expert j's rows of dy[l] h[f])
 *   dw_gate[j][f][l] = bf16(sum of d_a[f] u[l]), dw_up likewise with d_b,
 * the weight sums running over the rows in (wave, bank position) order. */
void orc_expert_ffn_backward(const orc_dims *d, const uint16_t *bank,
                             const int64_t *bank_offsets,
                             const int32_t *bank_src, const int32_t *bfill,
                             const uint16_t *w_gate, const uint16_t *w_up,
                             const uint16_t *w_down, const uint16_t *d_ret,
                             int64_t n_ret_rows, uint16_t *d_recv,
                             uint16_t *dw_gate, uint16_t *dw_up,
                             uint16_t *dw_down) {
  const int32_t L = d->latent, F = d->d_ff;
  const int32_t El = d->n_experts / d->n_ranks;
  const int64_t WL = (int64_t)F * L;
  double *gd = (double *)calloc((size_t)(El * WL), sizeof(double));
  double *gg = (double *)calloc((size_t)(El * WL), sizeof(double));
  double *gu = (double *)calloc((size_t)(El * WL), sizeof(double));
  double *u = (double *)malloc(sizeof(double) * (size_t)L);
  double *dy = (double *)malloc(sizeof(double) * (size_t)L);
  double *h = (double *)malloc(sizeof(double) * (size_t)F);
  double *da = (double *)malloc(sizeof(double) * (size_t)F);
  double *db = (double *)malloc(sizeof(double) * (size_t)F);
  memset(d_recv, 0, sizeof(uint16_t) * (size_t)(n_ret_rows * L));
  for (int32_t w = 0; w < d->n_waves; ++w)
    for (int32_t j = 0; j < El; ++j) {
      int32_t g = w * El + j;
      const uint16_t *Wg = w_gate + j * WL, *Wu = w_up + j * WL, *Wd = w_down + j * WL;
      for (int32_t p = 0; p < bfill[g]; ++p) {
        int64_t pos = group_start(d, bank_offsets, g) + p, src = bank_src[pos];
        for (int32_t l = 0; l < L; ++l) {
          u[l] = bf(bank[pos * L + l]);
          dy[l] = bf(d_ret[src * L + l]);
        }
        for (int32_t f = 0; f < F; ++f) {
          double dh = 0.0, a = 0.0, b = 0.0;
          for (int32_t l = 0; l < L; ++l) dh += dy[l] * bf(Wd[(int64_t)l * F + f]);
          dh = bf(to_bf(dh));
          for (int32_t l = 0; l < L; ++l) a += u[l] * bf(Wg[(int64_t)f * L + l]);
          for (int32_t l = 0; l < L; ++l) b += u[l] * bf(Wu[(int64_t)f * L + l]);
          h[f] = bf(to_bf(silu(a) * b));
          da[f] = bf(to_bf(dh * b * silu_grad(a)));
          db[f] = bf(to_bf(dh * silu(a)));
        }
        for (int32_t l = 0; l < L; ++l) {
          double acc = 0.0;
          for (int32_t f = 0; f < F; ++f)
            acc += da[f] * bf(Wg[(int64_t)f * L + l]) + db[f] * bf(Wu[(int64_t)f * L + l]);
          d_recv[src * L + l] = to_bf(acc);
        }
        for (int32_t l = 0; l < L; ++l)
          for (int32_t f = 0; f < F; ++f) gd[j * WL + (int64_t)l * F + f] += dy[l] * h[f];
        for (int32_t f = 0; f < F; ++f)
          for (int32_t l = 0; l < L; ++l) {
            gg[j * WL + (int64_t)f * L + l] += da[f] * u[l];
            gu[j * WL + (int64_t)f * L + l] += db[f] * u[l];
          }
      }
    }
  for (int64_t i = 0; i < El * WL; ++i) {
    dw_down[i] = to_bf(gd[i]);
    dw_gate[i] = to_bf(gg[i]);
    dw_up[i] = to_bf(gu[i]);
  }
  free(gd);
  free(gg);
  free(gu);
  free(u);
  free(dy);
  free(h);
  free(da);
  free(db);
}

/* Sender side.  d_pools holds the gradients of the pool rows (the sender's
 * [R][W][cap_send] layout, latent wide).  From z = x.W_ld, the pack copy and
 * the shared experts' inputs:
 *   dz[t]              = bf16(sum_j over kept (t, j) of d_pools[row(t,j)])
 *   dx[t][i]           = bf16(sum_l dz[t][l] W_ld[l][i]
 *                             + sum_s sum_f d_a[t,s,f] W_sg,s[f][i] + d_b[t,s,f] W_su,s[f][i])
 *   dw_lat_down[l][i]  = bf16(sum_t dz[t][l] x[t][i])               ([L][D])
 *   dws_gate[s][f][i]  = bf16(sum_t d_a[t,s,f] x[t][i]), dws_up likewise,
 * with d_a, d_b from d_shared ([T][2][S][Fs], the combine side's output). */
void orc_pack_backward(const orc_dims *d, const uint16_t *d_pools,
                       const int64_t *pool_offsets,
                       const int32_t *topk, const int32_t *slot,
                       const uint16_t *x, const uint16_t *d_shared,
                       const uint16_t *w_ld_t, const uint16_t *ws_gate,
                       const uint16_t *ws_up, uint16_t *dz, uint16_t *dx,
                       uint16_t *dw_lat_down, uint16_t *dws_gate,
                       uint16_t *dws_up) {
  const int64_t T = d->T;
  const int32_t L = d->latent, D = d->d_model, k = d->top_k;
  const int32_t S = d->n_shared, Fs = d->d_ff_shared;
  double *acc = (double *)malloc(sizeof(double) * (size_t)L);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t l = 0; l < L; ++l) acc[l] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t s = slot[t * k + j];
      int64_t row = s < 0 ? -1 : pool_row(d, pool_offsets, t, topk[t * k + j], s);
      if (row < 0) continue;
      for (int32_t l = 0; l < L; ++l) acc[l] += bf(d_pools[row * L + l]);
    }
    for (int32_t l = 0; l < L; ++l) dz[t * L + l] = to_bf(acc[l]);
    for (int32_t i = 0; i < D; ++i) {
      double o = 0.0;
      for (int32_t l = 0; l < L; ++l) o += bf(dz[t * L + l]) * bf(w_ld_t[(int64_t)l * D + i]);
      for (int32_t sh = 0; sh < S; ++sh)
        for (int32_t f = 0; f < Fs; ++f) {
          int64_t wi = ((int64_t)sh * Fs + f) * D + i;
          o += bf(d_shared[(t * 2 * S + sh) * Fs + f]) * bf(ws_gate[wi]) +
               bf(d_shared[(t * 2 * S + S + sh) * Fs + f]) * bf(ws_up[wi]);
        }
      dx[t * D + i] = to_bf(o);
    }
  }
  for (int32_t i = 0; i < D; ++i) {
    for (int32_t l = 0; l < L; ++l) {
      double a = 0.0;
      for (int64_t t = 0; t < T; ++t) a += bf(dz[t * L + l]) * bf(x[t * D + i]);
      dw_lat_down[(int64_t)l * D + i] = to_bf(a);
    }
    for (int32_t sh = 0; sh < S; ++sh)
      for (int32_t f = 0; f < Fs; ++f) {
        double ag = 0.0, au = 0.0;
        for (int64_t t = 0; t < T; ++t) {
          ag += bf(d_shared[(t * 2 * S + sh) * Fs + f]) * bf(x[t * D + i]);
          au += bf(d_shared[(t * 2 * S + S + sh) * Fs + f]) * bf(x[t * D + i]);
        }
        dws_gate[((int64_t)sh * Fs + f) * D + i] = to_bf(ag);
        dws_up[((int64_t)sh * Fs + f) * D + i] = to_bf(au);
      }
  }
  free(acc);
}

/* ------------------------------------------------------------------------ */
/* Backward on sampled outputs (full-size checks): the same arithmetic as    */
/* the functions above, for listed tokens, bank rows or weight entries.     */
/* ------------------------------------------------------------------------ */

/* Combine side for tokens[0..n): d_ret_rows [n][k][L] (the d_returned row
 * of each kept choice, 0 for a dropped one), d_gates [n][k], d_shared
 * [n][2][S][Fs].  Equal to orc_combine_backward's values for those tokens. */
void orc_combine_backward_tokens(const orc_dims *d, const uint16_t *returned,
                                 const int64_t *ret_offsets,
                                 const int32_t *topk, const int32_t *slot,
                                 const float *gates, const uint16_t *x,
                                 const uint16_t *w_lu_t, const uint16_t *ws_gate,
                                 const uint16_t *ws_up, const uint16_t *ws_down,
                                 const uint16_t *d_out, const int64_t *tokens,
                                 int64_t n, uint16_t *d_ret_rows,
                                 float *d_gates, uint16_t *d_shared) {
  const int32_t L = d->latent, D = d->d_model, k = d->top_k;
  const int32_t S = d->n_shared, Fs = d->d_ff_shared;
  double *dyl = (double *)malloc(sizeof(double) * (size_t)L);
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = tokens[r];
    const uint16_t *go = d_out + t * D;
    for (int32_t i = 0; i < L; ++i) {
      double acc = 0.0;
      for (int32_t c = 0; c < D; ++c) acc += bf(go[c]) * bf(w_lu_t[(int64_t)c * L + i]);
      dyl[i] = bf(to_bf(acc));
    }
    for (int32_t j = 0; j < k; ++j) {
      uint16_t *o = d_ret_rows + (r * k + j) * L;
      int32_t s = slot[t * k + j];
      int64_t row = s < 0 ? -1 : pool_row(d, ret_offsets, t, topk[t * k + j], s);
      if (row < 0) {
        memset(o, 0, sizeof(uint16_t) * (size_t)L);
        d_gates[r * k + j] = 0.0f;
        continue;
      }
      double g = gates[t * k + j], dot = 0.0;
      for (int32_t i = 0; i < L; ++i) {
        o[i] = to_bf(g * dyl[i]);
        dot += bf(returned[row * L + i]) * dyl[i];
      }
      d_gates[r * k + j] = (float)dot;
    }
    for (int32_t sh = 0; sh < S; ++sh)
      for (int32_t f = 0; f < Fs; ++f) {
        double dh = 0.0, a = 0.0, b = 0.0;
        for (int32_t c = 0; c < D; ++c)
          dh += bf(go[c]) * bf(ws_down[((int64_t)sh * D + c) * Fs + f]);
        dh = bf(to_bf(dh));
        const uint16_t *wg = ws_gate + ((int64_t)sh * Fs + f) * D;
        const uint16_t *wu = ws_up + ((int64_t)sh * Fs + f) * D;
        for (int32_t i = 0; i < D; ++i) a += bf(x[t * D + i]) * bf(wg[i]);
        for (int32_t i = 0; i < D; ++i) b += bf(x[t * D + i]) * bf(wu[i]);
        d_shared[(r * 2 * S + sh) * Fs + f] = to_bf(dh * b * silu_grad(a));
        d_shared[(r * 2 * S + S + sh) * Fs + f] = to_bf(dh * silu(a));
      }
  }
  free(dyl);
}

/* Weight-gradient entries of the combine side, summed over all T tokens in
 * order: which 0: dw_lat_up[ra[e]][cb[e]] = sum_t d_out[t][ra] ylat[t][cb];
 * which 1: dws_down[sh[e]][ra[e]][cb[e]] = sum_t d_out[t][ra] h_s[t][cb],
 * h_s = bf16(silu(x.W_sg,sh) (x.W_su,sh)) recomputed. */
void orc_combine_wgrad_entries(const orc_dims *d, const uint16_t *x,
                               const uint16_t *ylat, const uint16_t *ws_gate,
                               const uint16_t *ws_up, const uint16_t *d_out,
                               int32_t which, const int32_t *sh_idx,
                               const int32_t *ra, const int32_t *cb, int64_t n,
                               uint16_t *out) {
  const int64_t T = d->T;
  const int32_t L = d->latent, D = d->d_model, Fs = d->d_ff_shared;
  for (int64_t e = 0; e < n; ++e) {
    double acc = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      double v;
      if (which == 0) {
        v = bf(ylat[t * L + cb[e]]);
      } else {
        const uint16_t *wg = ws_gate + ((int64_t)sh_idx[e] * Fs + cb[e]) * D;
        const uint16_t *wu = ws_up + ((int64_t)sh_idx[e] * Fs + cb[e]) * D;
        double a = 0.0, b = 0.0;
        for (int32_t i = 0; i < D; ++i) a += bf(x[t * D + i]) * bf(wg[i]);
        for (int32_t i = 0; i < D; ++i) b += bf(x[t * D + i]) * bf(wu[i]);
        v = bf(to_bf(silu(a) * b));
      }
      acc += bf(d_out[t * D + ra[e]]) * v;
    }
    out[e] = to_bf(acc);
  }
}

/* Receiver side for bank positions pos[0..n) (kept rows): d_u [n][L], the
 * row each writes to d_recv[bank_src[pos]]. */
void orc_expert_ffn_backward_rows(const orc_dims *d, const uint16_t *bank,
                                  const int64_t *bank_offsets,
                                  const int32_t *bank_src,
                                  const uint16_t *w_gate, const uint16_t *w_up,
                                  const uint16_t *w_down, const uint16_t *d_ret,
                                  const int64_t *pos, int64_t n, uint16_t *d_u) {
  const int32_t L = d->latent, F = d->d_ff;
  const int32_t El = d->n_experts / d->n_ranks;
  const int64_t WL = (int64_t)F * L;
  double *da = (double *)malloc(sizeof(double) * (size_t)F);
  double *db = (double *)malloc(sizeof(double) * (size_t)F);
  for (int64_t r = 0; r < n; ++r) {
    const int64_t p = pos[r], src = bank_src[p];
    int32_t g = 0; /* bank group of position p */
    while (g + 1 < d->n_waves * El && group_start(d, bank_offsets, g + 1) <= p) ++g;
    const int32_t j = g % El;
    const uint16_t *Wg = w_gate + j * WL, *Wu = w_up + j * WL, *Wd = w_down + j * WL;
    for (int32_t f = 0; f < F; ++f) {
      double dh = 0.0, a = 0.0, b = 0.0;
      for (int32_t l = 0; l < L; ++l) dh += bf(d_ret[src * L + l]) * bf(Wd[(int64_t)l * F + f]);
      dh = bf(to_bf(dh));
      for (int32_t l = 0; l < L; ++l) a += bf(bank[p * L + l]) * bf(Wg[(int64_t)f * L + l]);
      for (int32_t l = 0; l < L; ++l) b += bf(bank[p * L + l]) * bf(Wu[(int64_t)f * L + l]);
      da[f] = bf(to_bf(dh * b * silu_grad(a)));
      db[f] = bf(to_bf(dh * silu(a)));
    }
    for (int32_t l = 0; l < L; ++l) {
      double acc = 0.0;
      for (int32_t f = 0; f < F; ++f)
        acc += da[f] * bf(Wg[(int64_t)f * L + l]) + db[f] * bf(Wu[(int64_t)f * L + l]);
      d_u[r * L + l] = to_bf(acc);
    }
  }
  free(da);
  free(db);
}

/* Weight-gradient entries of local expert j over its kept rows of every
 * wave, in (wave, position) order: which 0: dw_gate[j][ra][cb] (f, l);
 * 1: dw_up[j][ra][cb]; 2: dw_down[j][ra][cb] (l, f). */
void orc_expert_wgrad_entries(const orc_dims *d, const uint16_t *bank,
                              const int64_t *bank_offsets,
                              const int32_t *bank_src, const int32_t *bfill,
                              const uint16_t *w_gate, const uint16_t *w_up,
                              const uint16_t *w_down, const uint16_t *d_ret,
                              int32_t j, int32_t which, const int32_t *ra,
                              const int32_t *cb, int64_t n, uint16_t *out) {
  const int32_t L = d->latent, F = d->d_ff;
  const int32_t El = d->n_experts / d->n_ranks;
  const int64_t WL = (int64_t)F * L;
  const uint16_t *Wg = w_gate + j * WL, *Wu = w_up + j * WL, *Wd = w_down + j * WL;
  double *acc = (double *)calloc((size_t)n, sizeof(double));
  for (int32_t w = 0; w < d->n_waves; ++w) {
    const int32_t g = w * El + j;
    for (int32_t p = 0; p < bfill[g]; ++p) {
      const int64_t pos = group_start(d, bank_offsets, g) + p, src = bank_src[pos];
      const uint16_t *u = bank + pos * L, *dy = d_ret + src * L;
      for (int64_t e = 0; e < n; ++e) {
        const int32_t f = which == 2 ? cb[e] : ra[e];
        double dh = 0.0, a = 0.0, b = 0.0;
        for (int32_t l = 0; l < L; ++l) dh += bf(dy[l]) * bf(Wd[(int64_t)l * F + f]);
        dh = bf(to_bf(dh));
        for (int32_t l = 0; l < L; ++l) a += bf(u[l]) * bf(Wg[(int64_t)f * L + l]);
        for (int32_t l = 0; l < L; ++l) b += bf(u[l]) * bf(Wu[(int64_t)f * L + l]);
        if (which == 2) {
          acc[e] += bf(dy[ra[e]]) * bf(to_bf(silu(a) * b));
        } else {
          double dv = which == 0 ? bf(to_bf(dh * b * silu_grad(a))) : bf(to_bf(dh * silu(a)));
          acc[e] += dv * bf(u[cb[e]]);
        }
      }
    }
  }
  for (int64_t e = 0; e < n; ++e) out[e] = to_bf(acc[e]);
  free(acc);
}

/* Sender side for tokens[0..n): dz [n][L], dx [n][D]; d_shared is the full
 * [T][2][S][Fs] input. */
void orc_pack_backward_tokens(const orc_dims *d, const uint16_t *d_pools,
                              const int64_t *pool_offsets,
                              const int32_t *topk, const int32_t *slot,
                              const uint16_t *d_shared, const uint16_t *w_ld_t,
                              const uint16_t *ws_gate, const uint16_t *ws_up,
                              const int64_t *tokens, int64_t n, uint16_t *dz,
                              uint16_t *dx) {
  const int32_t L = d->latent, D = d->d_model, k = d->top_k;
  const int32_t S = d->n_shared, Fs = d->d_ff_shared;
  double *acc = (double *)malloc(sizeof(double) * (size_t)L);
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = tokens[r];
    for (int32_t l = 0; l < L; ++l) acc[l] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t s = slot[t * k + j];
      int64_t row = s < 0 ? -1 : pool_row(d, pool_offsets, t, topk[t * k + j], s);
      if (row < 0) continue;
      for (int32_t l = 0; l < L; ++l) acc[l] += bf(d_pools[row * L + l]);
    }
    for (int32_t l = 0; l < L; ++l) dz[r * L + l] = to_bf(acc[l]);
    for (int32_t i = 0; i < D; ++i) {
      double o = 0.0;
      for (int32_t l = 0; l < L; ++l) o += bf(dz[r * L + l]) * bf(w_ld_t[(int64_t)l * D + i]);
      for (int32_t sh = 0; sh < S; ++sh)
        for (int32_t f = 0; f < Fs; ++f) {
          int64_t wi = ((int64_t)sh * Fs + f) * D + i;
          o += bf(d_shared[(t * 2 * S + sh) * Fs + f]) * bf(ws_gate[wi]) +
               bf(d_shared[(t * 2 * S + S + sh) * Fs + f]) * bf(ws_up[wi]);
        }
      dx[r * D + i] = to_bf(o);
    }
  }
  free(acc);
}

/* Weight-gradient entries of the sender side over all T tokens in order:
 * which 0: dw_lat_down[ra][cb] = sum_t dz[t][ra] x[t][cb] (dz as in
 * orc_pack_backward); 1: dws_gate, 2: dws_up [sh*Fs + ra][cb] =
 * sum_t d_shared[t][gate or up][sh][ra] x[t][cb]. */
void orc_pack_wgrad_entries(const orc_dims *d, const uint16_t *d_pools,
                            const int64_t *pool_offsets,
                            const int32_t *topk, const int32_t *slot,
                            const uint16_t *x, const uint16_t *d_shared,
                            int32_t which, const int32_t *sh_idx,
                            const int32_t *ra, const int32_t *cb, int64_t n,
                            uint16_t *out) {
  const int64_t T = d->T;
  const int32_t L = d->latent, D = d->d_model, k = d->top_k;
  const int32_t S = d->n_shared, Fs = d->d_ff_shared;
  for (int64_t e = 0; e < n; ++e) {
    double acc = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      double v;
      if (which == 0) {
        double z = 0.0;
        for (int32_t j = 0; j < k; ++j) {
          int32_t s = slot[t * k + j];
          int64_t row = s < 0 ? -1 : pool_row(d, pool_offsets, t, topk[t * k + j], s);
          if (row >= 0) z += bf(d_pools[row * L + ra[e]]);
        }
        v = bf(to_bf(z));
      } else {
        v = bf(d_shared[(t * 2 * S + (which == 2 ? S : 0) + sh_idx[e]) * Fs + ra[e]]);
      }
      acc += v * bf(x[t * D + cb[e]]);
    }
    out[e] = to_bf(acc);
  }
}
