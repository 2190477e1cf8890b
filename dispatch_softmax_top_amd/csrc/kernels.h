// kernels.h -- host launchers shared between the translation units.
#pragma once
#include "common.h"

namespace moe {

// One K segment of a dense product: C += A[:, 0:K] . B[:, 0:K]^T.
struct DenseSeg {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B;
  int64_t ldb;
  int K;
};

// Tail split: the last, partly filled round of a product's block tiles can
// be cut along K into parts that write fp32 partial tiles to `part` (a
// buffer of gemm_split_bytes(), NULL: no split); a second kernel sums them.
int64_t gemm_split_bytes();

// Workspace pieces: the shared experts' intermediate [T, S*Fs] bf16, and the
// routed experts' intermediate and return-row flags of the FFN call.
inline int64_t shared_h_bytes(const moe_dims &d) {
  return align_up((int64_t)d.T * d.n_shared * d.d_ff_shared * 2, 256);
}
inline int64_t ffn_h_bytes(const moe_dims &d, int64_t bank_rows) {
  return align_up(bank_rows * d.d_ff * 2, 256);
}
inline int64_t ffn_flag_bytes(int64_t ret_rows) { return align_up(ret_rows * 4, 256); }

// C[M, N] (ldc) = sum over segments; M, N >= 1, every K % 32 == 0.
int gemm_latent_down(int M, int N, const DenseSeg &seg, uint16_t *C, int64_t ldc, hipStream_t s);
int gemm_up_shared(int M, int N, int nseg, const DenseSeg *segs, uint16_t *C, int64_t ldc,
                   float *part, hipStream_t s);

// H[M, S*F] = for each shared expert s: bf16(silu(x.Wg_s^T) * (x.Wu_s^T)).
int gemm_shared_swiglu(int M, const uint16_t *x, int64_t ldx, int K, const uint16_t *wg,
                       const uint16_t *wu, int S, int F, uint16_t *H, float *part,
                       hipStream_t s);

// Work queue of the two grouped FFN GEMMs (gemm_queue_bytes(), 256-byte
// aligned): counters [0, 16) zeroed before the SwiGLU GEMM (ret_rows_mark
// does it), slots from int 64 on.  NULL: static unit order.
int64_t gemm_queue_bytes();

// Routed experts over the bank's groups (group g uses local expert g % E_l):
// H rows = bank rows, H[:, 0:F] = bf16(silu(u.Wg^T) * (u.Wu^T)).
int gemm_expert_swiglu(const moe_dims &d, const uint16_t *bank, const int64_t *bank_offsets,
                       const int32_t *bfill, int64_t n_bank_rows, const uint16_t *wg,
                       const uint16_t *wu, uint16_t *H, float *part, int32_t *queue,
                       hipStream_t s);
// ret[bank_src[r]] = bf16(H[r] . Wd^T) for every kept bank row r.
int gemm_expert_down(const moe_dims &d, const uint16_t *H, const int64_t *bank_offsets,
                     const int32_t *bfill, const int32_t *bank_src, int64_t n_bank_rows,
                     const uint16_t *wd, uint16_t *ret, int64_t n_ret, float *part,
                     int32_t *queue, hipStream_t s);

// Return rows: flags[r] = 1 for every row some kept bank row writes (bank_src),
// then every unflagged row of ret [n_ret][L] set to zero.  zero16: NULL, or
// 16 ints cleared with the flags (the grouped GEMMs' queue counters).
int ret_rows_mark(const int32_t *bank_src, int64_t n_bank, int32_t *flags, int64_t n_ret,
                  int32_t *zero16, hipStream_t s);
int ret_rows_zero_unmarked(const int32_t *flags, uint16_t *ret, int L, int64_t n_ret,
                           hipStream_t s);

// Sum over each token's kept choices of gates[t, j] * rows[row(t, j)] (gates
// NULL: weight 1), rounded to bf16: the combine's gather (combine.hip).
int combine_gather_rows(const moe_dims &d, const uint16_t *rows, const int64_t *offsets,
                        const int32_t *topk, const int32_t *slot, const float *gates,
                        uint16_t *out, hipStream_t s);

// ---------------------------------------------------------------------------
// backward pass
// ---------------------------------------------------------------------------

// Workspace bytes of the backward calls; n_rows: bank rows (ragged FFN).
int64_t bwd_ws_bytes(const moe_dims &d, int call, int64_t n_rows);

// Packed per-group K ranges (ragged weight gradients): a group of `rows`
// bank rows takes its rows rounded up to whole K tiles of 32, and at least
// 8 K tiles (the fewest K tiles a product reads), so no product reads into
// the next group's range.
__host__ __device__ inline int64_t kpack_len(int64_t rows) {
  const int64_t r = (rows + 31) / 32 * 32;
  return r > 256 ? r : 256;
}

// C[M, N] (ldc) = sum over nseg <= 2 segments of A . B^T (bf16 out).
// tail_name: the launch name of the kernel finishing a split last round.
int gemm_nt(const char *name, const char *tail_name, int M, int N, int nseg,
            const DenseSeg *segs, uint16_t *C, int64_t ldc, float *part, hipStream_t s);
// nbatch products of one segment: product b at A + b*bsA, B + b*bsB, C + b*bsC.
int gemm_nt_batched(const char *name, const char *tail_name, int M, int N, const DenseSeg &seg,
                    int nbatch, int64_t bsA, int64_t bsB, uint16_t *C, int64_t ldc, int64_t bsC,
                    float *part, hipStream_t s);
// Independent products C_p[M_p, N_p] = A_p . B_p^T with one K, in one launch
// (at most 18).  With kfill, product p's K is only the sum over w < kW of
// kfill[w * kEl + kgroup] (rounded up; the operands are zero past it), read on
// the device: the bank's fill of one local expert over its waves.
struct NtProd {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B;
  int64_t ldb;
  uint16_t *C;
  int64_t ldc;
  int M, N;
  int kgroup;
};
// kpack: product p's K range starts at the sum of kpack_len(K rows of the
// groups before kgroup[p]) in its operands (the groups' ranges packed one
// after another, read on the device); otherwise at 0.
int gemm_nt_multi(const char *name, const char *tail_name, int nprod, const NtProd *prods, int K,
                  float *part, hipStream_t s, const int32_t *kfill = nullptr, int kW = 0,
                  int kEl = 0, bool kpack = false);
// Shared experts recomputed with the SwiGLU gradient epilogue: dH[:, dh_col0 +
// s*F + f] in, H = h_s [M, S*F] and AB [M, 2*S*F] (d_a of every expert, then
// d_b) out.
int gemm_shared_swiglu_bwd(int M, const uint16_t *x, int64_t ldx, int K, const uint16_t *wg,
                           const uint16_t *wu, int S, int F, const uint16_t *dH, int64_t ld_dh,
                           int dh_col0, uint16_t *H, uint16_t *AB, float *part, hipStream_t s);
// Routed experts recomputed over the bank (groups at g * cap_recv, or at
// bank_offsets in ragged mode) with the SwiGLU gradient epilogue: dH, H
// [bank rows, F], AB [bank rows, 2F].  With HT and ABT, h goes to HT
// instead of H and d_a | d_b also to ABT, transposed into the bank-order
// layout the weight gradients read (per-expert blocks of ldt columns, or with
// kpack one block of packed expert ranges; zero past each expert's fill up
// to its padded end), when the bank's product groups allow it; *transposed
// tells whether they did (else H is written and the caller transposes).
int gemm_expert_swiglu_bwd(const moe_dims &d, const uint16_t *bank, const int64_t *bank_offsets,
                           const int32_t *bfill,
                           int64_t n_bank_rows, const uint16_t *wg, const uint16_t *wu,
                           const uint16_t *dH, uint16_t *H, uint16_t *AB, float *part,
                           hipStream_t s, uint16_t *HT = nullptr, uint16_t *ABT = nullptr,
                           int64_t ldt = 0, bool kpack = false, bool *transposed = nullptr);
// Grouped over the bank's groups (bank_offsets: ragged mode, else NULL):
// out[dst[r]] = A[r] . B_j^T, A [bank rows][K], B [E_l][N][K].  queue: as
// for gemm_expert_down (counters 8..15 zeroed before the launch), or NULL.
int gemm_grouped_nt(const char *name, const char *tail_name, const moe_dims &d,
                    const uint16_t *A, int K, const int64_t *bank_offsets, const int32_t *bfill,
                    const int32_t *dst,
                    int64_t n_bank_rows, const uint16_t *B, int N, uint16_t *out, int64_t n_out,
                    float *part, int32_t *queue, hipStream_t s);

}  // namespace moe
