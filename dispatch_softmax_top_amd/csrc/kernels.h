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

// Routed experts over the bank's groups (group g uses local expert g % E_l):
// H rows = bank rows, H[:, 0:F] = bf16(silu(u.Wg^T) * (u.Wu^T)).
int gemm_expert_swiglu(const moe_dims &d, const uint16_t *bank, const int64_t *bank_offsets,
                       const int32_t *bfill, int64_t n_bank_rows, const uint16_t *wg,
                       const uint16_t *wu, uint16_t *H, float *part, hipStream_t s);
// ret[bank_src[r]] = bf16(H[r] . Wd^T) for every kept bank row r.
int gemm_expert_down(const moe_dims &d, const uint16_t *H, const int64_t *bank_offsets,
                     const int32_t *bfill, const int32_t *bank_src, int64_t n_bank_rows,
                     const uint16_t *wd, uint16_t *ret, int64_t n_ret, float *part,
                     hipStream_t s);

}  // namespace moe
