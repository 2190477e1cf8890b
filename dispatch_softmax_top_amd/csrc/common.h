// common.h -- shared pieces of libmoe: host-side checks, errors, launch
// bookkeeping, and device helpers for gfx950 (wave64, bf16 MFMA).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int hip_status(hipError_t e, const char *what);

// Argument checks shared by the entry points; return MOE_OK or an error.
// check_dims also checks the environment variable MOE_GEMM_CUS.
int check_dims(const moe_dims *d);
// MOE_GEMM_CUS, the CU count the GEMM launchers plan for: *cus = 0 if unset,
// else its value; an error unless it is a multiple of 8, at least 8.
int gemm_cus_env(int *cus);
int check_ptr(const void *p, const char *name, bool may_be_null = false);

inline int32_t experts_per_rank(const moe_dims &d) { return d.n_experts / d.n_ranks; }
inline int32_t tokens_per_wave(const moe_dims &d) { return (d.T + d.n_waves - 1) / d.n_waves; }
inline bool ragged(const moe_dims &d) { return d.cap_send == 0; }
// Return rows per receive row: 4 with dedup (one per tail id), else 1.
inline int ret_slots(const moe_dims &d) { return d.dedup ? 4 : 1; }
inline int64_t row_bytes(const moe_dims &d) { return 2 * (int64_t)d.latent + 16; }
// How a (token, choice) assignment finds its sender pool: key = dest * Wk +
// t / Tw, row = key * rows + slot.  Waves by token: (W, T_w, C_s).  Chunked
// waves: the key is the destination alone (Wk = 1, Tw past every token) and
// its pool holds all W chunks (rows = W * C_s).
struct PoolKey {
  int Wk, Tw, rows;
};
inline PoolKey pool_key(const moe_dims &d) {
  if (d.wave_mode == MOE_WAVES_CHUNKS) return {1, d.T + 1, d.n_waves * d.cap_send};
  return {d.n_waves, tokens_per_wave(d), d.cap_send};
}

// Launch bookkeeping: records hipEvents around a launch when timing is on.
struct ProfScope {
  ProfScope(const char *name, hipStream_t s);
  ~ProfScope();
  int slot;
  hipStream_t stream;
};

// Launch a kernel and report a launch error as MOE_ERR_HIP.
template <typename... KArgs, typename... Args>
int launch(const char *name, void (*kernel)(KArgs...), dim3 grid, dim3 block,
           size_t lds, hipStream_t s, Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return MOE_OK;
  ProfScope p(name, s);
  hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<KArgs>(args)...);
  return hip_status(hipGetLastError(), name);
}

#define MOE_TRY(x)                 \
  do {                             \
    int _rc = (x);                 \
    if (_rc != MOE_OK) return _rc; \
  } while (0)

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// ---------------------------------------------------------------------------
// device side
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's conversion
// instruction (v_cvt_pk_bf16_f32) under the default rounding mode, two
// values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// 16-byte global load / store, optionally non-temporal (streamed data that
// is touched once: the access does not displace reused lines in L2 / MALL).
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4 *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(u32x4 *p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Butterfly reductions over the 64 lanes of a wave (every lane gets the result).
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

// Lanes below this one.
__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Mask of the active lanes holding the same key (keys < 2^bits).
__device__ __forceinline__ uint64_t match_key(uint32_t key, int bits) {
  uint64_t m = ballot(true);
  for (int b = 0; b < bits; ++b) {
    uint64_t v = ballot((key >> b) & 1u);
    m &= ((key >> b) & 1u) ? v : ~v;
  }
  return m;
}

// Logistic sigmoid and silu(a) = a * sigmoid(a), with the hardware exp2 and
// reciprocal (each within about one ulp; the results are rounded to bf16).
__device__ __forceinline__ float sigmoid_f32(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}
__device__ __forceinline__ float silu_f32(float a) { return a * sigmoid_f32(a); }

// Dispatch order of workgroups is round-robin over the 8 XCDs.  Map the
// hardware block id to a logical tile id so that each XCD gets one
// contiguous range of tiles (neighbouring tiles share operand panels in
// that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int NX = 8;
  int xcd = bid % NX, local = bid / NX;
  int per = nblocks / NX, rem = nblocks % NX;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// For tiles of unequal cost (products whose K is known only on the device):
// XCD x takes groups x, x + 8, x + 16, ... of G consecutive tiles, so a run
// of long tiles is spread over every XCD instead of filling one or two, while
// the G tiles of a group still share an operand panel in one L2.  Blocks past
// the last whole round of 8 groups keep their own index.
template <int G>
__device__ __forceinline__ int xcd_spread(int bid, int nblocks) {
  constexpr int NX = 8;
  if (bid >= nblocks - nblocks % (NX * G)) return bid;
  const int xcd = bid % NX, local = bid / NX;
  return ((local / G) * NX + xcd) * G + local % G;
}

}  // namespace moe
