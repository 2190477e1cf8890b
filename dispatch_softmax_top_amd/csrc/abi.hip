// abi.hip -- host-side half of the C ABI: errors, argument checks,
// capacities, workspace sizes and the optional per-kernel event timing.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "kernels.h"
#include "rank.h"

namespace moe {

static thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_ptr(const void *p, const char *name, bool may_be_null) {
  if (!p) return may_be_null ? MOE_OK : fail(MOE_ERR_INVALID, "%s is NULL", name);
  if ((uintptr_t)p % 16) return fail(MOE_ERR_INVALID, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

int gemm_cus_env(int *cus) {
  *cus = 0;
  const char *e = getenv("MOE_GEMM_CUS");
  if (!e || !*e) return MOE_OK;
  char *end = nullptr;
  const long v = strtol(e, &end, 10);
  if (*end || v < 8 || v % 8 || v > (1 << 20))
    return fail(MOE_ERR_INVALID, "MOE_GEMM_CUS=%s: a multiple of 8, at least 8, expected", e);
  *cus = (int)v;
  return MOE_OK;
}

int check_dims(const moe_dims *d) {
  int cus = 0;
  MOE_TRY(gemm_cus_env(&cus));
  if (!d) return fail(MOE_ERR_INVALID, "dims is NULL");
  if (d->T < 1 || d->d_model < 1 || d->latent < 1 || d->n_experts < 1 || d->n_ranks < 1 ||
      d->top_k < 1 || d->n_waves < 1 || d->d_ff < 1 || d->n_shared < 0 ||
      d->d_ff_shared < 1 || d->cap_send < 0 || d->cap_recv < 0)
    return fail(MOE_ERR_INVALID, "dims: sizes must be positive (n_shared, caps >= 0)");
  if (d->n_experts % d->n_ranks)
    return fail(MOE_ERR_INVALID, "dims: n_experts %% n_ranks != 0");
  if ((d->cap_send == 0) != (d->cap_recv == 0))
    return fail(MOE_ERR_INVALID, "dims: cap_send and cap_recv must be both 0 (ragged) or both > 0");
  if (d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID, "dims: top_k > n_experts");
  if (d->wave_mode != MOE_WAVES_TOKENS && d->wave_mode != MOE_WAVES_CHUNKS)
    return fail(MOE_ERR_INVALID, "dims: wave_mode must be MOE_WAVES_TOKENS or MOE_WAVES_CHUNKS");
  if (d->wave_mode == MOE_WAVES_CHUNKS && d->cap_send == 0)
    return fail(MOE_ERR_INVALID, "dims: chunked waves need fixed capacities");
  if (d->dedup != 0 && d->dedup != 1) return fail(MOE_ERR_INVALID, "dims: dedup must be 0 or 1");
  if (d->dedup && d->cap_send == 0)
    return fail(MOE_ERR_INVALID, "dims: dedup needs fixed capacities");
  if (d->n_experts > 1024 || d->top_k > 32)
    return fail(MOE_ERR_UNSUPPORTED, "dims: n_experts <= 1024 and top_k <= 32 supported");
  if (d->latent % 64 || d->d_model % 64)
    return fail(MOE_ERR_UNSUPPORTED, "dims: latent and d_model must be multiples of 64");
  // the row-copy kernels keep a whole latent row in registers (16 chunks per lane)
  if (d->latent > 8192) return fail(MOE_ERR_UNSUPPORTED, "dims: latent <= 8192");
  if (d->d_ff % 128 || d->d_ff_shared % 128)
    return fail(MOE_ERR_UNSUPPORTED, "dims: d_ff and d_ff_shared must be multiples of 128");
  if ((int64_t)d->n_ranks * d->n_waves > 1024 ||
      (int64_t)d->n_waves * experts_per_rank(*d) > 1024)
    return fail(MOE_ERR_UNSUPPORTED, "dims: at most 1024 pools and 1024 bank groups");
  if (d->n_shared > 4) return fail(MOE_ERR_UNSUPPORTED, "dims: n_shared <= 4");
  if ((int64_t)d->T * d->top_k >= (1ll << 31))
    return fail(MOE_ERR_UNSUPPORTED, "dims: T * top_k must fit in int32");
  // the combine runs up to 16 waves per token (one per part of its row)
  if (d->T > (1 << 27)) return fail(MOE_ERR_UNSUPPORTED, "dims: T <= 2^27");
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// per-kernel event timing
// ---------------------------------------------------------------------------

struct Pending {
  const char *name;
  hipEvent_t a, b;
};
struct Total {
  std::string name;
  double ms;
  int64_t n;
};
static bool g_prof = false;
static std::vector<Pending> g_pending;
static std::vector<hipEvent_t> g_pool;
static std::vector<Total> g_totals;

static hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

ProfScope::ProfScope(const char *name, hipStream_t s) : slot(-1), stream(s) {
  if (!g_prof) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  (void)hipEventRecord(a, s);
  g_pending.push_back({name, a, b});
  slot = (int)g_pending.size() - 1;
}

ProfScope::~ProfScope() {
  if (slot >= 0) (void)hipEventRecord(g_pending[slot].b, stream);
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_last_error(void) { return g_err; }

int moe_capacity(const moe_dims *d, int64_t sn, int64_t sd, int64_t rn, int64_t rd,
                 int32_t *cap_send, int32_t *cap_recv) {
  clear_error();
  if (!d || !cap_send || !cap_recv) return fail(MOE_ERR_INVALID, "moe_capacity: NULL argument");
  if (sn <= 0 || sd <= 0 || rn <= 0 || rd <= 0)
    return fail(MOE_ERR_INVALID, "moe_capacity: capacity factors must be positive");
  if (d->T < 1 || d->n_waves < 1 || d->top_k < 1 || d->n_ranks < 1 || d->n_experts < 1 ||
      d->n_experts % d->n_ranks)
    return fail(MOE_ERR_INVALID, "moe_capacity: bad dims");
  // mean rows per buffer per wave, times cf, rounded up: ceil(num*Tw*k / (den*groups))
  int64_t tw = tokens_per_wave(*d);
  __int128 a = (__int128)sn * tw * d->top_k, b = (__int128)sd * d->n_ranks;
  __int128 cs = (a + b - 1) / b;
  a = (__int128)rn * tw * d->top_k;
  b = (__int128)rd * experts_per_rank(*d);
  __int128 cr = (a + b - 1) / b;
  if (cs > INT32_MAX || cr > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_capacity: overflow");
  *cap_send = (int32_t)cs;
  *cap_recv = (int32_t)cr;
  return MOE_OK;
}

int64_t moe_workspace_bytes(const moe_dims *d, int call, int64_t n_rows) {
  clear_error();
  MOE_TRY(check_dims(d));
  const int64_t R = d->n_ranks, W = d->n_waves, El = experts_per_rank(*d);
  switch (call) {
    case MOE_CALL_ROUTE:
      return 0;
    case MOE_CALL_PACK:  // per-tile key counts of the sender slot assignment
      return rank_ws_bytes((int64_t)d->T * d->top_k, (int)(R * W));
    case MOE_CALL_BANK: {  // per-tile key counts of the receiver slot assignment
      int64_t items = ragged(*d) ? n_rows : R * W * d->cap_send * ret_slots(*d);
      if (items < 0) return fail(MOE_ERR_INVALID, "moe_workspace_bytes: n_rows < 0");
      return rank_ws_bytes(items, (int)(W * El));
    }
    case MOE_CALL_FFN: {  // intermediate h, return-row flags, GEMM work queue, split partial tiles
      int64_t bank_rows = ragged(*d) ? n_rows : W * El * d->cap_recv;
      int64_t ret_rows = ragged(*d) ? n_rows : R * W * d->cap_send * ret_slots(*d);
      if (bank_rows < 0) return fail(MOE_ERR_INVALID, "moe_workspace_bytes: n_rows < 0");
      return ffn_h_bytes(*d, bank_rows) + ffn_flag_bytes(ret_rows) + gemm_queue_bytes() +
             gemm_split_bytes();
    }
    case MOE_CALL_COMBINE:  // shared experts' intermediate, split partial tiles
      return shared_h_bytes(*d) + gemm_split_bytes();
    case MOE_CALL_COMBINE_SHARED:  // split partial tiles
      return gemm_split_bytes();
    case MOE_CALL_COMBINE_BWD:
    case MOE_CALL_FFN_BWD:
    case MOE_CALL_PACK_BWD:  // transposed operands, intermediates, split partial tiles
      if (d->dedup) return fail(MOE_ERR_UNSUPPORTED, "moe_workspace_bytes: backward without dedup only");
      if (n_rows < 0) return fail(MOE_ERR_INVALID, "moe_workspace_bytes: n_rows < 0");
      return bwd_ws_bytes(*d, call, n_rows);
    default:
      return fail(MOE_ERR_INVALID, "moe_workspace_bytes: unknown call %d", call);
  }
}

int moe_profile_enable(int on) {
  g_prof = on != 0;
  return MOE_OK;
}

int moe_profile_collect(void) {
  clear_error();
  for (auto &p : g_pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(p.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.a, p.b);
    if (e != hipSuccess) return hip_status(e, "moe_profile_collect");
    Total *t = nullptr;
    for (auto &x : g_totals)
      if (x.name == p.name) t = &x;
    if (!t) {
      g_totals.push_back({p.name, 0.0, 0});
      t = &g_totals.back();
    }
    t->ms += ms;
    t->n += 1;
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  g_pending.clear();
  return MOE_OK;
}

int moe_profile_get(int i, char *name, int name_len, double *total_ms, int64_t *launches) {
  if (i < 0 || i >= (int)g_totals.size()) return MOE_ERR_INVALID;
  if (name && name_len > 0) snprintf(name, (size_t)name_len, "%s", g_totals[i].name.c_str());
  if (total_ms) *total_ms = g_totals[i].ms;
  if (launches) *launches = g_totals[i].n;
  return MOE_OK;
}

void moe_profile_reset(void) { g_totals.clear(); }

}  // extern "C"
