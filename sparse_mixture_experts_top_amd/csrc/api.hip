// C ABI of the scattered mixture-of-experts hot path (declared in
// include/smoe.h): host-side validation, workspace layout and the
// launch sequence of each entry point.  Nothing here allocates,
// synchronises or copies device memory, and no HIP object (stream, event)
// is created: work is enqueued on the caller's stream, and on the caller's
// second stream where an entry point takes one (struct smoe_aux).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernels.h"
#include "smoe.h"

using namespace smoe;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SMOE_OK;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(SMOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;

// events attached by smoe_set_role_events
hipEvent_t g_role_ev[SMOE_ROLE_COUNT][2] = {};

// The caller's second stream (struct smoe_aux), forked from the main
// stream with one event and joined back with the other.  Once forked, the
// join is recorded and waited for on every way out of the scope, errors
// included, so that no work on the second stream is left unordered with
// the caller's stream (and the buffers it reads) when the call returns.
struct Fork {
  const smoe_aux* aux;
  hipStream_t main;
  bool forked = false;
  Fork(const smoe_aux* a, hipStream_t st) : aux(a && a->stream && a->fork_event && a->join_event ? a : nullptr), main(st) {}
  bool usable() const { return aux != nullptr; }
  hipStream_t side() const { return static_cast<hipStream_t>(aux->stream); }
  hipError_t fork() {
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(aux->fork_event), main);
    if (e != hipSuccess) return e;
    e = hipStreamWaitEvent(side(), static_cast<hipEvent_t>(aux->fork_event), 0);
    if (e == hipSuccess) forked = true;
    return e;
  }
  hipError_t join() {
    if (!forked) return hipSuccess;
    forked = false;
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(aux->join_event), side());
    hipError_t w = hipStreamWaitEvent(main, static_cast<hipEvent_t>(aux->join_event), 0);
    return e != hipSuccess ? e : w;
  }
  ~Fork() { (void)join(); }
};

// Brackets the launches issued during its lifetime with the role's events.
struct RoleTimer {
  int role;
  hipStream_t st;
  RoleTimer(int r, hipStream_t s) : role(r), st(s) {
    if (g_role_ev[role][0]) (void)hipEventRecord(g_role_ev[role][0], st);
  }
  ~RoleTimer() {
    if (g_role_ev[role][1]) (void)hipEventRecord(g_role_ev[role][1], st);
  }
};

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures, so the *_workspace_bytes functions replay the exact layout.
struct Arena {
  char* base;
  size_t used = 0;
  explicit Arena(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    used = (used + kAlign - 1) / kAlign * kAlign;
    void* p = base ? base + used : nullptr;
    used += std::max<size_t>(bytes, 1);
    return p;
  }
};

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t esize(int dtype) { return dtype == SMOE_BF16 ? 2 : 4; }

int check_common(int64_t T, int32_t k, int32_t E, int32_t dtype) {
  if (dtype != SMOE_F32 && dtype != SMOE_BF16) return fail(SMOE_ERR_DTYPE, "dtype %d is not SMOE_F32/SMOE_BF16", dtype);
  if (E < 1 || E > kMaxExperts) return fail(SMOE_ERR_SHAPE, "E=%d outside [1, %d]", E, kMaxExperts);
  if (k < 1) return fail(SMOE_ERR_SHAPE, "k=%d < 1", k);
  if (T < 0) return fail(SMOE_ERR_SHAPE, "T=%lld < 0", (long long)T);
  if (T * int64_t(k) > INT32_MAX / 2) return fail(SMOE_ERR_SHAPE, "T*k=%lld too large", (long long)(T * k));
  return SMOE_OK;
}

int check_dim(int64_t d, const char* name) {
  if (d < 8 || d % 8 != 0 || d > (int64_t(1) << 24))
    return fail(SMOE_ERR_SHAPE, "%s=%lld must be a positive multiple of 8", name, (long long)d);
  return SMOE_OK;
}

// bf16 grouped products address their operands through buffer descriptors
// with 32-bit byte offsets: every tensor they read (a [T*k, d] activation,
// one expert's [d_in, d_out] weights) must stay below 4 GiB
int check_extent(int32_t dtype, int64_t rows, int64_t cols, const char* what) {
  constexpr int64_t kMaxBytes = int64_t(0xFFFFFFF0u);
  if (dtype == SMOE_BF16 && rows * cols * 2 > kMaxBytes)
    return fail(SMOE_ERR_SHAPE, "%s of %lld x %lld bf16 exceeds the 4 GiB operand limit", what, (long long)rows,
                (long long)cols);
  return SMOE_OK;
}

#define SMOE_TRY(x)            \
  do {                         \
    int _s = (x);              \
    if (_s != SMOE_OK) return _s; \
  } while (0)

#define SMOE_HIP(x, where)                              \
  do {                                                  \
    hipError_t _e = (x);                                \
    if (_e != hipSuccess) return hip_status(_e, where); \
  } while (0)

int need_ptr(const void* p, const char* name) {
  if (!p) return fail(SMOE_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(SMOE_ERR_SHAPE, "%s is not 16-byte aligned", name);
  return SMOE_OK;
}

GemmArgs blank_args(const int* offsets, const int* sidx, int E, int M) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.offsets = offsets;
  a.sidx = sidx;
  a.E = E;
  a.M = M;
  a.a_fan = a.b_fan = a.aux_fan = 1;
  return a;
}

// ---- workspace layouts ------------------------------------------------------
struct PlFwdWs {
  float* pairs = nullptr;
};
void layout_pl_fwd(Arena& ar, int64_t M, int64_t d_out, bool with_gates, PlFwdWs& w) {
  if (with_gates) w.pairs = static_cast<float*>(ar.take(size_t(M) * d_out * 4));
}

// Upper bound of split-K partial bytes for a weight-gradient product.
size_t dw_partial_bytes(int64_t M, int E, int64_t Mo, int64_t N, int bf16) {
  GemmArgs a = blank_args(nullptr, nullptr, E, int(M));
  a.Mo = int(Mo);
  a.N = int(N);
  GemmPlan pl;
  plan_gemm(a, pl, SEG_K, EPI_PARTIAL, 0, bf16, 1);
  return size_t(a.mt_ub) * size_t(Mo) * size_t(N) * 4;
}

int dg_slots(int64_t M, int E, int64_t N, int bf16) {
  GemmArgs a = blank_args(nullptr, nullptr, E, int(M));
  a.N = int(N);
  GemmPlan pl;
  plan_gemm(a, pl, SEG_M, EPI_STORE, 0, bf16, 1);
  return pl.slots;
}

struct PlBwdWs {
  float* pairs = nullptr;    // dx contributions [M, d_in] when x was read k times
  float* dgpart = nullptr;   // [slots, M]
  float* gg = nullptr;       // the gates in grouped order [M] (the dw product's row scales)
  float* partial = nullptr;  // dw split-K partials
};
void layout_pl_bwd(Arena& ar, int64_t T, int k, int E, int64_t x_rows, int64_t d_in, int64_t d_out, bool x_grouped,
                   bool with_gates, int bf16, PlBwdWs& w) {
  const int64_t M = T * k;
  const bool fan_k = !x_grouped && x_rows == T && k > 1;
  if (fan_k) w.pairs = static_cast<float*>(ar.take(size_t(M) * d_in * 4));
  if (with_gates) {
    w.dgpart = static_cast<float*>(ar.take(size_t(dg_slots(M, E, d_in, bf16)) * M * 4));
    w.gg = static_cast<float*>(ar.take(size_t(M) * 4));
  }
  w.partial = static_cast<float*>(ar.take(dw_partial_bytes(M, E, d_in, d_out, bf16)));
}

struct SavedLayout {
  size_t off[6];
  size_t total;
};
SavedLayout saved_layout(int64_t T, int k, int E, int64_t d_ff, int act, int dtype) {
  const int64_t M = T * k;
  Arena ar(nullptr);
  SavedLayout s;
  auto at = [&](size_t bytes) {
    ar.take(bytes);
    return ar.used - std::max<size_t>(bytes, 1);
  };
  s.off[0] = at(size_t(M) * 4);
  s.off[1] = at(size_t(M) * 4);
  s.off[2] = at(size_t(E) * 4);
  s.off[3] = at(size_t(E + 1) * 4);
  s.off[4] = at(size_t(M) * d_ff * esize(dtype));
  s.off[5] = act == SMOE_ACT_SWIGLU ? at(size_t(M) * d_ff * esize(dtype)) : SIZE_MAX;
  s.total = ar.used;
  return s;
}

struct MlpFwdWs {
  void* route = nullptr;
  void* a = nullptr;         // activation, grouped [M, d_ff]
  float* pairs = nullptr;    // expert outputs, scattered fp32 [M, d_model]
                             // (fused combine: the fp32 token sums [T, d_model])
};
void layout_mlp_fwd(Arena& ar, int64_t T, int k, int E, int64_t d_model, int64_t d_ff, int dtype, MlpFwdWs& w,
                    bool fused = false) {
  const int64_t M = T * k;
  w.route = ar.take(route_ws_bytes(M, E));
  w.a = ar.take(size_t(M) * d_ff * esize(dtype));
  w.pairs = static_cast<float*>(ar.take(size_t(fused ? T : M) * d_model * 4));
}

struct MlpBwdWs {
  float* dgpart = nullptr;
  void* dh1 = nullptr;
  void* dh3 = nullptr;
  void* ag = nullptr;        // gate-scaled activation g*a, grouped [M, d_ff]
  float* pairs = nullptr;
  float* partial = nullptr;
  float* partial2 = nullptr;
};
void layout_mlp_bwd(Arena& ar, int64_t T, int k, int E, int64_t d_model, int64_t d_ff, int act, int dtype,
                    MlpBwdWs& w) {
  const int64_t M = T * k;
  const int bf16 = dtype == SMOE_BF16;
  w.dgpart = static_cast<float*>(ar.take(size_t(dg_slots(M, E, d_ff, bf16)) * M * 4));
  w.dh1 = ar.take(size_t(M) * d_ff * esize(dtype));
  if (act == SMOE_ACT_SWIGLU) w.dh3 = ar.take(size_t(M) * d_ff * esize(dtype));
  w.ag = ar.take(size_t(M) * d_ff * esize(dtype));
  w.pairs = static_cast<float*>(ar.take(size_t(M) * d_model * 4));
  const size_t p1 = dw_partial_bytes(M, E, d_ff, d_model, bf16);
  const size_t p2 = dw_partial_bytes(M, E, d_model, d_ff, bf16);
  w.partial = static_cast<float*>(ar.take(std::max(p1, p2)));
  w.partial2 = static_cast<float*>(ar.take(p2));   // dW1 on the second stream
}

// Weight gradient dw[e] = sum over e's rows of A(r)^T B(r): GEMM + reduction.
// An fp32 dw that is written (not accumulated) takes the single-chunk
// experts straight from the product; a bf16 or accumulated dw takes every
// chunk through the partials, and the reduction rounds or adds once.
int run_dw(GemmArgs a, int bf16, void* dw, int dw_bf16, int accumulate, float* partial, hipStream_t st, int role,
           const char* where) {
  a.c0 = dw;
  a.partial = partial;
  a.dw_all_partial = (dw_bf16 || accumulate) ? 1 : 0;
  GemmPlan pl;
  plan_gemm(a, pl, SEG_K, a.kscale ? EPI_PARTIAL_GATED : EPI_PARTIAL, 0, bf16, 1);
  {
    RoleTimer t(role, st);
    SMOE_HIP(launch_gemm(a, pl, st), where);
  }
  RoleTimer t(SMOE_ROLE_DW_REDUCE, st);
  SMOE_HIP(launch_reduce_dw(partial, a.offsets, a.E, a.KS, int64_t(a.Mo) * a.N, dw, a.dw_all_partial, accumulate,
                            dw_bf16, st),
           where);
  return SMOE_OK;
}

// Router backward scratch: the dense dlogits D for the dw product, its
// single-group offsets and identity row index, the product's [d][ncol]
// result and its split-K partials.
struct RouterBwdWs {
  void* D = nullptr;
  int* offsets = nullptr;
  int* rows = nullptr;
  float* tmp = nullptr;
  float* partial = nullptr;
};
void layout_router_bwd(Arena& ar, int64_t T, int64_t d, int E, int bf16, RouterBwdWs& w) {
  int ep, ncol;
  gate_dlogit_cols(E, bf16, ep, ncol);
  w.D = ar.take(size_t(T) * ncol * (bf16 ? 2 : 4));
  w.offsets = static_cast<int*>(ar.take(2 * sizeof(int)));
  w.rows = static_cast<int*>(ar.take(size_t(T) * sizeof(int)));
  w.tmp = static_cast<float*>(ar.take(size_t(d) * ncol * 4));
  w.partial = static_cast<float*>(ar.take(dw_partial_bytes(T, 1, d, ncol, bf16)));
}

}  // namespace

extern "C" {

const char* smoe_status_string(int status) {
  switch (status) {
    case SMOE_OK: return "ok";
    case SMOE_ERR_NULL: return "a required pointer is NULL";
    case SMOE_ERR_SHAPE: return "sizes out of range, inconsistent or misaligned";
    case SMOE_ERR_DTYPE: return "unknown dtype or activation";
    case SMOE_ERR_WORKSPACE: return "workspace or saved buffer too small";
    case SMOE_ERR_UNSUPPORTED: return "request not supported by this build";
    case SMOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* smoe_last_error(void) { return g_last_error.c_str(); }

int smoe_abi_version(void) { return 2; }

static int check_router(int64_t T, int64_t d_model, int32_t E, int32_t k, int32_t dtype) {
  if (dtype != SMOE_F32 && dtype != SMOE_BF16) return fail(SMOE_ERR_DTYPE, "dtype %d is not SMOE_F32/SMOE_BF16", dtype);
  if (T < 0 || T > INT32_MAX / 2) return fail(SMOE_ERR_SHAPE, "T=%lld out of range", (long long)T);
  SMOE_TRY(check_dim(d_model, "d_model"));
  if (E < 1 || E > 64) return fail(SMOE_ERR_UNSUPPORTED, "router: E=%d outside [1, 64]", E);
  if (k < 1 || k > E || k > 8) return fail(SMOE_ERR_UNSUPPORTED, "router: k=%d outside [1, min(E, 8)]", k);
  return SMOE_OK;
}

int smoe_router_fwd(const void* x, const void* w, int64_t T, int64_t d_model, int32_t E, int32_t k, int32_t dtype,
                    int32_t* expert_idxs, float* gates, float* logits, void* stream) {
  SMOE_TRY(check_router(T, d_model, E, k, dtype));
  SMOE_TRY(need_ptr(w, "w"));
  if (T > 0) {
    SMOE_TRY(need_ptr(x, "x"));
    SMOE_TRY(need_ptr(expert_idxs, "expert_idxs"));
    SMOE_TRY(need_ptr(gates, "gates"));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  RoleTimer t(SMOE_ROLE_ROUTER_FWD, st);
  SMOE_HIP(launch_gate_fwd(x, w, T, int(d_model), E, k, dtype == SMOE_BF16, expert_idxs, gates, logits, st),
           "router_fwd");
  return ok();
}

size_t smoe_router_bwd_workspace_bytes(int64_t T, int64_t d_model, int32_t E) {
  if (T < 0 || T > INT32_MAX / 2 || d_model < 1 || d_model > (int64_t(1) << 24) || E < 1 || E > 64) return 0;
  Arena ar(nullptr);
  RouterBwdWs w;
  layout_router_bwd(ar, T, d_model, E, 1, w);
  const size_t b = ar.used;
  Arena af(nullptr);
  layout_router_bwd(af, T, d_model, E, 0, w);
  return std::max(b, af.used);
}

int smoe_router_bwd(const void* x, const void* w, int64_t T, int64_t d_model, int32_t E, int32_t k, int32_t dtype,
                    const int32_t* expert_idxs, const float* gates, const float* dgates, float* dw_out, void* dx,
                    int32_t accumulate_dx, void* ws, size_t ws_bytes, void* stream) {
  SMOE_TRY(check_router(T, d_model, E, k, dtype));
  SMOE_TRY(check_extent(dtype, T, d_model, "x"));
  SMOE_TRY(need_ptr(w, "w"));
  SMOE_TRY(need_ptr(dw_out, "dw_out"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {
    SMOE_HIP(launch_zero(dw_out, size_t(d_model) * E * 4, st), "router_bwd");
    return ok();
  }
  SMOE_TRY(need_ptr(x, "x"));
  SMOE_TRY(need_ptr(expert_idxs, "expert_idxs"));
  SMOE_TRY(need_ptr(gates, "gates"));
  SMOE_TRY(need_ptr(dgates, "dgates"));
  SMOE_TRY(need_ptr(dx, "dx"));
  SMOE_TRY(need_ptr(ws, "ws"));
  const size_t need = smoe_router_bwd_workspace_bytes(T, d_model, E);
  if (ws_bytes < need) return fail(SMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, need);
  const int bf16 = dtype == SMOE_BF16;
  Arena ar(ws);
  RouterBwdWs wl;
  layout_router_bwd(ar, T, d_model, E, bf16, wl);
  {
    RoleTimer t(SMOE_ROLE_ROUTER_DX, st);
    SMOE_HIP(launch_gate_dx(w, T, int(d_model), E, k, bf16, expert_idxs, gates, dgates, dx, accumulate_dx, wl.D,
                            wl.rows, wl.offsets, st),
             "router_bwd dx");
  }
  // dw^T [d][ncol] = x^T D as a weight-gradient product over one group of T
  // rows, then dw[e][c] from its columns
  int ep, ncol;
  gate_dlogit_cols(E, bf16, ep, ncol);
  GemmArgs a = blank_args(wl.offsets, wl.rows, 1, int(T));
  a.Mo = int(d_model);
  a.N = ncol;
  a.a0 = x;
  a.lda = d_model;
  a.a_rows = T;
  a.b0 = wl.D;
  a.ldb = ncol;
  a.b_rows = T;
  SMOE_TRY(run_dw(a, bf16, wl.tmp, 0, 0, wl.partial, st, SMOE_ROLE_ROUTER_DW, "router_bwd dw"));
  SMOE_HIP(launch_gate_dw_finish(wl.tmp, int(d_model), E, bf16, dw_out, st), "router_bwd dw");
  return ok();
}

// ------------------------------------------------------- MoA attention --
static int check_attn(int64_t T, int32_t k, int64_t seq_len, int64_t head_dim, int32_t dtype) {
  if (dtype != SMOE_F32 && dtype != SMOE_BF16) return fail(SMOE_ERR_DTYPE, "dtype %d is not SMOE_F32/SMOE_BF16", dtype);
  if (dtype != SMOE_BF16) return fail(SMOE_ERR_UNSUPPORTED, "attention: bf16 only");
  if (head_dim != 128) return fail(SMOE_ERR_UNSUPPORTED, "attention: head_dim=%lld (128 supported)", (long long)head_dim);
  if (k < 1 || k > 1024) return fail(SMOE_ERR_SHAPE, "k=%d out of range", k);
  if (T < 0 || seq_len < 1 || T % seq_len != 0)
    return fail(SMOE_ERR_SHAPE, "T=%lld must be a multiple of seq_len=%lld", (long long)T, (long long)seq_len);
  if (T * k > INT32_MAX / 2) return fail(SMOE_ERR_SHAPE, "T*k=%lld too large", (long long)(T * k));
  return SMOE_OK;
}

int smoe_moa_attention_fwd(const void* q, const void* k_, const void* v, const int32_t* sorted_scattered_idxs,
                           int64_t T, int32_t k, int64_t seq_len, int64_t head_dim, int32_t dtype, void* o, float* lse,
                           void* stream) {
  SMOE_TRY(check_attn(T, k, seq_len, head_dim, dtype));
  if (T == 0) return ok();
  SMOE_TRY(need_ptr(q, "q"));
  SMOE_TRY(need_ptr(k_, "k"));
  SMOE_TRY(need_ptr(v, "v"));
  SMOE_TRY(need_ptr(sorted_scattered_idxs, "sorted_scattered_idxs"));
  SMOE_TRY(need_ptr(o, "o"));
  SMOE_TRY(need_ptr(lse, "lse"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  RoleTimer t(SMOE_ROLE_ATTN_FWD, st);
  SMOE_HIP(launch_attn_fwd(q, k_, v, sorted_scattered_idxs, T * k, T, k, seq_len, o, lse, st), "moa_attention_fwd");
  return ok();
}

struct AttnBwdWs {
  float* D = nullptr;
  int* tile_lo = nullptr;
  int* tile_hi = nullptr;
  float* pdk = nullptr;
  float* pdv = nullptr;
};
static void layout_attn_bwd(Arena& ar, int64_t T, int64_t M, AttnBwdWs& w) {
  const int64_t ntiles = (M + 31) / 32;
  const size_t part = size_t(attn_query_splits(T)) * size_t(T) * 128 * 4;
  w.D = static_cast<float*>(ar.take(size_t(M) * 4));
  w.tile_lo = static_cast<int*>(ar.take(size_t(ntiles) * 8));   // two values per tile
  w.tile_hi = static_cast<int*>(ar.take(size_t(ntiles) * 8));
  w.pdk = static_cast<float*>(ar.take(part));
  w.pdv = static_cast<float*>(ar.take(part));
}

size_t smoe_moa_attention_bwd_workspace_bytes(int64_t T, int32_t k, int64_t seq_len, int64_t head_dim) {
  if (T < 0 || k < 1 || seq_len < 1 || head_dim != 128 || T * k > INT32_MAX / 2) return 0;
  Arena ar(nullptr);
  AttnBwdWs w;
  layout_attn_bwd(ar, T, T * k, w);
  return ar.used;
}

int smoe_moa_attention_bwd(const void* q, const void* k_, const void* v, const int32_t* sorted_scattered_idxs,
                           int64_t T, int32_t k, int64_t seq_len, int64_t head_dim, int32_t dtype, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           size_t ws_bytes, void* stream) {
  SMOE_TRY(check_attn(T, k, seq_len, head_dim, dtype));
  if (T == 0) return ok();
  SMOE_TRY(need_ptr(q, "q"));
  SMOE_TRY(need_ptr(k_, "k"));
  SMOE_TRY(need_ptr(v, "v"));
  SMOE_TRY(need_ptr(sorted_scattered_idxs, "sorted_scattered_idxs"));
  SMOE_TRY(need_ptr(o, "o"));
  SMOE_TRY(need_ptr(lse, "lse"));
  SMOE_TRY(need_ptr(dout, "dout"));
  SMOE_TRY(need_ptr(dq, "dq"));
  SMOE_TRY(need_ptr(dk, "dk"));
  SMOE_TRY(need_ptr(dv, "dv"));
  SMOE_TRY(need_ptr(ws, "ws"));
  const size_t need = smoe_moa_attention_bwd_workspace_bytes(T, k, seq_len, head_dim);
  if (ws_bytes < need) return fail(SMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  Arena ar(ws);
  AttnBwdWs wl;
  layout_attn_bwd(ar, T, T * k, wl);
  SMOE_HIP(launch_attn_bwd(q, k_, v, sorted_scattered_idxs, T * k, T, k, seq_len, o, lse, dout, dq, dk, dv, wl.D,
                           wl.tile_lo, wl.tile_hi, wl.pdk, wl.pdv, st, g_role_ev[SMOE_ROLE_ATTN_DQ][0],
                           g_role_ev[SMOE_ROLE_ATTN_DQ][1], g_role_ev[SMOE_ROLE_ATTN_DKV][0],
                           g_role_ev[SMOE_ROLE_ATTN_DKV][1]),
           "moa_attention_bwd");
  return ok();
}

int smoe_probe_mfma_loop(float* out, int32_t blocks, int32_t iters, void* stream) {
  SMOE_TRY(need_ptr(out, "out"));
  if (blocks < 1 || iters < 1) return fail(SMOE_ERR_SHAPE, "blocks=%d and iters=%d must be positive", blocks, iters);
  SMOE_HIP(launch_mfma_loop(out, blocks, iters, static_cast<hipStream_t>(stream)), "probe_mfma_loop");
  return ok();
}

int smoe_set_role_events(int32_t role, void* start_event, void* stop_event) {
  if (role < 0 || role >= SMOE_ROLE_COUNT) return fail(SMOE_ERR_SHAPE, "role %d outside [0, %d)", role, SMOE_ROLE_COUNT);
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(SMOE_ERR_NULL, "attach both events or neither");
  g_role_ev[role][0] = static_cast<hipEvent_t>(start_event);
  g_role_ev[role][1] = static_cast<hipEvent_t>(stop_event);
  return ok();
}

// ---------------------------------------------------------------- route --
size_t smoe_route_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return route_ws_bytes(T * k, E);
}

int smoe_route(const int32_t* expert_idxs, int64_t T, int32_t k, int32_t E, int32_t* sorted_expert_idxs,
               int32_t* sorted_scattered_idxs, int32_t* counts, int32_t* offsets, void* ws, size_t ws_bytes,
               void* stream) {
  SMOE_TRY(check_common(T, k, E, SMOE_F32));
  const int64_t M = T * k;
  if (M > 0 && (!expert_idxs || !sorted_expert_idxs || !sorted_scattered_idxs))
    return fail(SMOE_ERR_NULL, "routing arrays must not be NULL");
  if (!counts || !offsets || !ws) return fail(SMOE_ERR_NULL, "counts/offsets/ws must not be NULL");
  if (ws_bytes < route_ws_bytes(M, E))
    return fail(SMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, route_ws_bytes(M, E));
  SMOE_HIP(launch_route(expert_idxs, int(M), E, sorted_expert_idxs, sorted_scattered_idxs, counts, offsets, ws,
                        static_cast<hipStream_t>(stream)),
           "smoe_route");
  return ok();
}

int smoe_route_noalloc(const int32_t* expert_idxs, int64_t T, int32_t k, int32_t E, int32_t* sorted_expert_idxs,
                       int32_t* sorted_scattered_idxs, int32_t* counts, int32_t* offsets, void* stream) {
  SMOE_TRY(check_common(T, k, E, SMOE_F32));
  const int64_t M = T * k;
  if (M > 0 && (!expert_idxs || !sorted_expert_idxs || !sorted_scattered_idxs))
    return fail(SMOE_ERR_NULL, "routing arrays must not be NULL");
  if (!counts || !offsets) return fail(SMOE_ERR_NULL, "counts/offsets must not be NULL");
  const size_t need = route_ws_bytes(M, E) / sizeof(int);
  if (need > route_static_scratch_ints())
    return fail(SMOE_ERR_SHAPE, "T*k=%lld with E=%d needs %zu ints of scratch, beyond the static %zu "
                "(ceil(T*k/4096)*E must not exceed it)", (long long)M, E, need, route_static_scratch_ints());
  int* scr = nullptr;
  size_t cap = 0;
  SMOE_HIP(route_static_scratch(&scr, &cap), "smoe_route_noalloc scratch");
  SMOE_HIP(launch_route(expert_idxs, int(M), E, sorted_expert_idxs, sorted_scattered_idxs, counts, offsets, scr,
                        static_cast<hipStream_t>(stream)),
           "smoe_route_noalloc");
  return ok();
}

// ------------------------------------------------------ parallel linear --
size_t smoe_parallel_linear_fwd_workspace_bytes(int64_t T, int32_t k, int32_t E, int64_t d_in, int64_t d_out,
                                                int32_t with_gates, int32_t dtype) {
  (void)E; (void)d_in; (void)dtype;
  Arena ar(nullptr);
  PlFwdWs w;
  layout_pl_fwd(ar, T * k, d_out, with_gates != 0, w);
  return ar.used;
}

int smoe_parallel_linear_fwd(const void* x, int64_t x_rows, int64_t d_in, const void* w, int64_t d_out, int32_t E,
                             int64_t T, int32_t k, const int32_t* sorted_scattered_idxs, const int32_t* offsets,
                             int32_t x_grouped, int32_t y_grouped, const float* gates, void* y, int32_t dtype,
                             void* ws, size_t ws_bytes, void* stream) {
  SMOE_TRY(check_common(T, k, E, dtype));
  SMOE_TRY(check_dim(d_in, "d_in"));
  SMOE_TRY(check_dim(d_out, "d_out"));
  const int64_t M = T * k;
  if (x_grouped ? x_rows != M : (x_rows != T && x_rows != M))
    return fail(SMOE_ERR_SHAPE, "x_rows=%lld does not fit the layout (T=%lld, T*k=%lld)", (long long)x_rows,
                (long long)T, (long long)M);
  SMOE_TRY(check_extent(dtype, M, d_in, "x"));
  SMOE_TRY(check_extent(dtype, d_in, d_out, "w[e]"));
  if (gates && y_grouped) return fail(SMOE_ERR_SHAPE, "the gate-weighted combine needs a scattered output");
  SMOE_TRY(need_ptr(w, "w"));
  SMOE_TRY(need_ptr(offsets, "offsets"));
  if (M > 0) {
    SMOE_TRY(need_ptr(x, "x"));
    SMOE_TRY(need_ptr(y, "y"));
    SMOE_TRY(need_ptr(sorted_scattered_idxs, "sorted_scattered_idxs"));
  }
  Arena ar(ws);
  PlFwdWs wl;
  layout_pl_fwd(ar, M, d_out, gates != nullptr, wl);
  if (gates && (!ws || ws_bytes < ar.used))
    return fail(SMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, ar.used);
  if (M == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int bf16 = dtype == SMOE_BF16;
  GemmArgs a = blank_args(offsets, sorted_scattered_idxs, E, int(M));
  a.N = int(d_out);
  a.K = a.K0 = int(d_in);
  a.a0 = a.a1 = x;
  a.a_rows = x_rows;
  a.lda = d_in;
  a.a_scat = !x_grouped;
  a.a_fan = (!x_grouped && x_rows == T) ? k : 1;
  a.b0 = a.b1 = w;
  a.b_nk = 0;
  a.ldb = d_out;
  a.b_es = d_in * d_out;
  a.ldc = d_out;
  GemmPlan pl;
  if (gates) {
    a.c0 = wl.pairs;
    a.c_scat = 1;
    plan_gemm(a, pl, SEG_M, EPI_STORE, 0, bf16, 1);
    {
      RoleTimer t(SMOE_ROLE_PL_FWD, st);
      SMOE_HIP(launch_gemm(a, pl, st), "parallel_linear_fwd gemm");
    }
    RoleTimer t(SMOE_ROLE_COMBINE, st);
    SMOE_HIP(launch_combine(wl.pairs, gates, T, k, d_out, y, bf16, st), "parallel_linear_fwd combine");
  } else {
    a.c0 = y;
    a.c_scat = !y_grouped;
    plan_gemm(a, pl, SEG_M, EPI_STORE, 0, bf16, !bf16);
    RoleTimer t(SMOE_ROLE_PL_FWD, st);
    SMOE_HIP(launch_gemm(a, pl, st), "parallel_linear_fwd gemm");
  }
  return ok();
}

size_t smoe_parallel_linear_bwd_workspace_bytes(int64_t T, int32_t k, int32_t E, int64_t x_rows, int64_t d_in,
                                                int64_t d_out, int32_t x_grouped, int32_t with_gates,
                                                int32_t dtype) {
  Arena ar(nullptr);
  PlBwdWs w;
  layout_pl_bwd(ar, T, k, E, x_rows, d_in, d_out, x_grouped != 0, with_gates != 0, dtype == SMOE_BF16, w);
  return ar.used;
}

int smoe_parallel_linear_bwd(const void* x, int64_t x_rows, int64_t d_in, const void* w, int64_t d_out, int32_t E,
                             int64_t T, int32_t k, const int32_t* sorted_scattered_idxs, const int32_t* offsets,
                             int32_t x_grouped, int32_t y_grouped, const float* gates, const void* dy, void* dx,
                             int32_t dx_dtype, void* dw, int32_t dw_dtype, int32_t accumulate_dw, float* dgates,
                             int32_t dtype, void* ws, size_t ws_bytes, void* stream) {
  SMOE_TRY(check_common(T, k, E, dtype));
  SMOE_TRY(check_dim(d_in, "d_in"));
  SMOE_TRY(check_dim(d_out, "d_out"));
  if (dx_dtype != SMOE_F32 && dx_dtype != SMOE_BF16) return fail(SMOE_ERR_DTYPE, "dx_dtype %d", dx_dtype);
  if (dw_dtype != SMOE_F32 && dw_dtype != SMOE_BF16) return fail(SMOE_ERR_DTYPE, "dw_dtype %d", dw_dtype);
  if (dtype == SMOE_F32 && (dx_dtype != SMOE_F32 || dw_dtype != SMOE_F32))
    return fail(SMOE_ERR_DTYPE, "fp32 runs give fp32 dx and dw");
  const int64_t M = T * k;
  if (x_grouped ? x_rows != M : (x_rows != T && x_rows != M))
    return fail(SMOE_ERR_SHAPE, "x_rows=%lld does not fit the layout", (long long)x_rows);
  SMOE_TRY(check_extent(dtype, M, d_in, "x"));
  SMOE_TRY(check_extent(dtype, M, d_out, "dy"));
  SMOE_TRY(check_extent(dtype, d_in, d_out, "w[e]"));
  if (gates && y_grouped) return fail(SMOE_ERR_SHAPE, "the gate-weighted combine needs a scattered output");
  if (dgates && !gates) return fail(SMOE_ERR_NULL, "dgates needs gates");
  SMOE_TRY(need_ptr(w, "w"));
  SMOE_TRY(need_ptr(offsets, "offsets"));
  if (dx) SMOE_TRY(need_ptr(dx, "dx"));
  if (dw) SMOE_TRY(need_ptr(dw, "dw"));
  if (M > 0) {
    SMOE_TRY(need_ptr(x, "x"));
    SMOE_TRY(need_ptr(dy, "dy"));
    SMOE_TRY(need_ptr(sorted_scattered_idxs, "sorted_scattered_idxs"));
  }
  Arena ar(ws);
  PlBwdWs wl;
  const int bf16 = dtype == SMOE_BF16;
  layout_pl_bwd(ar, T, k, E, x_rows, d_in, d_out, x_grouped != 0, gates != nullptr, bf16, wl);
  if (!ws || ws_bytes < ar.used) return fail(SMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, ar.used);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int fan = (!x_grouped && x_rows == T) ? k : 1;
  const bool fan_k = fan > 1;
  const int dx_f32 = dx_dtype == SMOE_F32;

  if (M == 0) {
    if (dw && !accumulate_dw)
      SMOE_HIP(launch_zero(dw, size_t(E) * d_in * d_out * (dw_dtype == SMOE_BF16 ? 2 : 4), st), "parallel_linear_bwd");
    return ok();
  }
  // dx (and the gate gradient): dy rows against W^T
  if (dx || dgates) {
    GemmArgs a = blank_args(offsets, sorted_scattered_idxs, E, int(M));
    a.N = int(d_in);
    a.K = a.K0 = int(d_out);
    a.a0 = a.a1 = dy;
    a.a_rows = gates ? T : M;
    a.lda = d_out;
    a.a_scat = gates ? 1 : !y_grouped;
    a.a_fan = gates ? k : 1;
    a.b0 = a.b1 = w;
    a.b_nk = 1;
    a.ldb = d_out;
    a.b_es = d_in * d_out;
    a.gate = gates;
    a.ldc = d_in;
    if (dgates) {
      a.dgpart = wl.dgpart;
      a.aux0 = x;
      a.ldaux = d_in;
      a.aux_scat = !x_grouped;
      a.aux_fan = fan;
    }
    GemmPlan pl;
    if (fan_k) {
      a.c0 = dx ? wl.pairs : nullptr;
      a.c_scat = 1;
      plan_gemm(a, pl, SEG_M, EPI_STORE, 0, bf16, 1);
    } else {
      a.c0 = dx;
      a.c_scat = !x_grouped;
      plan_gemm(a, pl, SEG_M, EPI_STORE, 0, bf16, dx_f32);
    }
    {
      RoleTimer t(SMOE_ROLE_PL_DX, st);
      SMOE_HIP(launch_gemm(a, pl, st), "parallel_linear_bwd dx gemm");
    }
    if (fan_k && dx)
      SMOE_HIP(launch_combine(wl.pairs, nullptr, T, k, d_in, dx, !dx_f32, st), "parallel_linear_bwd ksum");
    if (dgates)
      SMOE_HIP(launch_reduce_dg(wl.dgpart, pl.slots, int(M), offsets, E, sorted_scattered_idxs, dgates, st),
               "parallel_linear_bwd dgates");
  }
  if (dw) {
    // dw[e] = sum (g u)^T dy[t]: with gates the product scales each row of
    // its A operand (u, read in place) by the row's gate in registers
    GemmArgs a = blank_args(offsets, sorted_scattered_idxs, E, int(M));
    a.Mo = int(d_in);
    a.N = int(d_out);
    if (gates) {
      SMOE_HIP(launch_grouped_gates(gates, sorted_scattered_idxs, offsets, E, int(M), wl.gg, st),
               "parallel_linear_bwd gates");
      a.kscale = wl.gg;
    }
    a.a0 = x;
    a.a_rows = x_rows;
    a.a_scat = !x_grouped;
    a.a_fan = fan;
    a.lda = d_in;
    a.b0 = dy;
    a.ldb = d_out;
    a.b_rows = gates ? T : M;
    a.b_scat = gates ? 1 : !y_grouped;
    a.b_fan = gates ? k : 1;
    SMOE_TRY(run_dw(a, bf16, dw, dw_dtype == SMOE_BF16, accumulate_dw != 0, wl.partial, st, SMOE_ROLE_PL_DW,
                    "parallel_linear_bwd dw"));
  }
  return ok();
}

// -------------------------------------------------------------- SMoE MLP --
static int check_mlp(int64_t T, int32_t k, int32_t E, int64_t d_model, int64_t d_ff, int32_t act, int32_t dtype,
                     const void* w3) {
  SMOE_TRY(check_common(T, k, E, dtype));
  SMOE_TRY(check_dim(d_model, "d_model"));
  SMOE_TRY(check_dim(d_ff, "d_ff"));
  SMOE_TRY(check_extent(dtype, T * k, d_model, "token rows"));
  SMOE_TRY(check_extent(dtype, T * k, d_ff, "hidden rows"));
  SMOE_TRY(check_extent(dtype, d_model, d_ff, "w[e]"));
  if (act != SMOE_ACT_GELU && act != SMOE_ACT_SWIGLU) return fail(SMOE_ERR_DTYPE, "unknown activation %d", act);
  if ((act == SMOE_ACT_SWIGLU) != (w3 != nullptr)) return fail(SMOE_ERR_NULL, "w3 must be given exactly for SWIGLU");
  return SMOE_OK;
}

size_t smoe_mlp_saved_bytes(int64_t T, int32_t k, int32_t E, int64_t d_model, int64_t d_ff, int32_t act,
                            int32_t dtype) {
  (void)d_model;
  return saved_layout(T, k, E, d_ff, act, dtype).total;
}

int smoe_mlp_saved_offsets(int64_t T, int32_t k, int32_t E, int64_t d_model, int64_t d_ff, int32_t act,
                           int32_t dtype, size_t off[6]) {
  (void)d_model;
  if (!off) return fail(SMOE_ERR_NULL, "off is NULL");
  SavedLayout s = saved_layout(T, k, E, d_ff, act, dtype);
  for (int i = 0; i < 6; ++i) off[i] = s.off[i];
  return ok();
}

size_t smoe_mlp_fwd_workspace_bytes(int64_t T, int32_t k, int32_t E, int64_t d_model, int64_t d_ff, int32_t act,
                                    int32_t dtype) {
  (void)act;
  Arena ar(nullptr);
  MlpFwdWs w;
  layout_mlp_fwd(ar, T, k, E, d_model, d_ff, dtype, w);
  return ar.used;
}

// fused: the down product adds its gated rows straight into an fp32 [T, d]
// token buffer (fp32 atomics) in place of the per-assignment rows and the
// separate combine; the buffer is the front of the per-assignment region.
static int mlp_fwd(const void* x, const void* w1, const void* w3, const void* w2, int64_t T, int64_t d_model,
                   int64_t d_ff, int32_t E, int32_t k, const int32_t* expert_idxs, const float* gates, int32_t act,
                   int32_t dtype, void* out, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                   const smoe_aux* aux, void* stream, bool fused) {
  SMOE_TRY(check_mlp(T, k, E, d_model, d_ff, act, dtype, w3));
  SMOE_TRY(need_ptr(w1, "w1"));
  SMOE_TRY(need_ptr(w2, "w2"));
  if (w3) SMOE_TRY(need_ptr(w3, "w3"));
  SMOE_TRY(need_ptr(saved, "saved"));
  SMOE_TRY(need_ptr(ws, "ws"));
  const int64_t M = T * k;
  if (M > 0) {
    SMOE_TRY(need_ptr(x, "x"));
    SMOE_TRY(need_ptr(out, "out"));
    SMOE_TRY(need_ptr(expert_idxs, "expert_idxs"));
    SMOE_TRY(need_ptr(gates, "gates"));
  }
  const SavedLayout sl = saved_layout(T, k, E, d_ff, act, dtype);
  if (saved_bytes < sl.total) return fail(SMOE_ERR_WORKSPACE, "saved_bytes=%zu < %zu", saved_bytes, sl.total);
  Arena ar(ws);
  MlpFwdWs wl;
  layout_mlp_fwd(ar, T, k, E, d_model, d_ff, dtype, wl, fused);
  if (ws_bytes < ar.used) return fail(SMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, ar.used);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* sv = static_cast<char*>(saved);
  int* s_exp = reinterpret_cast<int*>(sv + sl.off[0]);
  int* s_sct = reinterpret_cast<int*>(sv + sl.off[1]);
  int* counts = reinterpret_cast<int*>(sv + sl.off[2]);
  int* offsets = reinterpret_cast<int*>(sv + sl.off[3]);
  void* h1 = sv + sl.off[4];
  void* h3 = act == SMOE_ACT_SWIGLU ? sv + sl.off[5] : nullptr;
  void* av = wl.a;
  const int bf16 = dtype == SMOE_BF16;

  {
    RoleTimer t(SMOE_ROLE_ROUTE, st);
    SMOE_HIP(launch_route(expert_idxs, int(M), E, s_exp, s_sct, counts, offsets, wl.route, st), "mlp_fwd route");
  }
  if (M == 0) return ok();

  // layer 1: scattered x rows (fan-out k) -> grouped h (h1, h3) and a
  GemmArgs a = blank_args(offsets, s_sct, E, int(M));
  a.N = int(d_ff);
  a.K = a.K0 = int(d_model);
  a.a0 = a.a1 = x;
  a.a_rows = T;
  a.lda = d_model;
  a.a_scat = 1;
  a.a_fan = k;
  a.b0 = w1;
  a.b1 = act == SMOE_ACT_SWIGLU ? w3 : w1;
  a.b_nk = 0;
  a.ldb = d_ff;
  a.b_es = d_model * d_ff;
  a.c0 = h1;
  a.c1 = act == SMOE_ACT_SWIGLU ? h3 : av;
  a.c2 = av;
  a.ldc = d_ff;
  GemmPlan pl;
  if (act == SMOE_ACT_SWIGLU)
    plan_gemm(a, pl, SEG_M, EPI_SWIGLU_FWD, 1, bf16, 0);
  else
    plan_gemm(a, pl, SEG_M, EPI_GELU_FWD, 0, bf16, 0);

  // layer 2: grouped a -> scattered fp32 expert outputs
  GemmArgs b = blank_args(offsets, s_sct, E, int(M));
  b.N = int(d_model);
  b.K = b.K0 = int(d_ff);
  b.a0 = b.a1 = av;
  b.a_rows = M;
  b.lda = d_ff;
  b.b0 = b.b1 = w2;
  b.ldb = d_model;
  b.b_es = d_ff * d_model;
  b.c0 = wl.pairs;
  b.c_scat = 1;
  b.ldc = d_model;
  if (fused) {
    b.gate = gates;
    b.c_add_fan = k;
  }
  GemmPlan pb;
  plan_gemm(b, pb, SEG_M, EPI_STORE, 0, bf16, 1);
  if (fused) {
    RoleTimer t(SMOE_ROLE_COMBINE, st);
    SMOE_HIP(launch_zero(wl.pairs, size_t(T) * size_t(d_model) * sizeof(float), st), "mlp_fwd zero");
  }

  // With the caller's second stream: the m-tiles that exist whatever the
  // routing (whole groups of 8 below ceil(M / BM)) run both layers on the
  // caller's stream; the remaining, routing-dependent m-tiles run both
  // layers on the second stream beside them, so the last, partly filled
  // round of layer 2 overlaps layer 1's work instead of leaving most CUs
  // idle.  Each layer-2 tile reads only the rows its own m-tile's layer-1
  // tiles wrote, on the same stream.
  Fork fk(aux, st);
  const int64_t mt_head = (ceil_div64(M, pl.bm) / 8) * 8;
  const bool split = fk.usable() && bf16 && pl.bm == pb.bm && mt_head > 0 && mt_head * pb.n_tiles < pb.grid;
  if (split) {
    SMOE_HIP(fk.fork(), "mlp_fwd fork");
    GemmArgs at = a, bt = b;
    GemmPlan plt = pl, pbt = pb;
    at.g_base = int(mt_head * pl.n_tiles);
    bt.g_base = int(mt_head * pb.n_tiles);
    plt.grid = (pl.grid - at.g_base + 7) / 8 * 8;
    pbt.grid = (pb.grid - bt.g_base + 7) / 8 * 8;
    SMOE_HIP(launch_gemm(at, plt, fk.side()), "mlp_fwd layer 1");
    SMOE_HIP(launch_gemm(bt, pbt, fk.side()), "mlp_fwd layer 2");
    a.g_count = int(mt_head * pl.n_tiles);
    b.g_count = int(mt_head * pb.n_tiles);
    pl.grid = a.g_count;
    pb.grid = b.g_count;
  }
  {
    RoleTimer t(SMOE_ROLE_UP, st);
    SMOE_HIP(launch_gemm(a, pl, st), "mlp_fwd layer 1");
  }
  {
    RoleTimer t(SMOE_ROLE_DOWN, st);
    SMOE_HIP(launch_gemm(b, pb, st), "mlp_fwd layer 2");
  }
  SMOE_HIP(fk.join(), "mlp_fwd join");
  RoleTimer t(SMOE_ROLE_COMBINE, st);
  if (fused)
    SMOE_HIP(launch_combine(wl.pairs, nullptr, T, 1, d_model, out, bf16, st), "mlp_fwd convert");
  else
    SMOE_HIP(launch_combine(wl.pairs, gates, T, k, d_model, out, bf16, st), "mlp_fwd combine");
  return ok();
}

int smoe_mlp_fwd(const void* x, const void* w1, const void* w3, const void* w2, int64_t T, int64_t d_model,
                 int64_t d_ff, int32_t E, int32_t k, const int32_t* expert_idxs, const float* gates, int32_t act,
                 int32_t dtype, void* out, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                 const smoe_aux* aux, void* stream) {
  return mlp_fwd(x, w1, w3, w2, T, d_model, d_ff, E, k, expert_idxs, gates, act, dtype, out, saved, saved_bytes, ws,
                 ws_bytes, aux, stream, false);
}

size_t smoe_mlp_fwd_fused_combine_workspace_bytes(int64_t T, int32_t k, int32_t E, int64_t d_model, int64_t d_ff,
                                                  int32_t act, int32_t dtype) {
  (void)act;
  Arena ar(nullptr);
  MlpFwdWs w;
  layout_mlp_fwd(ar, T, k, E, d_model, d_ff, dtype, w, true);
  return ar.used;
}

int smoe_mlp_fwd_fused_combine(const void* x, const void* w1, const void* w3, const void* w2, int64_t T,
                               int64_t d_model, int64_t d_ff, int32_t E, int32_t k, const int32_t* expert_idxs,
                               const float* gates, int32_t act, int32_t dtype, void* out, void* saved,
                               size_t saved_bytes, void* ws, size_t ws_bytes, const smoe_aux* aux, void* stream) {
  return mlp_fwd(x, w1, w3, w2, T, d_model, d_ff, E, k, expert_idxs, gates, act, dtype, out, saved, saved_bytes, ws,
                 ws_bytes, aux, stream, true);
}

size_t smoe_mlp_bwd_workspace_bytes(int64_t T, int32_t k, int32_t E, int64_t d_model, int64_t d_ff, int32_t act,
                                    int32_t dtype) {
  Arena ar(nullptr);
  MlpBwdWs w;
  layout_mlp_bwd(ar, T, k, E, d_model, d_ff, act, dtype, w);
  return ar.used;
}

int smoe_mlp_bwd(const void* dout, const void* x, const void* w1, const void* w3, const void* w2, int64_t T,
                 int64_t d_model, int64_t d_ff, int32_t E, int32_t k, const int32_t* expert_idxs, const float* gates,
                 int32_t act, int32_t dtype, const void* saved, size_t saved_bytes, void* dx, void* dw1, void* dw3,
                 void* dw2, int32_t dw_dtype, float* dgates, void* ws, size_t ws_bytes, const smoe_aux* aux,
                 void* stream) {
  SMOE_TRY(check_mlp(T, k, E, d_model, d_ff, act, dtype, w3));
  if (dw_dtype != SMOE_F32 && dw_dtype != SMOE_BF16) return fail(SMOE_ERR_DTYPE, "dw_dtype %d", dw_dtype);
  if (dtype == SMOE_F32 && dw_dtype != SMOE_F32) return fail(SMOE_ERR_DTYPE, "fp32 runs give fp32 weight gradients");
  const int dw_bf16 = dw_dtype == SMOE_BF16;
  if ((act == SMOE_ACT_SWIGLU) != (dw3 != nullptr)) return fail(SMOE_ERR_NULL, "dw3 must be given exactly for SWIGLU");
  SMOE_TRY(need_ptr(w1, "w1"));
  SMOE_TRY(need_ptr(w2, "w2"));
  if (w3) SMOE_TRY(need_ptr(w3, "w3"));
  SMOE_TRY(need_ptr(saved, "saved"));
  SMOE_TRY(need_ptr(ws, "ws"));
  SMOE_TRY(need_ptr(dw1, "dw1"));
  SMOE_TRY(need_ptr(dw2, "dw2"));
  if (dw3) SMOE_TRY(need_ptr(dw3, "dw3"));
  const int64_t M = T * k;
  if (M > 0) {
    SMOE_TRY(need_ptr(dout, "dout"));
    SMOE_TRY(need_ptr(x, "x"));
    SMOE_TRY(need_ptr(dx, "dx"));
    SMOE_TRY(need_ptr(gates, "gates"));
  }
  (void)expert_idxs;  // the routing of the forward pass is read from `saved`
  const SavedLayout sl = saved_layout(T, k, E, d_ff, act, dtype);
  if (saved_bytes < sl.total) return fail(SMOE_ERR_WORKSPACE, "saved_bytes=%zu < %zu", saved_bytes, sl.total);
  Arena ar(ws);
  MlpBwdWs wl;
  layout_mlp_bwd(ar, T, k, E, d_model, d_ff, act, dtype, wl);
  if (ws_bytes < ar.used) return fail(SMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, ar.used);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* sv = static_cast<const char*>(saved);
  const int* s_sct = reinterpret_cast<const int*>(sv + sl.off[1]);
  const int* offsets = reinterpret_cast<const int*>(sv + sl.off[3]);
  const void* h1 = sv + sl.off[4];
  const void* h3 = act == SMOE_ACT_SWIGLU ? sv + sl.off[5] : nullptr;
  const int bf16 = dtype == SMOE_BF16;
  const bool swiglu = act == SMOE_ACT_SWIGLU;

  if (M == 0) {
    const size_t wb = size_t(E) * d_model * d_ff * (dw_bf16 ? 2 : 4);
    SMOE_HIP(launch_zero(dw1, wb, st), "mlp_bwd");
    SMOE_HIP(launch_zero(dw2, wb, st), "mlp_bwd");
    if (dw3) SMOE_HIP(launch_zero(dw3, wb, st), "mlp_bwd");
    return ok();
  }

  // 1. dA = dout W2^T per grouped row, activation backward fused: dh (dh1,
  //    dh3), the gate-scaled activation g*a (recomputed from the saved h) and
  //    the gate-gradient partials <a, dout W2^T>
  GemmArgs a = blank_args(offsets, s_sct, E, int(M));
  a.N = int(d_ff);
  a.K = a.K0 = int(d_model);
  a.a0 = a.a1 = dout;
  a.a_rows = T;
  a.lda = d_model;
  a.a_scat = 1;
  a.a_fan = k;
  a.b0 = a.b1 = w2;
  a.b_nk = 1;
  a.ldb = d_model;
  a.b_es = d_ff * d_model;
  a.gate = gates;
  a.aux0 = h1;
  a.aux1 = h3;
  a.ldaux = d_ff;
  a.dgpart = wl.dgpart;
  a.c0 = wl.dh1;
  a.c1 = wl.dh3;
  a.c2 = wl.ag;
  a.ldc = d_ff;
  GemmPlan pl;
  plan_gemm(a, pl, SEG_M, swiglu ? EPI_SWIGLU_BWD : EPI_GELU_BWD, 0, bf16, 0);
  {
    RoleTimer t(SMOE_ROLE_DA, st);
    SMOE_HIP(launch_gemm(a, pl, st), "mlp_bwd dA");
  }
  if (dgates) {
    RoleTimer t(SMOE_ROLE_DG_REDUCE, st);
    SMOE_HIP(launch_reduce_dg(wl.dgpart, pl.slots, int(M), offsets, E, s_sct, dgates, st), "mlp_bwd dgates");
  }

  // dW2[e] = sum (g a)^T dout
  GemmArgs dw2a = blank_args(offsets, s_sct, E, int(M));
  dw2a.Mo = int(d_ff);
  dw2a.N = int(d_model);
  dw2a.a0 = wl.ag;
  dw2a.a_rows = M;
  dw2a.lda = d_ff;
  dw2a.b0 = dout;
  dw2a.b_rows = T;
  dw2a.ldb = d_model;
  dw2a.b_scat = 1;
  dw2a.b_fan = k;
  // dW1[e] = sum x^T dh1 ; dW3[e] = sum x^T dh3
  GemmArgs dw1a = blank_args(offsets, s_sct, E, int(M));
  dw1a.Mo = int(d_model);
  dw1a.N = int(d_ff);
  dw1a.a0 = x;
  dw1a.a_rows = T;
  dw1a.lda = d_model;
  dw1a.a_scat = 1;
  dw1a.a_fan = k;
  dw1a.b0 = wl.dh1;
  dw1a.b_rows = M;
  dw1a.ldb = d_ff;
  GemmArgs dw3a = dw1a;
  dw3a.b0 = wl.dh3;

  // 2. dx contributions = dh W1^T (+ dh3 W3^T), then the k-sum.  The
  //    product's tiles that fill whole rounds of the chip go first; once
  //    they are done dW1 starts on a second stream, so that it fills the
  //    CUs the last, partial round of dx tiles leaves idle, and the caller's
  //    stream waits for it before dW2 (the two streams overlap only there:
  //    products running side by side for longer contend for L2).
  GemmArgs d = blank_args(offsets, s_sct, E, int(M));
  d.N = int(d_model);
  d.K0 = int(d_ff);
  d.K = swiglu ? int(2 * d_ff) : int(d_ff);
  d.a0 = wl.dh1;
  d.a1 = swiglu ? wl.dh3 : wl.dh1;
  d.a_rows = M;
  d.lda = d_ff;
  d.b0 = w1;
  d.b1 = swiglu ? w3 : w1;
  d.b_nk = 1;
  d.ldb = d_ff;
  d.b_es = d_model * d_ff;
  d.c0 = wl.pairs;
  d.c_scat = 1;
  d.ldc = d_model;
  GemmPlan pd;
  plan_gemm(d, pd, SEG_M, EPI_STORE, 0, bf16, 1);
  Fork fk(aux, st);
  const int64_t head = whole_round_tiles(d, pd);
  const bool overlap = fk.usable() && head > 0 && head < pd.grid;
  {
    RoleTimer t(SMOE_ROLE_DX, st);
    if (overlap) {
      GemmPlan p1 = pd, p2 = pd;
      p1.grid = head;
      d.g_count = int(head);
      SMOE_HIP(launch_gemm(d, p1, st), "mlp_bwd dx");
      SMOE_HIP(fk.fork(), "mlp_bwd fork");
      SMOE_TRY(run_dw(dw1a, bf16, dw1, dw_bf16, 0, wl.partial2, fk.side(), SMOE_ROLE_DW1, "mlp_bwd dW1"));
      d.g_base = int(head);
      d.g_count = 0;
      p2.grid = (pd.grid - head + 7) / 8 * 8;
      SMOE_HIP(launch_gemm(d, p2, st), "mlp_bwd dx");
    } else {
      SMOE_HIP(launch_gemm(d, pd, st), "mlp_bwd dx");
    }
  }
  {
    RoleTimer t(SMOE_ROLE_KSUM, st);
    SMOE_HIP(launch_combine(wl.pairs, nullptr, T, k, d_model, dx, bf16, st), "mlp_bwd ksum");
  }
  SMOE_HIP(fk.join(), "mlp_bwd join");
  // 3. the weight gradients
  SMOE_TRY(run_dw(dw2a, bf16, dw2, dw_bf16, 0, wl.partial, st, SMOE_ROLE_DW2, "mlp_bwd dW2"));
  if (!overlap) SMOE_TRY(run_dw(dw1a, bf16, dw1, dw_bf16, 0, wl.partial, st, SMOE_ROLE_DW1, "mlp_bwd dW1"));
  if (swiglu) SMOE_TRY(run_dw(dw3a, bf16, dw3, dw_bf16, 0, wl.partial, st, SMOE_ROLE_DW3, "mlp_bwd dW3"));
  return ok();
}

}  // extern "C"
