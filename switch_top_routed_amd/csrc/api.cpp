// C ABI of the Switch top-1 MoE layer: argument validation, workspace layout
// and the launch sequence.  Validation happens before any launch, so an error
// return (other than SWITCH_E_HIP) enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.hpp"
#include "switch_moe.h"

using namespace swm;

namespace {

thread_local char g_err[512] = "";

switch_status fail(switch_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

switch_status ok() {
  g_err[0] = '\0';
  return SWITCH_OK;
}

switch_status hip_fail(hipError_t e, const char* where) {
  return fail(SWITCH_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kMaxExperts = 1024;
constexpr int64_t kMaxTokens = (int64_t)1 << 30;
// 32-bit buffer offsets: a row of d_model elements times N <= 1024 experts
// (router) and one expert's d_model x d_ff weight matrix stay below 2^31 bytes
constexpr int32_t kMaxRow = 1 << 20;
constexpr int64_t kMaxWeight = (int64_t)1 << 30;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE_PTR(p)                                               \
  do {                                                               \
    if ((p) == nullptr) return fail(SWITCH_E_NULL, "%s is NULL", #p); \
  } while (0)

#define REQUIRE_ALIGN(p, a)                                                                       \
  do {                                                                                            \
    if (!aligned((p), (a))) return fail(SWITCH_E_ALIGN, "%s is not %d-byte aligned", #p, (int)(a)); \
  } while (0)

switch_status check_dtype(int32_t dtype) {
  if (dtype != SWITCH_F32 && dtype != SWITCH_BF16) return fail(SWITCH_E_UNSUPPORTED, "dtype %d is not supported", dtype);
  return SWITCH_OK;
}

switch_status check_tn(int64_t T, int32_t N) {
  if (T < 1 || T > kMaxTokens) return fail(SWITCH_E_SHAPE, "T=%lld outside [1, 2^30]", (long long)T);
  if (N < 1 || N > kMaxExperts) return fail(SWITCH_E_SHAPE, "N=%d outside [1, %d]", N, kMaxExperts);
  return SWITCH_OK;
}

switch_status check_rows(int32_t d, int32_t dtype, const char* name) {
  if (d < 1) return fail(SWITCH_E_SHAPE, "%s=%d must be >= 1", name, d);
  if (dtype == SWITCH_BF16 && d % 128 != 0) return fail(SWITCH_E_SHAPE, "%s=%d must be a multiple of 128 for bf16", name, d);
  if (dtype == SWITCH_F32 && d % 4 != 0) return fail(SWITCH_E_SHAPE, "%s=%d must be a multiple of 4 for f32", name, d);
  return SWITCH_OK;
}

switch_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need > 0 && ws == nullptr) return fail(SWITCH_E_NULL, "workspace is NULL (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(SWITCH_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  if (need > 0 && !aligned(ws, 256)) return fail(SWITCH_E_ALIGN, "workspace is not 256-byte aligned");
  return SWITCH_OK;
}

#define TRY(expr)                        \
  do {                                   \
    switch_status _s = (expr);           \
    if (_s != SWITCH_OK) return _s;      \
  } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

switch_status validate_route(const void* x, const void* w_gate, const float* bias, int64_t T, int32_t d, int32_t N,
                             int32_t dtype, const void* expert_id, const void* gate, const void* routed_count,
                             const void* f, const void* P, const void* l_aux) {
  TRY(check_dtype(dtype));
  TRY(check_tn(T, N));
  if (d < 1) return fail(SWITCH_E_SHAPE, "d_model=%d must be >= 1", d);
  if (d > kMaxRow) return fail(SWITCH_E_SHAPE, "d_model=%d exceeds 2^20", d);
  if (dtype == SWITCH_BF16 && d % 32 != 0) return fail(SWITCH_E_SHAPE, "d_model=%d must be a multiple of 32 for bf16 routing", d);
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(expert_id);
  REQUIRE_PTR(gate);
  REQUIRE_PTR(routed_count);
  REQUIRE_PTR(f);
  REQUIRE_PTR(P);
  REQUIRE_PTR(l_aux);
  REQUIRE_ALIGN(x, 16);
  REQUIRE_ALIGN(w_gate, 16);
  if (bias) REQUIRE_ALIGN(bias, 4);
  REQUIRE_ALIGN(expert_id, 4);
  REQUIRE_ALIGN(gate, 4);
  REQUIRE_ALIGN(routed_count, 4);
  REQUIRE_ALIGN(f, 4);
  REQUIRE_ALIGN(P, 4);
  REQUIRE_ALIGN(l_aux, 4);
  return SWITCH_OK;
}

switch_status validate_assign(const void* expert_id, const void* gate, int64_t T, int32_t N, int32_t C,
                              int32_t priority, const void* slot, const void* token_of_slot, const void* kept_count,
                              const void* n_dropped, const void* active, const void* n_active) {
  TRY(check_tn(T, N));
  if (C < 1 || C > T) return fail(SWITCH_E_SHAPE, "C=%d outside [1, T=%lld]", C, (long long)T);
  if ((int64_t)N * C > ((int64_t)1 << 31) - 1) return fail(SWITCH_E_SHAPE, "N*C exceeds 2^31-1");
  if (priority != SWITCH_TOKEN_ORDER && priority != SWITCH_GATE_DESC)
    return fail(SWITCH_E_UNSUPPORTED, "priority %d is not supported", priority);
  REQUIRE_PTR(expert_id);
  if (priority == SWITCH_GATE_DESC) REQUIRE_PTR(gate);
  REQUIRE_PTR(slot);
  REQUIRE_PTR(token_of_slot);
  REQUIRE_PTR(kept_count);
  REQUIRE_PTR(n_dropped);
  REQUIRE_PTR(active);
  REQUIRE_PTR(n_active);
  return SWITCH_OK;
}

switch_status validate_dispatch(const void* x, int32_t dtype, int64_t T, int32_t d, const void* token_of_slot,
                                const void* kept_count, int32_t N, int32_t C, const void* expert_in) {
  TRY(check_dtype(dtype));
  TRY(check_tn(T, N));
  if (C < 1 || C > T) return fail(SWITCH_E_SHAPE, "C=%d outside [1, T=%lld]", C, (long long)T);
  if (d < 1 || (d * (dtype == SWITCH_BF16 ? 2 : 4)) % 16 != 0)
    return fail(SWITCH_E_SHAPE, "d_model=%d: rows must be a multiple of 16 bytes", d);
  REQUIRE_PTR(x);
  REQUIRE_PTR(token_of_slot);
  REQUIRE_PTR(kept_count);
  REQUIRE_PTR(expert_in);
  REQUIRE_ALIGN(x, 16);
  REQUIRE_ALIGN(expert_in, 16);
  return SWITCH_OK;
}

switch_status validate_ffn(const void* expert_in, const void* w1, const void* w2, int32_t dtype, int32_t N, int32_t C,
                           int32_t d, int32_t dff, const void* kept_count, const void* active, const void* n_active,
                           const void* expert_out) {
  TRY(check_dtype(dtype));
  if (N < 1 || N > kMaxExperts) return fail(SWITCH_E_SHAPE, "N=%d outside [1, %d]", N, kMaxExperts);
  if (C < 1 || C > kMaxTokens) return fail(SWITCH_E_SHAPE, "C=%d must be >= 1", C);
  TRY(check_rows(d, dtype, "d_model"));
  TRY(check_rows(dff, dtype, "d_ff"));
  if (d > kMaxRow) return fail(SWITCH_E_SHAPE, "d_model=%d exceeds 2^20", d);
  if ((int64_t)d * dff > kMaxWeight)
    return fail(SWITCH_E_SHAPE, "d_model * d_ff = %lld exceeds 2^30", (long long)d * dff);
  REQUIRE_PTR(expert_in);
  REQUIRE_PTR(w1);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(kept_count);
  REQUIRE_PTR(active);
  REQUIRE_PTR(n_active);
  REQUIRE_PTR(expert_out);
  REQUIRE_ALIGN(expert_in, 16);
  REQUIRE_ALIGN(w1, 16);
  REQUIRE_ALIGN(w2, 16);
  REQUIRE_ALIGN(expert_out, 16);
  return SWITCH_OK;
}

switch_status validate_combine(const void* expert_out, const void* x, const void* shared_out, int32_t dtype, int64_t T,
                               int32_t d, const void* expert_id, const void* slot, const void* gate, int32_t N,
                               int32_t C, uint32_t flags, const void* y) {
  TRY(check_dtype(dtype));
  TRY(check_tn(T, N));
  if (C < 1) return fail(SWITCH_E_SHAPE, "C=%d must be >= 1", C);
  if (d < 1 || (d * (dtype == SWITCH_BF16 ? 2 : 4)) % 16 != 0)
    return fail(SWITCH_E_SHAPE, "d_model=%d: rows must be a multiple of 16 bytes", d);
  if (flags & ~(SWITCH_GATE_SCALE | SWITCH_RESIDUAL_ALL)) return fail(SWITCH_E_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  REQUIRE_PTR(expert_out);
  REQUIRE_PTR(x);
  REQUIRE_PTR(expert_id);
  REQUIRE_PTR(slot);
  if (flags & SWITCH_GATE_SCALE) REQUIRE_PTR(gate);
  REQUIRE_PTR(y);
  REQUIRE_ALIGN(expert_out, 16);
  REQUIRE_ALIGN(x, 16);
  if (shared_out) REQUIRE_ALIGN(shared_out, 16);
  REQUIRE_ALIGN(y, 16);
  return SWITCH_OK;
}

// ---------------------------------------------------------------------------
// whole-layer workspace layout
// ---------------------------------------------------------------------------
struct FwdLayout {
  int32_t C;
  int K;       // token choice: experts per token
  int M;       // Expanded Drop candidates (1: off)
  bool ec;     // expert choice
  bool fused;   // token order (top-1 or top-K): slots from one workgroup per expert right after the router
  bool gather;  // the dispatch folded into GEMM 1 (it reads each slot's token row from x)
  RoutePlan route;
  AssignPlan assign;
  FfnPlan ffn, sffn;
  size_t off_route, off_assign, off_term, off_tos, off_active, off_nact, off_xin, off_xout, off_ffn;
  size_t off_dense, off_sffn, off_sout, off_ev, off_gv, off_slotv, off_probs_t, off_pick, off_list, bytes;
};

// GEMM 1 gathers its rows from x through token_of_slot whenever the token
// matrix is addressable through 32-bit buffer offsets; the fused assignment
// also needs token order (top-1 or top-K token choice).

FwdLayout fwd_layout(const switch_moe_desc& d, int32_t C) {
  FwdLayout L{};
  L.C = C;
  const size_t esz = d.dtype == SWITCH_BF16 ? 2 : 4;
  L.K = d.top_k < 1 ? 1 : d.top_k;
  L.M = d.expand_choices < 1 ? 1 : d.expand_choices;
  L.ec = d.routing == SWITCH_EXPERT_CHOICE;
  L.route = route_plan(d.T, d.d_model, d.N, d.dtype);
  L.gather = (int64_t)d.T * d.d_model * (int64_t)esz < ((int64_t)1 << 31);
  L.fused = !L.ec && d.priority == SWITCH_TOKEN_ORDER && L.gather;
  L.ffn = ffn_plan(d.N, C, d.d_model, d.d_ff, d.dtype);
  size_t off = 0;
  L.off_route = off;
  off = align_up(off + L.route.bytes);
  if (L.fused) {
    L.off_term = off;
    off = align_up(off + (size_t)d.N * 8);
    if (L.K > 1) {  // the router's choice-major lists [K, T]
      L.off_ev = off;
      off = align_up(off + (size_t)L.K * d.T * 4);
      L.off_gv = off;
      off = align_up(off + (size_t)L.K * d.T * 4);
    }
  } else if (!L.ec) {
    const int64_t TV = (int64_t)L.K * d.T;  // assignments ("virtual tokens")
    L.assign = assign_plan(TV, d.N, C, d.priority);
    L.off_assign = off;
    off = align_up(off + L.assign.bytes);
    if (L.K > 1) {
      L.off_ev = off;
      off = align_up(off + (size_t)TV * 4);
      L.off_gv = off;
      off = align_up(off + (size_t)TV * 4);
      L.off_slotv = off;
      off = align_up(off + (size_t)TV * 4);
    }
  } else {
    L.off_probs_t = off;
    off = align_up(off + (size_t)d.T * d.N * 4);
    L.off_pick = off;
    off = align_up(off + (size_t)d.T * d.N * 4);
  }
  if (L.M > 1) {  // candidate lists [M, T] and one applicant list per expert
    L.off_ev = off;
    off = align_up(off + (size_t)L.M * d.T * 4);
    L.off_gv = off;
    off = align_up(off + (size_t)L.M * d.T * 4);
    L.off_list = off;
    off = align_up(off + (size_t)d.N * d.T * 4);
  }
  L.off_tos = off;
  off = align_up(off + (size_t)d.N * C * 4);
  L.off_active = off;
  off = align_up(off + (size_t)d.N * 4);
  L.off_nact = off;
  off = align_up(off + 4);
  L.off_xin = off;
  if (!L.gather) off = align_up(off + (size_t)d.N * C * d.d_model * esz);
  L.off_xout = off;
  off = align_up(off + (size_t)d.N * C * d.d_model * esz);
  L.off_ffn = off;
  off = align_up(off + L.ffn.bytes);
  if (d.d_ff_shared > 0) {
    L.sffn = ffn_plan(1, (int)d.T, d.d_model, d.d_ff_shared, d.dtype);
    L.off_dense = off;
    off = align_up(off + 3 * 4);
    L.off_sffn = off;
    off = align_up(off + L.sffn.bytes);
    L.off_sout = off;
    off = align_up(off + (size_t)d.T * d.d_model * esz);
  }
  L.bytes = off;
  return L;
}

switch_status validate_desc(const switch_moe_desc* d, int32_t* C) {
  if (d == nullptr) return fail(SWITCH_E_NULL, "desc is NULL");
  TRY(check_dtype(d->dtype));
  TRY(check_tn(d->T, d->N));
  TRY(check_rows(d->d_model, d->dtype, "d_model"));
  TRY(check_rows(d->d_ff, d->dtype, "d_ff"));
  if (d->d_ff_shared < 0) return fail(SWITCH_E_SHAPE, "d_ff_shared=%d must be >= 0", d->d_ff_shared);
  if (d->d_ff_shared > 0) TRY(check_rows(d->d_ff_shared, d->dtype, "d_ff_shared"));
  if (d->d_model > kMaxRow) return fail(SWITCH_E_SHAPE, "d_model=%d exceeds 2^20", d->d_model);
  if ((int64_t)d->d_model * d->d_ff > kMaxWeight || (int64_t)d->d_model * d->d_ff_shared > kMaxWeight)
    return fail(SWITCH_E_SHAPE, "d_model * d_ff (or d_ff_shared) exceeds 2^30");
  if (d->priority != SWITCH_TOKEN_ORDER && d->priority != SWITCH_GATE_DESC)
    return fail(SWITCH_E_UNSUPPORTED, "priority %d is not supported", d->priority);
  if (d->flags & ~(SWITCH_GATE_SCALE | SWITCH_RESIDUAL_ALL | SWITCH_RENORM | SWITCH_ACCUM_EXPERT_GRADS))
    return fail(SWITCH_E_UNSUPPORTED, "unknown flag bits 0x%x", d->flags);
  if (d->routing != SWITCH_TOKEN_CHOICE && d->routing != SWITCH_EXPERT_CHOICE)
    return fail(SWITCH_E_UNSUPPORTED, "routing %d is not supported", d->routing);
  const int K = d->top_k < 1 ? 1 : d->top_k;
  if (K > kMaxTopK || K > d->N) return fail(SWITCH_E_SHAPE, "top_k=%d outside [1, min(N, %d)]", K, kMaxTopK);
  if (d->routing == SWITCH_EXPERT_CHOICE && K != 1)
    return fail(SWITCH_E_UNSUPPORTED, "expert choice takes no top_k (top_k=%d)", d->top_k);
  if (K > 1 && (int64_t)K * d->T > kMaxTokens)
    return fail(SWITCH_E_SHAPE, "top_k * T = %lld exceeds 2^30", (long long)K * d->T);
  const int M = d->expand_choices < 1 ? 1 : d->expand_choices;
  if (M > 1) {
    if (K != 1 || d->routing != SWITCH_TOKEN_CHOICE)
      return fail(SWITCH_E_UNSUPPORTED, "Expanded Drop re-routes top-1 token choice only");
    if (M > kMaxTopK || M > d->N)
      return fail(SWITCH_E_SHAPE, "expand_choices=%d outside [2, min(N, %d)]", M, kMaxTopK);
    if (d->flags & SWITCH_RENORM) return fail(SWITCH_E_UNSUPPORTED, "SWITCH_RENORM applies to top-K only");
    if ((int64_t)M * d->T > kMaxTokens || (int64_t)d->N * d->T > ((int64_t)1 << 31) - 1)
      return fail(SWITCH_E_SHAPE, "Expanded Drop lists (M T, N T) exceed their index range");
  }
  int32_t c = d->C;
  if (c == 0) {
    c = switch_capacity(K * d->T, d->N, d->capacity_factor);  // K assignments per token
    if (c < 1) return fail(SWITCH_E_SHAPE, "capacity_factor=%g gives no capacity", d->capacity_factor);
    if (c > d->T) c = (int32_t)d->T;  // an expert receives each token at most once
  }
  if (c < 1 || c > d->T) return fail(SWITCH_E_SHAPE, "C=%d outside [1, T=%lld]", c, (long long)d->T);
  if (d->routing == SWITCH_EXPERT_CHOICE && c > kMaxExpertChoiceK)
    return fail(SWITCH_E_UNSUPPORTED, "expert choice with min(C, T) = %d beyond %d", c, kMaxExpertChoiceK);
  if (M > 1 && c > kMaxExpertChoiceK)
    return fail(SWITCH_E_UNSUPPORTED, "Expanded Drop with C = %d beyond %d", c, kMaxExpertChoiceK);
  if (d->weight_format != SWITCH_WEIGHTS_NATIVE && d->weight_format != SWITCH_WEIGHTS_MXFP4)
    return fail(SWITCH_E_UNSUPPORTED, "weight_format %d is not supported", d->weight_format);
  if (d->weight_format == SWITCH_WEIGHTS_MXFP4 && (d->dtype != SWITCH_BF16 || !mx_ffn_applies(c, d->d_model, d->d_ff)))
    return fail(SWITCH_E_UNSUPPORTED, "MXFP4 expert weights need a bf16 layer with C <= 64 (C=%d)", c);
  if ((int64_t)d->N * c > ((int64_t)1 << 31) - 1) return fail(SWITCH_E_SHAPE, "N*C exceeds 2^31-1");
  *C = c;
  return SWITCH_OK;
}

// training (the saved forward and the backward): the top-1 layer with native weights
switch_status check_trainable(const switch_moe_desc& d) {
  if (d.top_k > 1 || d.routing != SWITCH_TOKEN_CHOICE || d.weight_format != SWITCH_WEIGHTS_NATIVE ||
      d.expand_choices > 1)
    return fail(SWITCH_E_UNSUPPORTED, "training supports top-1 routing with native weights only");
  return SWITCH_OK;
}

switch_status validate_saved(const switch_moe_desc& d, const switch_moe_saved* sv) {
  REQUIRE_PTR(sv->probs);
  REQUIRE_PTR(sv->token_of_slot);
  REQUIRE_PTR(sv->active);
  REQUIRE_PTR(sv->n_active);
  REQUIRE_PTR(sv->h);
  REQUIRE_ALIGN(sv->probs, 4);
  REQUIRE_ALIGN(sv->token_of_slot, 4);
  REQUIRE_ALIGN(sv->active, 4);
  REQUIRE_ALIGN(sv->n_active, 4);
  REQUIRE_ALIGN(sv->h, 16);
  if (d.d_ff_shared > 0) {
    REQUIRE_PTR(sv->h_shared);
    REQUIRE_ALIGN(sv->h_shared, 16);
  }
  return SWITCH_OK;
}

// ---------------------------------------------------------------------------
// backward workspace layout
// ---------------------------------------------------------------------------
struct BwdLayout {
  bool fused;  // bf16 MFMA expert passes (else the generic GEMMs)
  int dg_parts;
  RouterBwdPlan rp;  // bf16 router backward
  size_t off_u, off_dz, off_dg, off_dxe, off_dlogit, off_colsum, off_dense, off_us, off_dzs, off_dxs;
  size_t off_hi, off_lo, off_rpart, bytes;
};

BwdLayout bwd_layout(const switch_moe_desc& d, int32_t C) {
  BwdLayout L{};
  const size_t esz = d.dtype == SWITCH_BF16 ? 2 : 4;
  const size_t NC = (size_t)d.N * C;
  L.fused = d.dtype == SWITCH_BF16 && fused_expert_bwd_applies(d.T, C, d.d_model, d.d_ff);
  L.dg_parts = L.fused ? d.d_ff / 64 : 1;
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = off;
    off = align_up(off + bytes);
  };
  if (!L.fused) take(L.off_u, NC * d.d_ff * 4);
  take(L.off_dz, NC * d.d_ff * esz);
  take(L.off_dg, NC * L.dg_parts * 4);
  take(L.off_dxe, NC * d.d_model * 4);
  take(L.off_dlogit, (size_t)d.T * d.N * 4);
  take(L.off_colsum, colsum_scratch_bytes(d.T, d.N));
  if (d.dtype == SWITCH_BF16) {
    L.rp = router_bwd_plan(d.T, d.N, d.d_model);
    take(L.off_hi, L.rp.planes_bytes);
    take(L.off_lo, L.rp.planes_bytes);
    take(L.off_rpart, L.rp.partial_bytes);
  }
  if (d.d_ff_shared > 0) {
    take(L.off_dense, 3 * 4);
    if (!(d.dtype == SWITCH_BF16 && dense_bwd_applies(d.T, d.d_model, d.d_ff_shared)))
      take(L.off_us, (size_t)d.T * d.d_ff_shared * 4);  // the generic path's fp32 U
    take(L.off_dzs, (size_t)d.T * d.d_ff_shared * esz);
    take(L.off_dxs, (size_t)d.T * d.d_model * 4);
  }
  L.bytes = off;
  return L;
}

}  // namespace

extern "C" {

int32_t switch_capacity(int64_t T, int32_t N, double capacity_factor) {
  if (T < 1 || N < 1 || !(capacity_factor > 0.0) || !std::isfinite(capacity_factor)) return -1;
  const int32_t cap_t = (int32_t)(T < INT32_MAX ? T : INT32_MAX);
  // far from both ends the double estimate decides alone
  const double est = capacity_factor * (double)T / (double)N;
  if (est > 2.0 * (double)T + 2.0) return cap_t;
  if (est < 0.25) return 1;
  // capacity_factor is taken at its decimal value: the shortest decimal string
  // that reads back as the same double (what a caller wrote, e.g. 1.1, not
  // 1.100000000000000088817...).  cf = M 10^E, C = ceil(M 10^E T / N), exact.
  char buf[40];
  for (int prec = 1; prec <= 17; ++prec) {
    snprintf(buf, sizeof(buf), "%.*e", prec - 1, capacity_factor);
    if (std::strtod(buf, nullptr) == capacity_factor) break;
  }
  unsigned __int128 M = 0;
  int digits_after = 0, exp10 = 0;
  bool after = false;
  const char* q = buf;
  for (; *q && *q != 'e' && *q != 'E'; ++q) {
    if (*q == '.') {
      after = true;
    } else if (*q >= '0' && *q <= '9') {
      M = M * 10 + (unsigned)(*q - '0');
      if (after) ++digits_after;
    }
  }
  if (*q == 'e' || *q == 'E') exp10 = (int)std::strtol(q + 1, nullptr, 10);
  const int E = exp10 - digits_after;  // cf = M 10^E, M < 10^17
  unsigned __int128 num = M * (unsigned __int128)T, den = (unsigned __int128)N;
  // |E| stays small here: est in [0.25, 2T + 2] with M < 10^17 bounds it
  if (E >= 0) {
    for (int i = 0; i < E; ++i) num *= 10;
  } else {
    for (int i = 0; i < -E; ++i) den *= 10;
  }
  const unsigned __int128 c = (num + den - 1) / den;
  if (c > (unsigned __int128)cap_t) return cap_t;
  return c < 1 ? 1 : (int32_t)c;
}

size_t switch_route_workspace_bytes(int64_t T, int32_t d_model, int32_t N, int32_t dtype) {
  if (T < 1 || N < 1 || d_model < 1) return 0;
  return route_plan(T, d_model, N, dtype).bytes;
}

switch_status switch_route(const void* x, const void* w_gate, const float* bias, int64_t T, int32_t d_model,
                           int32_t N, int32_t dtype, int32_t* expert_id, float* gate, int32_t* routed_count,
                           float* f, float* P, float* l_aux, void* ws, size_t ws_bytes, void* stream) {
  TRY(validate_route(x, w_gate, bias, T, d_model, N, dtype, expert_id, gate, routed_count, f, P, l_aux));
  const RoutePlan pl = route_plan(T, d_model, N, dtype);
  TRY(check_ws(ws, ws_bytes, pl.bytes));
  hipError_t e = launch_route(pl, x, w_gate, bias, T, d_model, N, dtype, expert_id, gate, routed_count, f, P, l_aux,
                              static_cast<char*>(ws), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "switch_route");
  return ok();
}

size_t switch_assign_workspace_bytes(int64_t T, int32_t N, int32_t C, int32_t priority) {
  if (T < 1 || N < 1) return 0;
  return assign_plan(T, N, C, priority).bytes;
}

switch_status switch_assign_capacity(const int32_t* expert_id, const float* gate, int64_t T, int32_t N, int32_t C,
                                     int32_t priority, int32_t* slot, int32_t* token_of_slot, int32_t* kept_count,
                                     int32_t* n_dropped, int32_t* active, int32_t* n_active, void* ws,
                                     size_t ws_bytes, void* stream) {
  TRY(validate_assign(expert_id, gate, T, N, C, priority, slot, token_of_slot, kept_count, n_dropped, active,
                      n_active));
  const AssignPlan pl = assign_plan(T, N, C, priority);
  TRY(check_ws(ws, ws_bytes, pl.bytes));
  hipError_t e = launch_assign(pl, expert_id, gate, T, N, C, priority, slot, token_of_slot, kept_count, n_dropped,
                               active, n_active, static_cast<char*>(ws), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "switch_assign_capacity");
  return ok();
}

switch_status switch_dispatch(const void* x, int32_t dtype, int64_t T, int32_t d_model, const int32_t* token_of_slot,
                              const int32_t* kept_count, int32_t N, int32_t C, void* expert_in, void* stream) {
  TRY(validate_dispatch(x, dtype, T, d_model, token_of_slot, kept_count, N, C, expert_in));
  hipError_t e = launch_dispatch(x, dtype, T, d_model, token_of_slot, kept_count, N, C, expert_in,
                                 as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "switch_dispatch");
  return ok();
}

size_t switch_expert_ffn_workspace_bytes(int32_t N, int32_t C, int32_t d_model, int32_t d_ff, int32_t dtype) {
  if (N < 1 || C < 1 || d_model < 1 || d_ff < 1) return 0;
  return ffn_plan(N, C, d_model, d_ff, dtype).bytes;
}

switch_status switch_expert_ffn(const void* expert_in, const void* w1, const void* w2, int32_t dtype, int32_t N,
                                int32_t C, int32_t d_model, int32_t d_ff, const int32_t* kept_count,
                                const int32_t* active, const int32_t* n_active, void* expert_out, void* ws,
                                size_t ws_bytes, void* stream) {
  TRY(validate_ffn(expert_in, w1, w2, dtype, N, C, d_model, d_ff, kept_count, active, n_active, expert_out));
  const FfnPlan pl = ffn_plan(N, C, d_model, d_ff, dtype);
  TRY(check_ws(ws, ws_bytes, pl.bytes));
  hipError_t e = launch_ffn(pl, expert_in, w1, w2, dtype, N, C, d_model, d_ff, kept_count, active, n_active,
                            expert_out, static_cast<char*>(ws), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "switch_expert_ffn");
  return ok();
}

switch_status switch_combine(const void* expert_out, const void* x, const void* shared_out, int32_t dtype, int64_t T,
                             int32_t d_model, const int32_t* expert_id, const int32_t* slot, const float* gate,
                             int32_t N, int32_t C, uint32_t flags, void* y, void* stream) {
  TRY(validate_combine(expert_out, x, shared_out, dtype, T, d_model, expert_id, slot, gate, N, C, flags, y));
  hipError_t e = launch_combine(expert_out, x, shared_out, dtype, T, d_model, expert_id, slot, gate, N, C, flags, y,
                                as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "switch_combine");
  return ok();
}

switch_status switch_quantize_mxfp4(const void* w, int32_t dtype, int64_t batches, int32_t K, int32_t Ncols,
                                    uint8_t* codes, uint8_t* scales, void* stream) {
  TRY(check_dtype(dtype));
  if (batches < 1 || batches > 65535) return fail(SWITCH_E_SHAPE, "batches=%lld outside [1, 65535]", (long long)batches);
  if (K < 128 || K % 128 != 0 || K > (1 << 21)) return fail(SWITCH_E_SHAPE, "K=%d: a multiple of 128 up to 2^21", K);
  if (Ncols < 1) return fail(SWITCH_E_SHAPE, "Ncols=%d must be >= 1", Ncols);
  REQUIRE_PTR(w);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_ALIGN(codes, 16);
  hipError_t e = launch_mx_quantize(w, dtype, batches, K, Ncols, codes, scales, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "switch_quantize_mxfp4");
  return ok();
}

size_t switch_moe_workspace_bytes(const switch_moe_desc* desc) {
  int32_t C = 0;
  if (validate_desc(desc, &C) != SWITCH_OK) return 0;
  return fwd_layout(*desc, C).bytes;
}

}  // extern "C"

// The whole layer; `ev` (7 events or NULL) marks the stage boundaries on the stream.
static switch_status moe_forward(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                 const switch_moe_outputs* out, void* ws, size_t ws_bytes, void* stream,
                                 void* const* ev, const switch_moe_saved* sv = nullptr) {
  int32_t C = 0;
  TRY(validate_desc(desc, &C));
  if (in == nullptr) return fail(SWITCH_E_NULL, "inputs is NULL");
  if (out == nullptr) return fail(SWITCH_E_NULL, "outputs is NULL");
  const switch_moe_desc& d = *desc;
  TRY(validate_route(in->x, in->w_gate, in->bias, d.T, d.d_model, d.N, d.dtype, out->expert_id, out->gate,
                     out->routed_count, out->f, out->P, out->l_aux));
  REQUIRE_PTR(in->w1);
  REQUIRE_PTR(in->w2);
  REQUIRE_ALIGN(in->w1, 16);
  REQUIRE_ALIGN(in->w2, 16);
  const bool mxw = d.weight_format == SWITCH_WEIGHTS_MXFP4;
  if (mxw) {
    REQUIRE_PTR(in->w1_scale);
    REQUIRE_PTR(in->w2_scale);
    REQUIRE_ALIGN(in->w1_scale, 4);
    REQUIRE_ALIGN(in->w2_scale, 4);
  }
  REQUIRE_PTR(out->y);
  REQUIRE_ALIGN(out->y, 16);
  REQUIRE_PTR(out->slot);
  REQUIRE_PTR(out->kept_count);
  REQUIRE_PTR(out->n_dropped);
  if (d.d_ff_shared > 0) {
    REQUIRE_PTR(in->ws1);
    REQUIRE_PTR(in->ws2);
    REQUIRE_ALIGN(in->ws1, 16);
    REQUIRE_ALIGN(in->ws2, 16);
  }
  if (sv != nullptr) {
    TRY(check_trainable(d));
    TRY(validate_saved(d, sv));
  }
  const FwdLayout L = fwd_layout(d, C);
  TRY(check_ws(ws, ws_bytes, L.bytes));
  char* w = static_cast<char*>(ws);
  hipStream_t st = as_stream(stream);
  int32_t* tos = sv != nullptr ? sv->token_of_slot : reinterpret_cast<int32_t*>(w + L.off_tos);
  int32_t* active = sv != nullptr ? sv->active : reinterpret_cast<int32_t*>(w + L.off_active);
  int32_t* nact = sv != nullptr ? sv->n_active : reinterpret_cast<int32_t*>(w + L.off_nact);
  RouteExtra rex;
  rex.probs = sv != nullptr ? sv->probs : nullptr;
  rex.K = L.K;
  rex.renorm = (d.flags & SWITCH_RENORM) != 0;
  if (L.K > 1 || L.M > 1) {
    rex.ev_cm = reinterpret_cast<int32_t*>(w + L.off_ev);
    rex.gv_cm = reinterpret_cast<float*>(w + L.off_gv);
  }
  if (L.M > 1) {
    rex.K = L.M;
    rex.expand = 1;
  }
  if (L.ec) rex.probs_t = reinterpret_cast<float*>(w + L.off_probs_t);
  void* h_save = sv != nullptr ? sv->h : nullptr;
  const MxWeights mxs{static_cast<const uint8_t*>(in->w1), in->w1_scale, static_cast<const uint8_t*>(in->w2),
                      in->w2_scale};
  const MxWeights* mxp = mxw ? &mxs : nullptr;
  void* xin = w + L.off_xin;
  void* xout = w + L.off_xout;
  auto mark = [&](int i) -> hipError_t {
    return (ev != nullptr && ev[i] != nullptr) ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), st) : hipSuccess;
  };

  hipError_t e = mark(0);
  if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
  e = launch_route(L.route, in->x, in->w_gate, in->bias, d.T, d.d_model, d.N, d.dtype, out->expert_id, out->gate,
                   out->routed_count, out->f, out->P, out->l_aux, w + L.off_route, st, L.fused, rex);
  if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/route");
  if ((e = mark(1)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
  // the first (streaming) GEMM builds the assignment's cross-expert results
  // itself, so no kernel runs between the assignment and the GEMM
  const bool gemm_finalizes =
      L.fused && L.M == 1 && ffn_stream_applies(d.dtype, C, d.d_model, d.d_ff, mxp != nullptr);
  ActiveFromKept afk;
  if (gemm_finalizes) {
    afk.kept = out->kept_count;
    afk.term = reinterpret_cast<const double*>(w + L.off_term);
    afk.active = active;
    afk.n_active = nact;
    afk.n_dropped = out->n_dropped;
    afk.l_aux = out->l_aux;
    afk.TV = (int64_t)L.K * d.T;
  }
  if (L.fused) {
    // token order: one workgroup per expert takes its tokens into slots (and
    // reduces the router statistics); GEMM 1 then reads each slot's token row
    // straight from x
    e = launch_assign_token(L.route, d.T, L.K, d.N, C, L.K > 1 ? rex.ev_cm : out->expert_id,
                            reinterpret_cast<double*>(w + L.off_term),
                            out->routed_count, out->f, out->P, out->l_aux, out->slot, tos, out->kept_count,
                            out->n_dropped, active, nact, w + L.off_route, st, !gemm_finalizes && L.M == 1);
    if (e == hipSuccess && L.M > 1)  // the expansion's finalize also takes L_aux over
      e = launch_expand(rex.ev_cm, rex.gv_cm, d.T, d.N, C, L.M, 0, out->slot, out->expert_id, out->gate, tos,
                        out->kept_count, active, nact, out->n_dropped, reinterpret_cast<int32_t*>(w + L.off_list), st,
                        reinterpret_cast<const double*>(w + L.off_term), out->l_aux);
    if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/assign");
    if ((e = mark(2)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
    if ((e = mark(3)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
    e = launch_ffn(L.ffn, in->x, in->w1, in->w2, d.dtype, d.N, C, d.d_model, d.d_ff, out->kept_count, active, nact,
                   xout, w + L.off_ffn, st, tos, d.T, h_save, mxp, gemm_finalizes ? &afk : nullptr);
  } else {
    if (L.ec) {
      e = launch_ec_select(rex.probs_t, d.T, d.N, C, tos, reinterpret_cast<int32_t*>(w + L.off_pick),
                           out->kept_count, active, nact, out->n_dropped, st);
    } else if (L.K > 1) {
      // rank the K T assignments as one list, then back to token rows and [T, K] slots
      int32_t* slot_v = reinterpret_cast<int32_t*>(w + L.off_slotv);
      e = launch_assign(L.assign, rex.ev_cm, rex.gv_cm, (int64_t)L.K * d.T, d.N, C, d.priority, slot_v, tos,
                        out->kept_count, out->n_dropped, active, nact, w + L.off_assign, st);
      if (e == hipSuccess) e = launch_topk_fixup(slot_v, d.T, L.K, tos, (int64_t)d.N * C, out->slot, st);
    } else {
      e = launch_assign(L.assign, out->expert_id, out->gate, d.T, d.N, C, d.priority, out->slot, tos,
                        out->kept_count, out->n_dropped, active, nact, w + L.off_assign, st);
      if (e == hipSuccess && L.M > 1)
        e = launch_expand(rex.ev_cm, rex.gv_cm, d.T, d.N, C, L.M, d.priority == SWITCH_GATE_DESC ? 1 : 0, out->slot,
                          out->expert_id, out->gate, tos, out->kept_count, active, nact, out->n_dropped,
                          reinterpret_cast<int32_t*>(w + L.off_list), st);
    }
    if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/assign");
    if ((e = mark(2)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
    if (!L.gather) {
      e = launch_dispatch(in->x, d.dtype, d.T, d.d_model, tos, out->kept_count, d.N, C, xin, st);
      if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/dispatch");
    }
    if ((e = mark(3)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
    e = launch_ffn(L.ffn, L.gather ? in->x : xin, in->w1, in->w2, d.dtype, d.N, C, d.d_model, d.d_ff, out->kept_count,
                   active, nact, xout, w + L.off_ffn, st, L.gather ? tos : nullptr, L.gather ? d.T : 0, h_save, mxp);
  }
  if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/expert_ffn");
  if ((e = mark(4)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
  void* sout = nullptr;
  // top-1 token choice with a shared expert on the tiled GEMM: its second GEMM
  // does the combine as it writes S, so S never goes to memory and no combine
  // kernel runs (the events 5 and 6 then bracket nothing)
  const bool fused_combine = d.d_ff_shared > 0 && !L.ec && L.K == 1 && d.dtype == SWITCH_BF16 &&
                             tiled_ffn_applies((int)d.T, d.d_model, d.d_ff_shared);
  if (d.d_ff_shared > 0) {
    int32_t* dk = reinterpret_cast<int32_t*>(w + L.off_dense);
    e = launch_dense_plan(dk, dk + 1, dk + 2, (int32_t)d.T, st);
    if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/shared_plan");
    sout = w + L.off_sout;
    CombineArgs cmb;
    if (fused_combine) {
      cmb.eo = static_cast<const uint16_t*>(xout);
      cmb.x = static_cast<const uint16_t*>(in->x);
      cmb.expert_id = out->expert_id;
      cmb.slot = out->slot;
      cmb.gate = out->gate;
      cmb.N = d.N;
      cmb.C = C;
      cmb.flags = d.flags;
      cmb.y = static_cast<uint16_t*>(out->y);
    }
    e = launch_ffn(L.sffn, in->x, in->ws1, in->ws2, d.dtype, 1, (int)d.T, d.d_model, d.d_ff_shared, dk, dk + 1,
                   dk + 2, sout, w + L.off_sffn, st, nullptr, 0, sv != nullptr ? sv->h_shared : nullptr, nullptr,
                   nullptr, fused_combine ? &cmb : nullptr);
    if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/shared_ffn");
  }
  if ((e = mark(5)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
  if (fused_combine)
    e = hipSuccess;
  else if (L.ec)
    e = launch_combine_picks(1, xout, in->x, sout, d.dtype, d.T, d.d_model, 1, nullptr, nullptr, nullptr,
                             reinterpret_cast<const int32_t*>(w + L.off_pick), rex.probs_t, d.N, C, d.flags,
                             out->slot, out->n_dropped, out->y, st);
  else if (L.K > 1)
    e = launch_combine_picks(0, xout, in->x, sout, d.dtype, d.T, d.d_model, L.K, out->expert_id, out->slot,
                             out->gate, nullptr, nullptr, d.N, C, d.flags, nullptr, nullptr, out->y, st);
  else
    e = launch_combine(xout, in->x, sout, d.dtype, d.T, d.d_model, out->expert_id, out->slot, out->gate, d.N, C,
                       d.flags, out->y, st);
  if (e != hipSuccess) return hip_fail(e, "switch_moe_forward/combine");
  if ((e = mark(6)) != hipSuccess) return hip_fail(e, "switch_moe_forward/event");
  return ok();
}

namespace swm {
switch_status abi_forward(const switch_moe_desc* desc, const switch_moe_inputs* in, const switch_moe_outputs* out,
                          void* ws, size_t ws_bytes, void* stream) {
  return moe_forward(desc, in, out, ws, ws_bytes, stream, nullptr);
}
switch_status abi_forward_bytes(const switch_moe_desc* desc, size_t* bytes) {
  int32_t C = 0;
  TRY(validate_desc(desc, &C));
  *bytes = fwd_layout(*desc, C).bytes;
  return SWITCH_OK;
}
switch_status abi_fail(switch_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace swm

extern "C" {

switch_status switch_moe_forward(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                 const switch_moe_outputs* out, void* ws, size_t ws_bytes, void* stream) {
  return moe_forward(desc, in, out, ws, ws_bytes, stream, nullptr);
}

switch_status switch_moe_forward_timed(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                       const switch_moe_outputs* out, void* ws, size_t ws_bytes, void* stream,
                                       void* const* stage_events) {
  if (stage_events == nullptr) return fail(SWITCH_E_NULL, "stage_events is NULL");
  return moe_forward(desc, in, out, ws, ws_bytes, stream, stage_events);
}

switch_status switch_moe_forward_train(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                       const switch_moe_outputs* out, const switch_moe_saved* saved, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (saved == nullptr) return fail(SWITCH_E_NULL, "saved is NULL");
  return moe_forward(desc, in, out, ws, ws_bytes, stream, nullptr, saved);
}

size_t switch_moe_backward_workspace_bytes(const switch_moe_desc* desc) {
  int32_t C = 0;
  if (validate_desc(desc, &C) != SWITCH_OK || check_trainable(*desc) != SWITCH_OK) return 0;
  return bwd_layout(*desc, C).bytes;
}

}  // extern "C"

// The layer backward; `ev` (6 events or NULL) marks the stage boundaries on the stream.
static switch_status moe_backward(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                  const switch_moe_outputs* fwd, const switch_moe_saved* saved, const void* dy,
                                  const float* dl_aux, const switch_moe_grads* grads, void* ws, size_t ws_bytes,
                                  void* stream, void* const* ev) {
  int32_t C = 0;
  TRY(validate_desc(desc, &C));
  if (in == nullptr) return fail(SWITCH_E_NULL, "inputs is NULL");
  if (fwd == nullptr) return fail(SWITCH_E_NULL, "fwd is NULL");
  if (saved == nullptr) return fail(SWITCH_E_NULL, "saved is NULL");
  if (grads == nullptr) return fail(SWITCH_E_NULL, "grads is NULL");
  const switch_moe_desc& d = *desc;
  TRY(check_trainable(d));
  const bool gate_scale = (d.flags & SWITCH_GATE_SCALE) != 0;
  REQUIRE_PTR(in->x);
  REQUIRE_PTR(in->w_gate);
  REQUIRE_PTR(in->w1);
  REQUIRE_PTR(in->w2);
  REQUIRE_ALIGN(in->x, 16);
  REQUIRE_ALIGN(in->w_gate, 16);
  REQUIRE_ALIGN(in->w1, 16);
  REQUIRE_ALIGN(in->w2, 16);
  REQUIRE_PTR(fwd->expert_id);
  REQUIRE_PTR(fwd->slot);
  REQUIRE_PTR(fwd->kept_count);
  REQUIRE_PTR(fwd->f);
  if (gate_scale) REQUIRE_PTR(fwd->gate);
  TRY(validate_saved(d, saved));
  REQUIRE_PTR(dy);
  REQUIRE_ALIGN(dy, 16);
  REQUIRE_PTR(grads->dx);
  REQUIRE_PTR(grads->dw_gate);
  REQUIRE_PTR(grads->dw1);
  REQUIRE_PTR(grads->dw2);
  REQUIRE_ALIGN(grads->dx, 16);
  REQUIRE_ALIGN(grads->dw_gate, 16);
  REQUIRE_ALIGN(grads->dw1, 16);
  REQUIRE_ALIGN(grads->dw2, 16);
  if (grads->dbias) REQUIRE_ALIGN(grads->dbias, 4);
  if (d.d_ff_shared > 0) {
    REQUIRE_PTR(in->ws1);
    REQUIRE_PTR(in->ws2);
    REQUIRE_PTR(grads->dws1);
    REQUIRE_PTR(grads->dws2);
    REQUIRE_ALIGN(grads->dws1, 16);
    REQUIRE_ALIGN(grads->dws2, 16);
  }
  const BwdLayout L = bwd_layout(d, C);
  const bool accum = (d.flags & SWITCH_ACCUM_EXPERT_GRADS) != 0;
  if (accum && !L.fused)
    return fail(SWITCH_E_UNSUPPORTED,
                "SWITCH_ACCUM_EXPERT_GRADS needs the fused bf16 expert backward (C <= 160, d and d_ff multiples of 64)");
  TRY(check_ws(ws, ws_bytes, L.bytes));
  char* w = static_cast<char*>(ws);
  hipStream_t st = as_stream(stream);
  const int dt = d.dtype, dm = d.d_model, dff = d.d_ff, N = d.N;
  const int64_t T = d.T;
  const int32_t* kept = fwd->kept_count;
  const int32_t* tos = saved->token_of_slot;
  float* U = L.fused ? nullptr : reinterpret_cast<float*>(w + L.off_u);
  void* dZ = w + L.off_dz;
  float* dg = gate_scale ? reinterpret_cast<float*>(w + L.off_dg) : nullptr;
  float* dxe = reinterpret_cast<float*>(w + L.off_dxe);
  float* dlogit = reinterpret_cast<float*>(w + L.off_dlogit);
  const float* gsc = gate_scale ? fwd->gate : nullptr;
  hipError_t e;
#define BWD_TRY(expr, what)                                    \
  do {                                                         \
    if ((e = (expr)) != hipSuccess) return hip_fail(e, what);  \
  } while (0)
  auto mark = [&](int i) -> hipError_t {
    return (ev != nullptr && ev[i] != nullptr) ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), st) : hipSuccess;
  };
  BWD_TRY(mark(0), "switch_moe_backward/event");
  if (L.fused) {
    ExpertBwdArgs A{};
    A.w1 = in->w1;
    A.w2 = in->w2;
    A.x = in->x;
    A.dy = dy;
    A.h = saved->h;
    A.gate = gsc;
    A.tos = tos;
    A.kept = kept;
    A.active = saved->active;
    A.n_active = saved->n_active;
    A.dz = dZ;
    A.dw1 = grads->dw1;
    A.dw2 = grads->dw2;
    A.dgp = reinterpret_cast<float*>(w + L.off_dg);
    A.dxe = dxe;
    A.T = T;
    A.N = N;
    A.C = C;
    A.d = dm;
    A.dff = dff;
    A.accum = accum ? 1 : 0;
    if (!accum) BWD_TRY(launch_zero_idle_experts(A, st), "switch_moe_backward/zero");
    BWD_TRY(mark(1), "switch_moe_backward/event");
    BWD_TRY(launch_expert_bwd_pass(A, 2, st), "switch_moe_backward/w2_pass");
    BWD_TRY(mark(2), "switch_moe_backward/event");
    BWD_TRY(launch_expert_bwd_pass(A, 1, st), "switch_moe_backward/w1_pass");
  } else {
  BWD_TRY(mark(1), "switch_moe_backward/event");
  // routed experts.  U = dY W2^T over each expert's kept tokens
  BWD_TRY(launch_gemm_generic(GemmOperand{dy, dm, 0, tos, nullptr, 0}, 0,
                              GemmOperand{in->w2, dm, (int64_t)dff * dm, nullptr, nullptr, 1},
                              GemmOut{U, dff, (int64_t)C * dff}, 1, dt, N, C, dff, dm, C, kept, 1, st),
          "switch_moe_backward/U");
  // dZ = s U [H > 0], dg = <U, H>
  BWD_TRY(launch_dz_rows(U, saved->h, dZ, dg, kept, tos, gsc, N, C, dff, dt, st), "switch_moe_backward/dZ");
  // dW2 = H^T (s dY)
  BWD_TRY(launch_gemm_generic(GemmOperand{saved->h, dff, (int64_t)C * dff, nullptr, nullptr, 1}, 0,
                              GemmOperand{dy, dm, 0, tos, gsc, 0}, GemmOut{grads->dw2, dm, (int64_t)dff * dm}, 0, dt,
                              N, dff, dm, C, C, kept, 2, st),
          "switch_moe_backward/dW2");
  BWD_TRY(mark(2), "switch_moe_backward/event");
  // dW1 = X^T dZ
  BWD_TRY(launch_gemm_generic(GemmOperand{in->x, dm, 0, tos, nullptr, 1}, 0,
                              GemmOperand{dZ, dff, (int64_t)C * dff, nullptr, nullptr, 0},
                              GemmOut{grads->dw1, dff, (int64_t)dm * dff}, 0, dt, N, dm, dff, C, C, kept, 2, st),
          "switch_moe_backward/dW1");
  // dX_e = dZ W1^T
  BWD_TRY(launch_gemm_generic(GemmOperand{dZ, dff, (int64_t)C * dff, nullptr, nullptr, 0}, 0,
                              GemmOperand{in->w1, dff, (int64_t)dm * dff, nullptr, nullptr, 1},
                              GemmOut{dxe, dm, (int64_t)C * dm}, 1, dt, N, C, dm, dff, C, kept, 1, st),
          "switch_moe_backward/dX");
  }
  BWD_TRY(mark(3), "switch_moe_backward/event");
  // shared dense expert on every token
  float* dxs = nullptr;
  if (d.d_ff_shared > 0) {
    const int dfs = d.d_ff_shared;
    int32_t* dk = reinterpret_cast<int32_t*>(w + L.off_dense);
    float* Us = reinterpret_cast<float*>(w + L.off_us);
    void* dZs = w + L.off_dzs;
    dxs = reinterpret_cast<float*>(w + L.off_dxs);
    if (dt == SWITCH_BF16 && dense_bwd_applies(T, dm, dfs)) {
      BWD_TRY(launch_shared_bwd_dense(in->x, dy, in->ws1, in->ws2, saved->h_shared, dZs, dxs, grads->dws1,
                                      grads->dws2, T, dm, dfs, st),
              "switch_moe_backward/shared_dense");
    } else {
    BWD_TRY(launch_dense_plan(dk, dk + 1, dk + 2, (int32_t)T, st), "switch_moe_backward/shared_plan");
    BWD_TRY(launch_gemm_generic(GemmOperand{dy, dm, 0, nullptr, nullptr, 0}, 0,
                                GemmOperand{in->ws2, dm, 0, nullptr, nullptr, 1}, GemmOut{Us, dfs, 0}, 1, dt, 1,
                                (int)T, dfs, dm, (int)T, nullptr, 0, st),
            "switch_moe_backward/shared_U");
    BWD_TRY(launch_dz_rows(Us, saved->h_shared, dZs, nullptr, dk, nullptr, nullptr, 1, (int)T, dfs, dt, st),
            "switch_moe_backward/shared_dZ");
    BWD_TRY(launch_gemm_generic(GemmOperand{saved->h_shared, dfs, 0, nullptr, nullptr, 1}, 0,
                                GemmOperand{dy, dm, 0, nullptr, nullptr, 0}, GemmOut{grads->dws2, dm, 0}, 0, dt, 1,
                                dfs, dm, (int)T, (int)T, nullptr, 0, st),
            "switch_moe_backward/shared_dW2");
    BWD_TRY(launch_gemm_generic(GemmOperand{in->x, dm, 0, nullptr, nullptr, 1}, 0,
                                GemmOperand{dZs, dfs, 0, nullptr, nullptr, 0}, GemmOut{grads->dws1, dfs, 0}, 0, dt, 1,
                                dm, dfs, (int)T, (int)T, nullptr, 0, st),
            "switch_moe_backward/shared_dW1");
    BWD_TRY(launch_gemm_generic(GemmOperand{dZs, dfs, 0, nullptr, nullptr, 0}, 0,
                                GemmOperand{in->ws1, dfs, 0, nullptr, nullptr, 1}, GemmOut{dxs, dm, 0}, 1, dt, 1,
                                (int)T, dm, dfs, (int)T, nullptr, 0, st),
            "switch_moe_backward/shared_dX");
    }
  }
  BWD_TRY(mark(4), "switch_moe_backward/event");
  // router: softmax gradient, dW_g = dlogit^T x, db, and dx
  BWD_TRY(launch_router_grad(saved->probs, fwd->expert_id, fwd->slot, dg, L.dg_parts, fwd->f, dl_aux, T, N, C,
                             dlogit, st),
          "switch_moe_backward/router");
  if (grads->dbias != nullptr)
    BWD_TRY(launch_colsum(dlogit, T, N, reinterpret_cast<float*>(w + L.off_colsum), grads->dbias, st),
            "switch_moe_backward/db");
  const int residual_all = (d.flags & SWITCH_RESIDUAL_ALL) != 0;
  if (dt == SWITCH_BF16) {
    BWD_TRY(launch_router_bwd_mfma(L.rp, dlogit, in->x, in->w_gate, dxe, dy, dxs, fwd->expert_id, fwd->slot, T, dm,
                                   N, C, residual_all, reinterpret_cast<uint16_t*>(w + L.off_hi),
                                   reinterpret_cast<uint16_t*>(w + L.off_lo), reinterpret_cast<float*>(w + L.off_rpart),
                                   grads->dw_gate, grads->dx, st),
            "switch_moe_backward/router_mfma");
  } else {
    BWD_TRY(launch_gemm_generic(GemmOperand{dlogit, N, 0, nullptr, nullptr, 1}, 1,
                                GemmOperand{in->x, dm, 0, nullptr, nullptr, 0}, GemmOut{grads->dw_gate, dm, 0}, 1, dt,
                                1, N, dm, (int)T, (int)T, nullptr, 0, st),
            "switch_moe_backward/dW_g");
    BWD_TRY(launch_dx_assemble(dlogit, in->w_gate, dxe, dy, dxs, fwd->expert_id, fwd->slot, T, dm, N, C,
                               residual_all, grads->dx, dt, st),
            "switch_moe_backward/dx");
  }
  BWD_TRY(mark(5), "switch_moe_backward/event");
#undef BWD_TRY
  return ok();
}

extern "C" {

switch_status switch_moe_backward(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                  const switch_moe_outputs* fwd, const switch_moe_saved* saved, const void* dy,
                                  const float* dl_aux, const switch_moe_grads* grads, void* ws, size_t ws_bytes,
                                  void* stream) {
  return moe_backward(desc, in, fwd, saved, dy, dl_aux, grads, ws, ws_bytes, stream, nullptr);
}

switch_status switch_moe_backward_timed(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                        const switch_moe_outputs* fwd, const switch_moe_saved* saved,
                                        const void* dy, const float* dl_aux, const switch_moe_grads* grads, void* ws,
                                        size_t ws_bytes, void* stream, void* const* stage_events) {
  if (stage_events == nullptr) return fail(SWITCH_E_NULL, "stage_events is NULL");
  return moe_backward(desc, in, fwd, saved, dy, dl_aux, grads, ws, ws_bytes, stream, stage_events);
}

const char* switch_status_str(switch_status s) {
  switch (s) {
    case SWITCH_OK: return "ok";
    case SWITCH_E_NULL: return "null pointer";
    case SWITCH_E_SHAPE: return "invalid shape";
    case SWITCH_E_UNSUPPORTED: return "unsupported value";
    case SWITCH_E_WORKSPACE: return "workspace too small";
    case SWITCH_E_HIP: return "HIP launch failure";
    case SWITCH_E_ALIGN: return "misaligned pointer";
  }
  return "unknown status";
}

const char* switch_last_error(void) { return g_err; }

}  // extern "C"
