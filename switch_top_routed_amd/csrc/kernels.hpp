// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Every launcher enqueues on `stream` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "switch_moe.h"

namespace swm {

// ---------------- router ----------------
struct RoutePlan {
  int split;        // 0: fused kernel; >0: number of k-chunks of the split path
  int tm;           // 16-token tiles per workgroup (fused path)
  bool kslice;      // fused path with the 4 waves splitting K (long rows, N <= 128)
  int tile_rows;    // tokens per workgroup (= per partial row)
  int64_t nblk;     // number of per-workgroup partial rows
  size_t off_part_p, off_part_cnt, off_logits, off_wgf, bytes;
};
RoutePlan route_plan(int64_t T, int d, int N, int dtype);
// stats_later == false: statistics (routed_count, f, P, l_aux) by a final
// reduction kernel; true: they are left to launch_assign_token
// Router options beyond top-1:
//   probs != NULL: the softmax of every token is written too ([T, N] fp32);
//   K > 1: top-K choices, expert_id / gate are [T, K] (t * K + j), routed_count
//          counts all K T assignments and f_i = count_i / (K T); renorm divides
//          each token's K gates by their sum;
//   ev_cm / gv_cm != NULL: the choices and gates also in choice-major order
//          ([K, T]: j * T + t), the "virtual token" list the slot assignment ranks.
constexpr int kMaxTopK = 8;
struct RouteExtra {
  float* probs = nullptr;
  float* probs_t = nullptr;  // the softmax transposed, [N, T] (expert choice)
  int K = 1;
  int renorm = 0;
  int32_t* ev_cm = nullptr;
  float* gv_cm = nullptr;
  int expand = 0;  // K choices are Expanded Drop candidates: stats, expert_id and gate stay top-1
};
hipError_t launch_route(const RoutePlan& pl, const void* x, const void* wg, const float* bias, int64_t T, int d, int N,
                        int dtype, int32_t* expert_id, float* gate, int32_t* routed_count, float* f, float* P,
                        float* l_aux, char* ws, hipStream_t st, bool stats_later = false,
                        const RouteExtra& ex = RouteExtra{});
// token-order slots and the router statistics (after launch_route with
// stats_later): one workgroup per expert, then one for the cross-expert
// results; term: fp64 [N] scratch
// (K > 1: expert_id is the choice-major [K, T] list, slot is [T, K])
// finalize == false: the cross-expert results are left to the first GEMM (ActiveFromKept)
hipError_t launch_assign_token(const RoutePlan& pl, int64_t T, int K, int N, int C, const int32_t* expert_id, double* term,
                               int32_t* routed_count, float* f, float* P, float* l_aux, int32_t* slot,
                               int32_t* token_of_slot, int32_t* kept_count, int32_t* n_dropped, int32_t* active,
                               int32_t* n_active, char* ws, hipStream_t st, bool finalize = true);

// ---------------- capacity / slots ----------------
struct AssignPlan {
  int64_t nblk;  // 256-token blocks
  size_t off_blockcount, off_blockoff, off_local_rank, off_total, off_seg_start, off_perm, off_keys, bytes;
};
AssignPlan assign_plan(int64_t T, int N, int C, int priority);
hipError_t launch_assign(const AssignPlan& pl, const int32_t* expert_id, const float* gate, int64_t T, int N, int C,
                         int priority, int32_t* slot, int32_t* token_of_slot, int32_t* kept_count,
                         int32_t* n_dropped, int32_t* active, int32_t* n_active, char* ws, hipStream_t st);

// ---------------- dispatch / combine ----------------
hipError_t launch_dispatch(const void* x, int dtype, int64_t T, int d, const int32_t* token_of_slot,
                           const int32_t* kept_count, int N, int C, void* expert_in, hipStream_t st);
hipError_t launch_combine(const void* expert_out, const void* x, const void* shared_out, int dtype, int64_t T, int d,
                          const int32_t* expert_id, const int32_t* slot, const float* gate, int N, int C,
                          uint32_t flags, void* y, hipStream_t st);

// ---------------- expert FFN ----------------
// MXFP4 expert weights (codes [N][Ncols][K/2], E8M0 scales [N][Ncols][K/32] for
// W1 (K = d, Ncols = d_ff) and W2 (K = d_ff, Ncols = d)); bf16 activations
struct MxWeights {
  const uint8_t *w1_codes, *w1_scales, *w2_codes, *w2_scales;
};
struct FfnPlan {
  int mt;    // 16-row tiles per work item (bf16 path)
  int mch;   // m-chunks per expert
  int grid;  // persistent workgroups
  int h_tiles;  // > 0: the workspace hidden matrix is fragment-blocked, h_tiles 16-row tiles per expert
  size_t off_h, bytes;
};
FfnPlan ffn_plan(int N, int C, int d, int dff, int dtype);
// two launches of one kernel (phase 1: H = ReLU(X W1), phase 2: Y = H W2).
// gather != NULL: xin is the token matrix [a_rows, d] and row r of expert e is
// token gather[e * C + r] (token_of_slot), so no dispatched copy is needed.
// h_out != NULL: the hidden activation [N, C, dff] goes there instead of the
// workspace (kept for the backward pass).
// The cross-expert results of the token-order assignment, built by every
// workgroup of the first GEMM from the kept counts instead of by a kernel of
// their own (streaming bf16 GEMMs only, ffn_stream_applies): the active list
// in expert order and n_active (workgroup 0 writes both for the second GEMM),
// n_dropped = TV - sum of kept counts, and L_aux = N sum_i f_i P_i through
// route_finalize's tree.  kept == NULL: off (active / n_active are read).
struct ActiveFromKept {
  const int32_t* kept = nullptr;
  const double* term = nullptr;  // f_i P_i [N]
  int32_t* active = nullptr;
  int32_t* n_active = nullptr;
  int32_t* n_dropped = nullptr;
  float* l_aux = nullptr;
  int64_t TV = 0;  // choices in the assignment list (T K)
};
// The top-1 combine (combine_rows' arithmetic) done by the shared expert's
// second GEMM as it writes each row of its output S: y[t] = (x[t] if the token
// was dropped or RESIDUAL_ALL) + (s_t o_t if kept) + S[t], with o_t the routed
// expert's output row.  y == NULL: off (the GEMM writes S).
struct CombineArgs {
  const uint16_t* eo = nullptr;  // routed expert outputs [N][C][d]
  const uint16_t* x = nullptr;   // token rows [T][d]
  const int32_t* expert_id = nullptr;
  const int32_t* slot = nullptr;
  const float* gate = nullptr;
  int N = 0, C = 0;
  uint32_t flags = 0;
  uint16_t* y = nullptr;  // [T][d]
};
bool ffn_stream_applies(int dtype, int C, int d, int dff, bool mx);
hipError_t launch_ffn(const FfnPlan& pl, const void* xin, const void* w1, const void* w2, int dtype, int N, int C, int d,
                      int dff, const int32_t* kept_count, const int32_t* active, const int32_t* n_active, void* xout,
                      char* ws, hipStream_t st, const int32_t* gather = nullptr, int64_t a_rows = 0,
                      void* h_out = nullptr, const MxWeights* mx = nullptr, const ActiveFromKept* afk = nullptr,
                      const CombineArgs* cmb = nullptr);
bool mx_ffn_applies(int C, int d, int dff);
hipError_t launch_ffn_mx(const void* xin, const MxWeights& mw, int N, int C, int d, int dff,
                         const int32_t* kept_count, const int32_t* active, const int32_t* n_active, void* xout,
                         void* h, hipStream_t st, const int32_t* gather, int64_t a_rows,
                         const ActiveFromKept& afk);
hipError_t launch_mx_quantize(const void* w, int dtype, int64_t batches, int K, int Ncols, uint8_t* codes,
                              uint8_t* scales, hipStream_t st);
// writes {M}, {0}, {1} for the dense (shared-expert) FFN
// LDS-tiled MFMA GEMM (direct global-to-LDS loads, transposing LDS reads) for
// experts with more than 64 rows and the dense shared FFN
bool tiled_ffn_applies(int C, int d, int dff);
hipError_t launch_tiled_dma(const void* A, const void* W, void* out, const int32_t* kept, const int32_t* active,
                            const int32_t* n_active, int N, int C, int K, int Ncols, int relu, hipStream_t st,
                            const int32_t* gather = nullptr, int64_t a_rows = 0, const CombineArgs* cmb = nullptr);
hipError_t launch_dense_plan(int32_t* kept, int32_t* active, int32_t* n_active, int32_t M, hipStream_t st);

// ---------------- backward ----------------
// operand of the generic GEMM: element (i, j) of batch b is
// ptr[(gather ? gather[b * C + i] : b * bstride-offset + i) * ld + j], times
// row_scale[physical row] when row_scale != NULL; trans swaps the roles of
// (i, j) (see gemm_generic)
struct GemmOperand {
  const void* ptr;
  int64_t ld, bstride;
  const int32_t* gather;
  const float* row_scale;
  int trans;
};
struct GemmOut {
  void* ptr;
  int64_t ld, bstride;
};
// extent: 0 fixed sizes, 1 rows M_b = min(kept[b], C), 2 reduction K_b = min(kept[b], C)
hipError_t launch_gemm_generic(const GemmOperand& a, int a_f32, const GemmOperand& b, const GemmOut& o, int o_f32,
                               int dtype, int batches, int M, int Nn, int K, int C, const int32_t* kept, int extent,
                               hipStream_t st);
hipError_t launch_dz_rows(const float* U, const void* H, void* dZ, float* dg, const int32_t* kept,
                          const int32_t* tos, const float* gate, int N, int C, int dff, int dtype, hipStream_t st);
// dg: per-slot partial sums [N*C][nparts] of dgate (NULL: no gate gradient)
hipError_t launch_router_grad(const float* probs, const int32_t* eid, const int32_t* slot, const float* dg,
                              int nparts, const float* f, const float* dl_aux, int64_t T, int N, int C,
                              float* dlogit, hipStream_t st);
size_t colsum_scratch_bytes(int64_t T, int N);
hipError_t launch_colsum(const float* a, int64_t T, int N, float* scratch, float* out, hipStream_t st);
hipError_t launch_dx_assemble(const float* dlogit, const void* wg, const float* dxe, const void* dy, const float* dxs,
                              const int32_t* eid, const int32_t* slot, int64_t T, int d, int N, int C,
                              int residual_all, void* dx, int dtype, hipStream_t st);

// fused MFMA expert backward (bf16): pass over W2 (U, dZ, dg partials, dW2),
// then over W1 (dX_e, dW1); experts that kept no token get zero gradients
struct ExpertBwdArgs {
  const void *w1, *w2, *x, *dy, *h;
  const float* gate;  // per-token gate scale, or NULL (scaling off)
  const int32_t *tos, *kept, *active, *n_active;
  void *dz, *dw1, *dw2;
  float *dgp, *dxe;   // dg partials [N*C][d_ff/64]; dX_e [N][C][d]
  int64_t T;
  int N, C, d, dff;
  int accum = 0;      // add the weight gradients to dw1 / dw2 (idle experts untouched)
};
bool fused_expert_bwd_applies(int64_t T, int C, int d, int dff);
hipError_t launch_zero_idle_experts(const ExpertBwdArgs& a, hipStream_t st);
// which = 2: pass over W2 (dZ, dg partials, dW2); 1: pass over W1 (dX_e, dW1)
hipError_t launch_expert_bwd_pass(const ExpertBwdArgs& a, int which, hipStream_t st);

// router backward on MFMA (bf16 layers): dlogit split into bf16 hi / lo planes
// [T][NP], dW_g from per-chunk partials [S][N][d], dx assembled with the expert,
// pass-through and shared terms
struct RouterBwdPlan {
  int NP, TC, S;  // experts padded to 64; tokens per chunk; chunks
  size_t planes_bytes, partial_bytes;  // one plane; all partials
};
RouterBwdPlan router_bwd_plan(int64_t T, int N, int d);
hipError_t launch_router_bwd_mfma(const RouterBwdPlan& p, const float* dlogit, const void* x, const void* wg,
                                  const float* dxe, const void* dy, const float* dxs, const int32_t* eid,
                                  const int32_t* slot, int64_t T, int d, int N, int C, int residual_all,
                                  uint16_t* hi, uint16_t* lo, float* partial, float* dw_gate, void* dx,
                                  hipStream_t st);

// ---------------- routing variants ----------------
// top-K: slots [T, K] from the ranks of the virtual-token list; token_of_slot
// virtual indices -> token rows (in place)
hipError_t launch_topk_fixup(const int32_t* slot_v, int64_t T, int K, int32_t* tos, int64_t NC, int32_t* slot,
                             hipStream_t st);
// expert choice: each expert's min(C, T) highest-probability tokens from the
// transposed softmax; pick [T, N] (slot or -1), n_dropped zeroed for the combine
constexpr int kMaxExpertChoiceK = 8192;
hipError_t launch_ec_select(const float* probs_t, int64_t T, int N, int C, int32_t* tos, int32_t* pick,
                            int32_t* kept_count, int32_t* active, int32_t* n_active, int32_t* n_dropped,
                            hipStream_t st);
// combine over each token's picks: mode 0 top-K ([T, K] ids, slots, gates),
// mode 1 expert choice (pick [T, N], gates from probs_t; writes npick [T] and
// counts unpicked tokens into n_dropped)
hipError_t launch_combine_picks(int mode, const void* expert_out, const void* x, const void* shared_out, int dtype,
                                int64_t T, int d, int K, const int32_t* eid, const int32_t* slot, const float* gate,
                                const int32_t* pick, const float* probs_t, int N, int C, uint32_t flags,
                                int32_t* npick, int32_t* n_dropped, void* y, hipStream_t st);

// Expanded Drop: rounds 1 .. M-1 over the candidates ev_cm / gv_cm [M, T]
// after the top-1 assignment (slot, token_of_slot, kept_count in place;
// expert_id / gate rewritten for re-routed tokens), then active, n_active and
// n_dropped.  list: workspace [N, T] int32.  C <= kMaxExpertChoiceK.
hipError_t launch_expand(const int32_t* ev_cm, const float* gv_cm, int64_t T, int N, int C, int M, int gate_order,
                         int32_t* slot, int32_t* expert_id, float* gate, int32_t* tos, int32_t* kept_count,
                         int32_t* active, int32_t* n_active, int32_t* n_dropped, int32_t* list, hipStream_t st,
                         const double* term = nullptr, float* l_aux = nullptr);

// shared dense expert backward on LDS-tiled MFMA (bf16): dZs = (dY Ws2^T) *
// [Hs > 0], dWs2 = Hs^T dY, dWs1 = x^T dZs, dXs = dZs Ws1^T (fp32)
bool dense_bwd_applies(int64_t T, int d, int dffs);
hipError_t launch_shared_bwd_dense(const void* x, const void* dy, const void* ws1, const void* ws2, const void* hs,
                                   void* dzs, float* dxs, void* dws1, void* dws2, int64_t T, int d, int dffs,
                                   hipStream_t st);

inline size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

// ---------------- C ABI internals shared by the entry-point sources ----------------
// switch_moe_forward itself (validation, then the launches on `ws`)
switch_status abi_forward(const switch_moe_desc* desc, const switch_moe_inputs* in, const switch_moe_outputs* out,
                          void* ws, size_t ws_bytes, void* stream);
// validates desc; *bytes = the forward's workspace size
switch_status abi_forward_bytes(const switch_moe_desc* desc, size_t* bytes);
// sets the thread-local message of switch_last_error and returns s
switch_status abi_fail(switch_status s, const char* msg);

}  // namespace swm
