/*
 * switch_moe.h -- C ABI of a Switch top-1 mixture-of-experts layer (forward
 * and backward) for AMD Instinct MI355X (gfx950), one GPU, every expert
 * resident.
 *
 * Sources for the operations (page title, then section):
 *   [TOP1] "Top-1 Routing" concept page (compassingai.com): Core mechanism,
 *          Load balancing, Token Dropping, Key parameters and compute.
 *   [SWT]  Switch Transformers summary page (personwebsite.pages.dev,
 *          moe-switch): Switch-layer passage (k = 1, gate value as the
 *          multiplier), expert-capacity passage, Eq. 4 auxiliary loss
 *          passage, selective-precision passage.
 *   [CAP]  "MoE expert capacity factor and token dropping" (wiblog.cn):
 *          Where capacity comes from, After overflow, training-step
 *          flowchart, inference section (Expanded Drop).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers; the descriptor structs and scalar
 *     arguments live on the host.  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream).  Every call only enqueues work on
 *     `stream` and returns; nothing is synchronised and nothing is copied to
 *     the host.
 *   - The caller owns every buffer (inputs, outputs and workspace).  The
 *     library never allocates or frees memory and keeps no state between
 *     calls.  Inputs are read only.  Workspace contents are undefined on
 *     entry and on return.
 *   - Layouts are row-major: x [T, d_model]; w_gate [N, d_model];
 *     w1 [N, d_model, d_ff]; w2 [N, d_ff, d_model]; expert buffers
 *     [N, C, d_model]; y [T, d_model]; shared ws1 [d_model, d_ff_s],
 *     ws2 [d_ff_s, d_model].
 *   - dtype: SWITCH_F32 (float) or SWITCH_BF16 (bfloat16 storage with fp32
 *     arithmetic inside every kernel).  The router always computes in fp32
 *     and returns fp32 gates ([SWT] selective precision).
 *   - Errors: validation runs before any launch, so an error return other
 *     than SWITCH_E_HIP enqueues no work.  SWITCH_E_HIP means a launch
 *     failed; outputs are then undefined.  switch_last_error() returns a
 *     thread-local message describing the last failure.  No C++ exception
 *     crosses the ABI.
 *   - Shape rules: T >= 1; 1 <= N <= 1024; 1 <= C <= T; pointers 16-byte
 *     aligned.  bf16: d_model and d_ff multiples of 128.  f32: d_model a
 *     multiple of 4.  d_model <= 2^20 and d_model * d_ff <= 2^30 (one
 *     expert's weight matrix stays under 2 GiB in bf16: the kernels address
 *     it through 32-bit buffer offsets).
 *   - Determinism: identical inputs give bitwise identical outputs (no
 *     floating-point atomics; every reduction has a fixed order).
 */
#ifndef SWITCH_MOE_H
#define SWITCH_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum switch_status {
  SWITCH_OK = 0,
  SWITCH_E_NULL = 1,        /* a required pointer is NULL */
  SWITCH_E_SHAPE = 2,       /* a size violates the shape rules */
  SWITCH_E_UNSUPPORTED = 3, /* dtype / priority / flag value not supported */
  SWITCH_E_WORKSPACE = 4,   /* workspace smaller than the *_workspace_bytes figure */
  SWITCH_E_HIP = 5,         /* a HIP launch failed */
  SWITCH_E_ALIGN = 6        /* a pointer is not 16-byte aligned */
} switch_status;

typedef enum switch_dtype { SWITCH_F32 = 0, SWITCH_BF16 = 1 } switch_dtype;

/* Overflow priority inside one expert ([CAP] After overflow and flowchart;
 * token order is the plain reading of "the excess tokens" in [TOP1]
 * Token Dropping). */
typedef enum switch_priority {
  SWITCH_TOKEN_ORDER = 0, /* earlier tokens first */
  SWITCH_GATE_DESC = 1    /* higher gate first; equal gates: earlier token first */
} switch_priority;

/* Combine flags.  SWITCH_GATE_SCALE: y = gate * E(x) ([SWT] Switch-layer
 * passage); without it y = E(x) ([TOP1] Core mechanism).  The pages
 * disagree, so this is a flag.  SWITCH_RESIDUAL_ALL: kept tokens also get
 * + x (the Transformer residual around the layer, [TOP1] MoE layer figure).
 * Dropped tokens always get y = x. */
#define SWITCH_GATE_SCALE 1u
#define SWITCH_RESIDUAL_ALL 2u
/* Top-K only: divide each token's K gates by their sum (the gate of choice j
 * is otherwise p[t, e_tj], the top-1 definition applied to every choice). */
#define SWITCH_RENORM 4u
/* Backward only: the routed experts' weight gradients accumulate into the
 * caller's dw1 / dw2 (dW[e] += dL/dW[e], the fp32 sum of the stored bf16
 * value and the new one, rounded once) instead of overwriting them.  An
 * expert that kept no token has a zero gradient and is not touched at all,
 * which spares a layer with many idle experts (the 384-expert decode batch)
 * the write of their zeros.  Gradient accumulation over several batches is
 * the use ([CAP] training-step flowchart: the step backpropagates into the
 * experts); every other output is written as without the flag.  Needs the
 * fused bf16 expert backward (C <= 160, d_model and d_ff multiples of 64):
 * otherwise switch_moe_backward returns SWITCH_E_UNSUPPORTED.  The forward
 * ignores it. */
#define SWITCH_ACCUM_EXPERT_GRADS 8u

/* Routing ("Top-1 Routing" page, Variants: token choice, where each token
 * picks its top-K experts, and expert choice, where each expert picks its top
 * tokens and is balanced by construction). */
typedef enum switch_routing {
  SWITCH_TOKEN_CHOICE = 0,  /* top-K, K = desc.top_k (0 or 1: the Switch top-1 layer) */
  SWITCH_EXPERT_CHOICE = 1  /* expert i takes the min(C, T) tokens with the highest p[t, i] */
} switch_routing;

/* ------------------------------------------------------------------------
 * Capacity ([TOP1] Token Dropping; [SWT] expert capacity; [CAP] Where
 * capacity comes from): C = max(1, ceil(capacity_factor * T / N)), clamped
 * to T.  capacity_factor is taken at its decimal value (the shortest decimal
 * string that reads back as the same double), and the ceiling is exact: 1.1
 * with T = 100, N = 10 gives 11, not the 12 that double arithmetic rounds to.
 * Host-only.  Returns -1 if T < 1, N < 1 or capacity_factor is not a finite
 * value > 0.
 * ---------------------------------------------------------------------- */
int32_t switch_capacity(int64_t T, int32_t N, double capacity_factor);

/* ------------------------------------------------------------------------
 * Router ([TOP1] Core mechanism and Load balancing; [SWT] Switch layer,
 * Eq. 4 passage, selective precision).
 *   logits l[t,i] = sum_k w_gate[i,k] x[t,k] + bias[i]   (fp32)
 *   p = softmax_i(l);  expert_id[t] = argmax_i l[t,i] (lowest index on ties);
 *   gate[t] = p[t, expert_id[t]]
 *   routed_count[i] = #{t : expert_id[t] = i};  f[i] = routed_count[i] / T
 *   P[i] = (1/T) sum_t p[t,i];  l_aux[0] = N * sum_i f[i] P[i]
 * x, w_gate: dtype; bias: fp32 [N] or NULL; outputs: expert_id int32 [T],
 * gate fp32 [T], routed_count int32 [N], f fp32 [N], P fp32 [N], l_aux fp32
 * [1].  f counts argmax decisions before any capacity cut; l_aux excludes
 * the training coefficient alpha.
 * ---------------------------------------------------------------------- */
size_t switch_route_workspace_bytes(int64_t T, int32_t d_model, int32_t N, int32_t dtype);
switch_status switch_route(const void* x, const void* w_gate, const float* bias, int64_t T, int32_t d_model,
                           int32_t N, int32_t dtype, int32_t* expert_id, float* gate, int32_t* routed_count,
                           float* f, float* P, float* l_aux, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Capacity / slot assignment ([CAP] After overflow and flowchart steps
 * C-F; [TOP1] Token Dropping).  Each token's rank among the tokens routed
 * to its expert under `priority`; kept iff rank < C.
 *   slot[t] = rank if kept else -1                       int32 [T]
 *   token_of_slot[e*C + s] = token in slot s, -1 if empty int32 [N*C]
 *   kept_count[e] = min(routed_count[e], C)              int32 [N]
 *   n_dropped[0] = T - sum_e kept_count[e]               int32 [1]
 *   active[0..n_active) = experts with kept_count > 0, ascending; rest
 *   undefined                                            int32 [N]
 *   n_active[0]                                          int32 [1]
 * gate (fp32 [T]) is read only for SWITCH_GATE_DESC (may be NULL for
 * token order).  Integer results are exact.
 * ---------------------------------------------------------------------- */
size_t switch_assign_workspace_bytes(int64_t T, int32_t N, int32_t C, int32_t priority);
switch_status switch_assign_capacity(const int32_t* expert_id, const float* gate, int64_t T, int32_t N, int32_t C,
                                     int32_t priority, int32_t* slot, int32_t* token_of_slot, int32_t* kept_count,
                                     int32_t* n_dropped, int32_t* active, int32_t* n_active, void* ws,
                                     size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Dispatch into fixed per-expert buffers ([CAP] Where capacity comes from:
 * fixed slots turn dynamic routing into static shapes).
 *   expert_in[e, s, :] = x[token_of_slot[e*C+s], :]  for s < kept_count[e]
 * Rows s >= kept_count[e] are not written.  Bit copy.
 * ---------------------------------------------------------------------- */
switch_status switch_dispatch(const void* x, int32_t dtype, int64_t T, int32_t d_model, const int32_t* token_of_slot,
                              const int32_t* kept_count, int32_t N, int32_t C, void* expert_in, void* stream);

/* ------------------------------------------------------------------------
 * Expert FFN ([TOP1] Key parameters and compute: two-layer FFN, biases
 * ignored; ReLU activation).
 *   expert_out[e, s, :] = ReLU(expert_in[e, s, :] . w1[e]) . w2[e]
 * for e in active[0..n_active) and s < kept_count[e].  Empty slots and
 * inactive experts are never read (their weights are not touched); rows
 * s >= kept_count[e] of expert_out are not written.  bf16: the hidden
 * activation is rounded to bf16 between the two GEMMs, both accumulate in
 * fp32, the output is rounded once to bf16.
 * A dense FFN over M rows is the case N = 1, C = M, kept_count = {M},
 * active = {0}, n_active = {1}.
 * ---------------------------------------------------------------------- */
size_t switch_expert_ffn_workspace_bytes(int32_t N, int32_t C, int32_t d_model, int32_t d_ff, int32_t dtype);
switch_status switch_expert_ffn(const void* expert_in, const void* w1, const void* w2, int32_t dtype, int32_t N,
                                int32_t C, int32_t d_model, int32_t d_ff, const int32_t* kept_count,
                                const int32_t* active, const int32_t* n_active, void* expert_out, void* ws,
                                size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Combine ([TOP1] Core mechanism; [SWT] Switch-layer passage; dropped
 * tokens: [TOP1] Token Dropping, [SWT] expert capacity, [CAP] After
 * overflow, residual bypass).
 *   kept t (slot[t] >= 0): y[t] = (flags & GATE_SCALE ? gate[t] : 1) *
 *        expert_out[expert_id[t], slot[t]] (+ x[t] if RESIDUAL_ALL)
 *   dropped t:             y[t] = x[t]
 *   and + shared_out[t] for every t when shared_out != NULL.
 * Arithmetic in fp32, rounded once to dtype; a dropped row without a
 * shared term is a bit copy.
 * ---------------------------------------------------------------------- */
switch_status switch_combine(const void* expert_out, const void* x, const void* shared_out, int32_t dtype, int64_t T,
                             int32_t d_model, const int32_t* expert_id, const int32_t* slot, const float* gate,
                             int32_t N, int32_t C, uint32_t flags, void* y, void* stream);

/* ------------------------------------------------------------------------
 * MXFP4 expert weights (the open-MoE routing comparison page: gpt-oss ships
 * its MoE weights in MXFP4 to fit one GPU; format: OCP Microscaling v1.0).
 * Blocks of 32 consecutive elements along the GEMM's reduction dimension share
 * one E8M0 scale byte (2^(byte - 127)); elements are FP4 E2M1 codes, two per
 * byte, the lower index in the low nibble.  Quantization: E = clamp(floor(
 * log2(max |v|)) - 2, -127, 127) (-127 for an all-zero block); each v / 2^E
 * rounds to the nearest E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the
 * even mantissa, saturating at 6; the sign bit is the sign of v.
 * ---------------------------------------------------------------------- */
typedef enum switch_weight_format {
  SWITCH_WEIGHTS_NATIVE = 0, /* w1 / w2 in the layer dtype */
  SWITCH_WEIGHTS_MXFP4 = 1   /* w1 / w2 MXFP4 codes + scales; bf16 layers with C <= 64, forward only */
} switch_weight_format;

/* Quantize w [batches, K, Ncols] (dtype) along K:
 *   codes [batches, Ncols, K/2] (bytes), scales [batches, Ncols, K/32].
 * K must be a multiple of 128 and at most 2^21.  For the experts: w1 with
 * K = d_model, Ncols = d_ff; w2 with K = d_ff, Ncols = d_model.  Bit-exact and
 * deterministic. */
switch_status switch_quantize_mxfp4(const void* w, int32_t dtype, int64_t batches, int32_t K, int32_t Ncols,
                                    uint8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------
 * The whole layer: route -> capacity/slots -> dispatch -> expert FFN ->
 * (shared FFN) -> combine, enqueued on one stream.  Results equal those of
 * the per-stage entry points above, bit for bit.  When
 * T * d_model * sizeof(dtype) < 2^31 the first expert GEMM reads each slot's
 * token row from x through token_of_slot, so no dispatched copy is made (every
 * routing); with token-order priority the slots also come from one workgroup
 * per expert right after the router, while gate-descending priority runs the
 * assignment kernels of switch_assign_capacity.
 * ---------------------------------------------------------------------- */
typedef struct switch_moe_desc {
  int64_t T;
  int32_t d_model;
  int32_t d_ff;
  int32_t N;
  int32_t C;                /* 0: derive from capacity_factor */
  double capacity_factor;
  int32_t dtype;            /* switch_dtype */
  int32_t priority;         /* switch_priority */
  uint32_t flags;           /* SWITCH_GATE_SCALE | SWITCH_RESIDUAL_ALL */
  int32_t d_ff_shared;      /* 0: no shared expert; else one always-on dense
                               FFN added to every token ([TOP1] History,
                               shared experts) */
  int32_t top_k;            /* token choice: experts per token, 0 or 1 = top-1,
                               at most 8 and at most N */
  int32_t routing;          /* switch_routing */
  int32_t weight_format;    /* switch_weight_format of w1 / w2 */
  int32_t expand_choices;   /* Expanded Drop: 0 or 1 = off; M in [2, min(N, 8)]
                               = re-route overflow tokens over their M
                               highest-logit experts (top-1 token choice only) */
} switch_moe_desc;

typedef struct switch_moe_inputs {
  const void* x;
  const void* w_gate;
  const float* bias; /* NULL: no router bias */
  const void* w1;    /* dtype [N, d_model, d_ff]; MXFP4: codes [N, d_ff, d_model/2] */
  const void* w2;    /* dtype [N, d_ff, d_model]; MXFP4: codes [N, d_model, d_ff/2] */
  const void* ws1;   /* shared expert, only if d_ff_shared > 0 (always dtype) */
  const void* ws2;
  const uint8_t* w1_scale; /* MXFP4 only: E8M0 [N, d_ff, d_model/32] */
  const uint8_t* w2_scale; /* MXFP4 only: E8M0 [N, d_model, d_ff/32] */
} switch_moe_inputs;

typedef struct switch_moe_outputs {
  void* y;               /* [T, d_model] dtype (required) */
  int32_t* expert_id;    /* [T] (required) */
  float* gate;           /* [T] (required) */
  int32_t* slot;         /* [T] (required) */
  int32_t* routed_count; /* [N] (required) */
  int32_t* kept_count;   /* [N] (required) */
  int32_t* n_dropped;    /* [1] (required) */
  float* f;              /* [N] (required) */
  float* P;              /* [N] (required) */
  float* l_aux;          /* [1] (required) */
} switch_moe_outputs;

size_t switch_moe_workspace_bytes(const switch_moe_desc* desc);
switch_status switch_moe_forward(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                 const switch_moe_outputs* out, void* ws, size_t ws_bytes, void* stream);

/* Routing variants of switch_moe_forward (desc.top_k > 1, or desc.routing =
 * SWITCH_EXPERT_CHOICE).  Capacity, buffers, the expert FFN and the shared
 * expert are those of the top-1 layer.
 *   Top-K token choice: each token's K highest logits (ties to the lower
 *   index), gate_tj = p[t, e_tj] (SWITCH_RENORM: divided by the token's K-gate
 *   sum).  C = min(T, max(1, ceil(capacity_factor * K * T / N))) unless
 *   desc.C is set.  The K T assignments are ranked inside each expert as one
 *   list ordered j * T + t (every first choice before every second choice;
 *   SWITCH_GATE_DESC: by descending gate, ties in that order).  Outputs:
 *   expert_id, gate and slot hold [T, K] (choice j of token t at t * K + j);
 *   routed_count counts all K T assignments, f_i = routed_count_i / (K T),
 *   P and l_aux as for top-1; n_dropped counts dropped assignments.
 *   y_t = sum over the token's kept assignments of (gate-scale ? gate : 1) *
 *   E(x_t) (+ x_t with SWITCH_RESIDUAL_ALL); a token with no kept assignment
 *   passes through (y_t = x_t).
 *   Expert choice: C = max(1, ceil(capacity_factor * T / N)) unless desc.C
 *   is set (min(C, T) <= 8192); expert i takes the min(C, T) tokens with the
 *   highest p[t, i] (ties to the lower token) into slots by descending p.
 *   y_t = sum over the experts that took t of (gate-scale ? p[t, i] : 1) *
 *   E_i(x_t) (+ x_t with SWITCH_RESIDUAL_ALL); a token no expert took passes
 *   through.  Outputs: expert_id, gate, routed_count, f, P, l_aux are the
 *   argmax (top-1) statistics of the same router; kept_count[i] = min(C, T);
 *   slot[t] = the number of experts that took token t; n_dropped = the
 *   number of tokens no expert took.
 *   Expanded Drop (desc.expand_choices = M >= 2; [CAP] inference section:
 *   overflow tokens of full experts consider further experts of their
 *   candidate set, so that lightly loaded experts' spare capacity is used).
 *   Top-1 token choice with capacity C = max(1, ceil(capacity_factor * T /
 *   N)) unless desc.C is set (C <= 8192).  A token's candidates are its M
 *   highest logits (ties to the lower index).  Round 0 is the top-1
 *   assignment; in round r = 1 .. M-1 every token still without a slot
 *   applies to its candidate r, and expert i fills its C - kept_i free slots
 *   with that round's applicants in the priority order (token order: by
 *   token index; SWITCH_GATE_DESC: by descending p[t, i], ties to the lower
 *   token), after the slots already taken.  Outputs: expert_id, gate and slot
 *   name the expert holding the token, p at that expert and the slot (a
 *   token no candidate took keeps its first choice with slot -1 and passes
 *   through); kept_count, n_dropped as after the last round; routed_count, f,
 *   P, l_aux are the first-choice (top-1) statistics.  SWITCH_RENORM is not
 *   accepted.
 * The training entry points below support top-1 only (SWITCH_E_UNSUPPORTED
 * otherwise). */

/* switch_moe_forward with its stage boundaries recorded on `stream`, for
   timing the stages of the very launches a caller measures.  stage_events
   holds 7 hipEvent_t handles created by the caller (entries may be NULL and
   are then skipped; the array itself may not be NULL -> SWITCH_E_NULL):
     [0] before the route, [1] before the capacity/slot assignment,
     [2] before the dispatch, [3] before the routed expert FFN (two GEMM
     launches), [4] after it (before the shared dense expert, if any),
     [5] before the combine, [6] after the combine.
   When the first expert GEMM reads each slot's token row straight from x (no
   dispatch copy; see above), [2] and [3] mark one point.
   Outputs, workspace, validation and errors are those of switch_moe_forward;
   a failed event record returns SWITCH_E_HIP. */
switch_status switch_moe_forward_timed(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                       const switch_moe_outputs* out, void* ws, size_t ws_bytes, void* stream,
                                       void* const* stage_events);

/* switch_moe_forward for callers that cannot allocate device memory (code
   under HIP graph capture, tight serving loops, harnesses that forbid
   hipMalloc): the same launches, outputs, validation and errors, with the
   workspace taken from a library-owned device array of
   switch_moe_noalloc_max_bytes() bytes (64 MiB) instead of an argument.  The
   array is resident on every GPU the library runs on, from its first use
   until the process ends; this call allocates nothing (no hipMalloc, no
   hipFree, no allocating library routine).  A layer whose workspace
   (switch_moe_workspace_bytes) exceeds the array is rejected with
   SWITCH_E_WORKSPACE before anything is enqueued.  All calls on one GPU
   share its array, which keeps the last call's contents: calls that overlap
   on one GPU (two streams or threads) race and must be serialised by the
   caller.  Not for training (no saved tensors). */
switch_status switch_moe_forward_noalloc(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                         const switch_moe_outputs* out, void* stream);
/* size of the array behind switch_moe_forward_noalloc, in bytes */
size_t switch_moe_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------
 * Training: the forward that keeps what the backward needs, and the
 * backward pass of the whole layer.
 *
 * The gate value multiplies the expert output, which is what lets the
 * gradient reach the router ([SWT] Switch-layer passage); f counts argmax
 * decisions and is not differentiable, so the auxiliary loss reaches the
 * router through P alone ([SWT] Eq. 4 passage); the training step
 * backpropagates into router and experts ([CAP] training-step flowchart).
 * The argmax, the capacity ranks and the ReLU pattern are taken from the
 * forward and are not differentiated.
 * ---------------------------------------------------------------------- */
typedef struct switch_moe_saved {
  float* probs;            /* [T, N] fp32: router softmax p (required) */
  int32_t* token_of_slot;  /* [N * C]: token in each slot, -1 if empty (required) */
  int32_t* active;         /* [N]: experts with kept_count > 0, ascending (required) */
  int32_t* n_active;       /* [1] (required) */
  void* h;                 /* [N, C, d_ff] dtype: ReLU(x_t . w1[e]) of each filled
                              slot; rows of empty slots undefined (required) */
  void* h_shared;          /* [T, d_ff_shared] dtype: ReLU(x . ws1); required iff
                              d_ff_shared > 0 */
} switch_moe_saved;

/* switch_moe_forward that also writes `saved` (caller-owned device buffers).
   Every output of switch_moe_forward is bit-identical; the extra writes are
   the softmax (T * N * 4 bytes) and the slot tables; the hidden activations
   go to `saved` instead of the workspace.  Same workspace size. */
switch_status switch_moe_forward_train(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                       const switch_moe_outputs* out, const switch_moe_saved* saved, void* ws,
                                       size_t ws_bytes, void* stream);

typedef struct switch_moe_grads {
  void* dx;         /* [T, d_model] dtype (required) */
  float* dw_gate;   /* [N, d_model] fp32 (required; the router trains in fp32) */
  float* dbias;     /* [N] fp32, or NULL: not computed */
  void* dw1;        /* [N, d_model, d_ff] dtype (required; zero for experts
                       that kept no token) */
  void* dw2;        /* [N, d_ff, d_model] dtype (required; idem) */
  void* dws1;       /* [d_model, d_ff_shared] dtype; required iff d_ff_shared > 0 */
  void* dws2;       /* [d_ff_shared, d_model] dtype; idem */
} switch_moe_grads;

/* Gradient of  L = sum_t <dy_t, y_t> + dl_aux * l_aux  for the forward run by
   switch_moe_forward_train with the same desc and inputs:
     combine  kept t:  dO_t = s_t dy_t (s_t = gate[t] with SWITCH_GATE_SCALE,
                       else 1), dgate_t = <dy_t, O_t> (0 without the flag);
              dropped t, and every t with SWITCH_RESIDUAL_ALL: dx_t += dy_t
     expert e (rows X = its kept tokens, Z = X w1[e], H = ReLU(Z)):
              dw2[e] = H^T dO;  dZ = (dO w2[e]^T) * [H > 0];  dw1[e] = X^T dZ;
              dx_t += (dZ w1[e]^T)_t
     router   dp_ti = [i = e_t] dgate_t + dl_aux * N * f_i / T;
              dlogit_t = p_t * (dp_t - <p_t, dp_t>);
              dw_gate = dlogit^T x;  dbias = sum_t dlogit_t;  dx += dlogit w_gate
     shared   the dense FFN's three products on every token (S = ReLU(x ws1) ws2).
   `fwd` is the forward's outputs (read: expert_id, gate, slot, kept_count,
   f) and `saved` its saved tensors; dy [T, d_model] dtype; dl_aux: device
   fp32 [1], or NULL for 0.  Every gradient is overwritten (not accumulated).
   Accumulation is fp32 everywhere; bf16 gradients are rounded once, except
   that dO = s dy and dZ are rounded to bf16 as GEMM operands.  Shape rules
   and errors are those of switch_moe_forward; deterministic.
   switch_moe_backward_workspace_bytes returns 0 for a description that the
   forward rejects or that training does not support (top_k > 1, expert
   choice, Expanded Drop, MXFP4 weights). */
size_t switch_moe_backward_workspace_bytes(const switch_moe_desc* desc);
switch_status switch_moe_backward(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                  const switch_moe_outputs* fwd, const switch_moe_saved* saved, const void* dy,
                                  const float* dl_aux, const switch_moe_grads* grads, void* ws, size_t ws_bytes,
                                  void* stream);

/* switch_moe_backward with its stage boundaries recorded on `stream`.
   stage_events holds 6 hipEvent_t handles (entries may be NULL and are then
   skipped; the array itself may not be NULL -> SWITCH_E_NULL):
     [0] start, [1] before the pass over w2 (after zeroing the weight
     gradients of experts that kept no token), [2] before the pass over w1,
     [3] after it, [4] after the shared dense expert (if any), [5] after the
     router gradient and dx (end).
   Everything else is that of switch_moe_backward; a failed event record
   returns SWITCH_E_HIP. */
switch_status switch_moe_backward_timed(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                        const switch_moe_outputs* fwd, const switch_moe_saved* saved,
                                        const void* dy, const float* dl_aux, const switch_moe_grads* grads, void* ws,
                                        size_t ws_bytes, void* stream, void* const* stage_events);

/* Static description of a status code. */
const char* switch_status_str(switch_status s);
/* Thread-local message of the last error on this thread ("" if none). */
const char* switch_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SWITCH_MOE_H */
