"""fp64 CPU oracle of the Switch top-1 MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call
this package: only the tests, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the HIP path.

Every step is the plain definition from the pages, evaluated in float64 on
the stored input values (bf16 inputs are widened exactly), with no
intermediate rounding and no blocking beyond grouping one expert's tokens
into one library matmul.  Sources (page title, then section):

  [TOP1]  "Top-1 Routing" concept page (compassingai.com), sections
          Core mechanism, Load balancing, Token Dropping,
          Key parameters and compute.
  [SWT]   Switch Transformers summary page (personwebsite.pages.dev,
          moe-switch): the Switch-layer passage (k = 1 routing, gate value
          as multiplier), the expert-capacity passage, the Eq. 4 auxiliary
          loss passage, the selective-precision passage.
  [CAP]   "MoE expert capacity factor and token dropping" (wiblog.cn),
          sections Where capacity comes from, After overflow, and the
          training-step flowchart.

Readings where the pages are silent or disagree (each one is also listed
with its reason in the design notes):
  * gate scaling of the combine is a flag (TOP1 Core mechanism says Switch
    omits it; SWT Switch-layer passage says the gate value multiplies);
  * dropped tokens pass through unchanged (TOP1 Token Dropping,
    SWT expert capacity, CAP After overflow, residual-bypass option);
  * C = max(1, ceil(cf * T / N));
  * f_i counts argmax decisions before the capacity cut, P_i averages over
    all T tokens, L_aux is returned without the alpha coefficient;
  * argmax ties go to the lowest index; gate-descending ties to the lower
    token index; slot = priority rank.

The backward pass of the layer lives in oracle/backward.py; the routing
variants next to top-1 (top-K token choice, expert choice) in
oracle/routing.py; MXFP4 expert weights in oracle/mxfp4.py; Expanded Drop
(re-routing of overflow tokens at inference) in oracle/expanded.py.

Parity status: every function here is pinned by the CPU tests
(brute-force evaluation, closed forms, invariants, a hand-worked example);
none is "parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional

import numpy as np

TOKEN_ORDER = "token"
GATE_DESC = "gate"


# ---------------------------------------------------------------------------
# storage -> fp64
# ---------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.  bf16 arrives as uint16 bit patterns."""
    if dtype == "bf16":
        u = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        # buffers read back from the device may hold signalling-NaN patterns (poisoned empty slots);
        # widening them is still exact, so numpy's invalid-value flag is not an error here
        with np.errstate(invalid="ignore"):
            return u.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# step 1-3: router  [TOP1 Core mechanism; SWT Switch-layer passage]
# ---------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t, i] = sum_k W_g[i, k] x[t, k] (+ b_i).  x [T, d], W_g [N, d] (fp64)."""
    l = x @ w_gate.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """p[t, i] = exp(l[t, i] - m_t) / sum_j exp(l[t, j] - m_t), m_t = max_j l[t, j]."""
    m = l.max(axis=1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=1, keepdims=True)


def route(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray] = None):
    """Top-1 choice: expert_id = argmax_i p (first index on ties), gate = p[expert_id].

    Returns (logits, p, expert_id int32 [T], gate fp64 [T]).
    """
    l = router_logits(x, w_gate, bias)
    p = softmax(l)
    e = np.argmax(l, axis=1).astype(np.int32)  # softmax is strictly monotone
    g = p[np.arange(p.shape[0]), e]
    return l, p, e, g


# ---------------------------------------------------------------------------
# step 4: load statistics and auxiliary loss  [TOP1 Load balancing; SWT Eq. 4]
# ---------------------------------------------------------------------------
def aux_loss(expert_id: np.ndarray, p: np.ndarray, N: int):
    """routed_count_i = #{t: e_t = i}; f_i = count_i / T; P_i = (1/T) sum_t p[t, i];
    L_aux = N * sum_i f_i * P_i.  Returns (routed_count, f, P, l_aux)."""
    T = p.shape[0]
    count = np.bincount(expert_id, minlength=N).astype(np.int64)
    f = count / T
    P = p.sum(axis=0) / T
    return count, f, P, float(N * np.sum(f * P))


# ---------------------------------------------------------------------------
# step 5: capacity  [TOP1 Token Dropping; SWT expert capacity; CAP Where capacity comes from]
# ---------------------------------------------------------------------------
def capacity(T: int, N: int, capacity_factor: float) -> int:
    """C = max(1, ceil(cf * T / N)), evaluated on the decimal value of cf."""
    v = Fraction(repr(float(capacity_factor))) * T / N
    c = -((-v.numerator) // v.denominator)
    return max(1, int(c))


# ---------------------------------------------------------------------------
# step 6: slots  [CAP After overflow + flowchart (group, count, sort, keep); TOP1 Token Dropping]
# ---------------------------------------------------------------------------
def assign_slots(expert_id: np.ndarray, gate: np.ndarray, N: int, C: int, priority: str = TOKEN_ORDER):
    """Rank every token among the tokens routed to its expert; keep rank < C.

    Token order: rank by ascending t.  Gate-descending: by descending gate,
    ties to the lower t.  Returns dict with slot [T] (-1 = dropped),
    token_of_slot [N, C] (-1 = empty), kept_count [N], n_dropped, active
    (experts with kept_count > 0, ascending).
    """
    if priority not in (TOKEN_ORDER, GATE_DESC):
        raise ValueError(priority)
    T = expert_id.shape[0]
    slot = np.full(T, -1, dtype=np.int32)
    token_of_slot = np.full((N, C), -1, dtype=np.int32)
    kept = np.zeros(N, dtype=np.int32)
    for e in range(N):
        toks = np.nonzero(expert_id == e)[0]          # ascending t
        if priority == GATE_DESC and toks.size:
            order = np.lexsort((toks, -gate[toks]))   # primary: -gate, secondary: t
            toks = toks[order]
        k = min(toks.size, C)
        slot[toks[:k]] = np.arange(k, dtype=np.int32)
        token_of_slot[e, :k] = toks[:k]
        kept[e] = k
    active = np.nonzero(kept > 0)[0].astype(np.int32)
    return dict(slot=slot, token_of_slot=token_of_slot, kept_count=kept,
                n_dropped=int(T - kept.sum()), active=active)


# ---------------------------------------------------------------------------
# step 7: dispatch into per-expert [N, C, d] buffers  [CAP Where capacity comes from]
# ---------------------------------------------------------------------------
def dispatch(x: np.ndarray, token_of_slot: np.ndarray, kept_count: np.ndarray) -> np.ndarray:
    """buf[e, s, :] = x[token_of_slot[e, s], :] for s < kept_count[e]; empty slots NaN."""
    N, C = token_of_slot.shape
    buf = np.full((N, C, x.shape[1]), np.nan)
    for e in range(N):
        k = kept_count[e]
        buf[e, :k] = x[token_of_slot[e, :k]]
    return buf


# ---------------------------------------------------------------------------
# step 8: expert FFN  [TOP1 Key parameters and compute: two-layer FFN, no bias; ReLU]
# ---------------------------------------------------------------------------
def relu(a: np.ndarray) -> np.ndarray:
    return np.maximum(a, 0.0)


def ffn(rows: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """ReLU(rows @ W1) @ W2 for rows [m, d], W1 [d, d_ff], W2 [d_ff, d]."""
    return relu(rows @ w1) @ w2


def expert_ffn(buf: np.ndarray, kept_count: np.ndarray, w1_of, w2_of) -> np.ndarray:
    """out[e, s] = ffn(buf[e, s]) for filled slots; empty slots NaN.

    w1_of(e) / w2_of(e) return expert e's fp64 weights (so a caller can widen
    one expert at a time)."""
    N, C, d = buf.shape
    out = np.full((N, C, d), np.nan)
    for e in range(N):
        k = kept_count[e]
        if k:
            out[e, :k] = ffn(buf[e, :k], w1_of(e), w2_of(e))
    return out


# ---------------------------------------------------------------------------
# step 9: combine  [TOP1 Core mechanism; SWT Switch-layer passage; TOP1 Token
# Dropping / SWT expert capacity / CAP After overflow for dropped tokens]
# ---------------------------------------------------------------------------
def combine(out: np.ndarray, x: np.ndarray, expert_id: np.ndarray, slot: np.ndarray, gate: np.ndarray,
            gate_scale: bool = True, residual_all: bool = False, shared: Optional[np.ndarray] = None):
    """kept t:    y_t = (gate_scale ? g_t : 1) * out[e_t, slot_t]  (+ x_t if residual_all)
    dropped t: y_t = x_t
    and + shared_t for every t when a shared expert is present."""
    T = x.shape[0]
    y = x.copy()
    kept = slot >= 0
    t = np.nonzero(kept)[0]
    o = out[expert_id[t], slot[t]]
    if gate_scale:
        o = gate[t][:, None] * o
    y[t] = (x[t] + o) if residual_all else o
    if shared is not None:
        y = y + shared
    return y


# ---------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------
def moe_forward(x, w_gate, bias, w1_of, w2_of, N: int, capacity_factor: float = 1.0, C: Optional[int] = None,
                priority: str = TOKEN_ORDER, gate_scale: bool = True, residual_all: bool = False,
                ws1=None, ws2=None):
    """Full forward in fp64.  x [T, d] and weights already widened to fp64.

    Returns a dict with every intermediate the layer defines."""
    T = x.shape[0]
    logits, p, e, g = route(x, w_gate, bias)
    count, f, P, l_aux = aux_loss(e, p, N)
    if C is None or C == 0:
        C = capacity(T, N, capacity_factor)
    a = assign_slots(e, g, N, C, priority)
    buf = dispatch(x, a["token_of_slot"], a["kept_count"])
    out = expert_ffn(buf, a["kept_count"], w1_of, w2_of)
    shared = ffn(x, ws1, ws2) if ws1 is not None else None
    y = combine(out, x, e, a["slot"], g, gate_scale, residual_all, shared)
    return dict(logits=logits, p=p, expert_id=e, gate=g, routed_count=count, f=f, P=P, l_aux=l_aux,
                C=C, buf=buf, out=out, shared=shared, y=y, **a)


def moe_forward_stored(inp, capacity_factor=None, C=None, priority=None, gate_scale=None, residual_all=None):
    """Convenience: run `moe_forward` on a workloads.Inputs (stored arrays)."""
    wl = inp.wl
    dt = wl.dtype
    x = widen(inp.x, dt)
    wg = widen(inp.w_gate, dt)
    ws1 = widen(inp.ws1, dt) if inp.ws1 is not None else None
    ws2 = widen(inp.ws2, dt) if inp.ws2 is not None else None
    return moe_forward(
        x, wg, inp.bias, lambda e: widen(inp.w1[e], dt), lambda e: widen(inp.w2[e], dt), wl.N,
        capacity_factor=wl.capacity_factor if capacity_factor is None else capacity_factor, C=C,
        priority=wl.priority if priority is None else priority,
        gate_scale=wl.gate_scale if gate_scale is None else gate_scale,
        residual_all=wl.residual_all if residual_all is None else residual_all,
        ws1=ws1, ws2=ws2)
