"""fp64 oracle of the routing variants next to top-1: top-K token choice and
expert choice.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Sources (page title, then section):
  [TOP1] "Top-1 Routing" concept page (compassingai.com): the introduction
         (top-2 routing activates two experts per token, as in GShard),
         Variants (token choice: each token picks its top-K experts; expert
         choice: each expert picks its top tokens and is balanced by
         construction), the routing comparison table (under expert choice a
         token can be picked by several experts or by none).
  Everything else (softmax router, capacity, buffers, the expert FFN, the
  combine, the pass-through of tokens that no expert processes) is the top-1
  layer of oracle/__init__.py.

Readings where the pages give no detail (each is listed in the design notes):
  * top-K: the K experts with the highest logits (ties to the lower index),
    in descending order; gate_tj = p[t, e_tj] (the top-1 definition applied
    to each choice), optionally renormalised over the K choices;
  * top-K capacity C = max(1, ceil(cf * K * T / N)) (K assignments per token);
  * top-K priority: the assignments are ranked as one list of "virtual
    tokens" v = j * T + t (choice-major: every first choice before every
    second choice); token order ranks by ascending v, gate-descending by
    descending gate with ties to the lower v;
  * top-K f_i counts all K * T assignments: f_i = count_i / (K T), so
    L_aux = N sum_i f_i P_i is 1 under uniform routing as for top-1;
  * expert choice: expert i takes the min(C, T) tokens with the highest
    p[t, i] (ties to the lower t), C = max(1, ceil(cf * T / N)); slot = rank
    in that order; the gate of a pick is p[t, i];
  * combine: y_t = sum over the token's kept picks of (gate-scale ? g : 1) *
    E(x_t) (+ x_t with the residual flag); a token with no kept pick passes
    through (y_t = x_t), as a dropped top-1 token does.

Parity status: pinned by per-token brute force in pure Python
(tests/bruteforce.py), by the special cases K = 1 (the top-1 layer) and
"every expert takes every token" / "K = N without drops" (both the dense
softmax-weighted mixture, checked against an einsum), and by invariants.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional

import numpy as np

from . import TOKEN_ORDER, GATE_DESC, dispatch, expert_ffn, ffn, router_logits, softmax


def route_topk(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray], K: int, renorm: bool = False):
    """Returns (logits, p, expert_ids [T, K] int32, gates [T, K] fp64)."""
    l = router_logits(x, w_gate, bias)
    p = softmax(l)
    T, N = l.shape
    if not 1 <= K <= N:
        raise ValueError("K must be in [1, N]")
    order = np.argsort(-l, axis=1, kind="stable")[:, :K]  # stable: ties keep the lower index first
    e = order.astype(np.int32)
    g = np.take_along_axis(p, order, axis=1)
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    return l, p, e, g


def aux_loss_topk(expert_ids: np.ndarray, p: np.ndarray, N: int):
    """count_i = #{(t, j): e_tj = i}; f_i = count_i / (K T); P_i = mean_t p_ti; L_aux = N sum f_i P_i."""
    T, K = expert_ids.shape
    count = np.bincount(expert_ids.ravel(), minlength=N).astype(np.int64)
    f = count / (K * T)
    P = p.sum(axis=0) / T
    return count, f, P, float(N * np.sum(f * P))


def capacity_topk(T: int, N: int, K: int, capacity_factor: float) -> int:
    """C = max(1, ceil(cf * K * T / N)), on the decimal value of cf."""
    v = Fraction(repr(float(capacity_factor))) * K * T / N
    return max(1, int(-((-v.numerator) // v.denominator)))


def assign_slots_topk(expert_ids: np.ndarray, gates: np.ndarray, N: int, C: int, priority: str = TOKEN_ORDER):
    """Rank the K T assignments inside each expert (virtual token v = j T + t).

    Returns dict with slot [T, K] (-1 = dropped), token_of_slot [N, C] (token
    index, -1 = empty), kept_count [N], n_dropped (assignments), active."""
    if priority not in (TOKEN_ORDER, GATE_DESC):
        raise ValueError(priority)
    T, K = expert_ids.shape
    ev = expert_ids.T.ravel()          # virtual order: v = j * T + t
    gv = gates.T.ravel()
    slot_v = np.full(K * T, -1, dtype=np.int32)
    token_of_slot = np.full((N, C), -1, dtype=np.int32)
    kept = np.zeros(N, dtype=np.int32)
    for i in range(N):
        vs = np.nonzero(ev == i)[0]    # ascending v
        if priority == GATE_DESC and vs.size:
            vs = vs[np.lexsort((vs, -gv[vs]))]
        k = min(vs.size, C)
        slot_v[vs[:k]] = np.arange(k, dtype=np.int32)
        token_of_slot[i, :k] = vs[:k] % T
        kept[i] = k
    slot = slot_v.reshape(K, T).T.copy()
    return dict(slot=slot, token_of_slot=token_of_slot, kept_count=kept,
                n_dropped=int(K * T - kept.sum()), active=np.nonzero(kept > 0)[0].astype(np.int32))


def combine_picks(out: np.ndarray, x: np.ndarray, pick_e: np.ndarray, pick_s: np.ndarray, pick_g: np.ndarray,
                  gate_scale: bool = True, residual_all: bool = False, shared: Optional[np.ndarray] = None):
    """y_t = sum_j [pick_s[t, j] >= 0] (gate_scale ? pick_g : 1) out[pick_e, pick_s]
    (+ x_t with the residual flag); x_t when the token has no kept pick; + shared."""
    T = x.shape[0]
    y = np.empty_like(x)
    for t in range(T):
        acc = None
        for j in range(pick_e.shape[1]):
            s = pick_s[t, j]
            if s < 0:
                continue
            o = out[pick_e[t, j], s]
            term = pick_g[t, j] * o if gate_scale else o
            acc = term if acc is None else acc + term
        if acc is None:
            y[t] = x[t]
        else:
            y[t] = acc + x[t] if residual_all else acc
    if shared is not None:
        y = y + shared
    return y


def moe_forward_topk(x, w_gate, bias, w1_of, w2_of, N: int, K: int = 2, capacity_factor: float = 1.0,
                     C: Optional[int] = None, priority: str = TOKEN_ORDER, gate_scale: bool = True,
                     residual_all: bool = False, renorm: bool = False, ws1=None, ws2=None):
    """Top-K token-choice layer forward in fp64."""
    T = x.shape[0]
    l, p, e, g = route_topk(x, w_gate, bias, K, renorm)
    count, f, P, l_aux = aux_loss_topk(e, p, N)
    if C is None or C == 0:
        C = capacity_topk(T, N, K, capacity_factor)
    a = assign_slots_topk(e, g, N, C, priority)
    buf = dispatch(x, a["token_of_slot"], a["kept_count"])
    out = expert_ffn(buf, a["kept_count"], w1_of, w2_of)
    shared = ffn(x, ws1, ws2) if ws1 is not None else None
    y = combine_picks(out, x, e, a["slot"], g, gate_scale, residual_all, shared)
    return dict(logits=l, p=p, expert_ids=e, gates=g, routed_count=count, f=f, P=P, l_aux=l_aux, C=C, buf=buf,
                out=out, shared=shared, y=y, **a)


def select_expert_choice(p: np.ndarray, C: int):
    """Expert i takes the min(C, T) tokens with the highest p[:, i] (ties to the lower t).

    Returns dict with token_of_slot [N, C] (-1 = empty), kept_count [N], and
    pick [T, N]: the slot of token t in expert i, or -1."""
    T, N = p.shape
    k = min(C, T)
    token_of_slot = np.full((N, C), -1, dtype=np.int32)
    pick = np.full((T, N), -1, dtype=np.int32)
    for i in range(N):
        ts = np.lexsort((np.arange(T), -p[:, i]))[:k]
        token_of_slot[i, :k] = ts
        pick[ts, i] = np.arange(k, dtype=np.int32)
    kept = np.full(N, k, dtype=np.int32)
    return dict(token_of_slot=token_of_slot, kept_count=kept, pick=pick,
                active=np.arange(N, dtype=np.int32), n_unpicked=int(np.sum((pick < 0).all(axis=1))))


def moe_forward_expert_choice(x, w_gate, bias, w1_of, w2_of, N: int, capacity_factor: float = 1.0,
                              C: Optional[int] = None, gate_scale: bool = True, residual_all: bool = False,
                              ws1=None, ws2=None):
    """Expert-choice layer forward in fp64."""
    T = x.shape[0]
    l = router_logits(x, w_gate, bias)
    p = softmax(l)
    if C is None or C == 0:
        v = Fraction(repr(float(capacity_factor))) * T / N
        C = max(1, int(-((-v.numerator) // v.denominator)))
    s = select_expert_choice(p, C)
    buf = dispatch(x, s["token_of_slot"], s["kept_count"])
    out = expert_ffn(buf, s["kept_count"], w1_of, w2_of)
    shared = ffn(x, ws1, ws2) if ws1 is not None else None
    pe = np.broadcast_to(np.arange(N, dtype=np.int32), (T, N))
    y = combine_picks(out, x, pe, s["pick"], p, gate_scale, residual_all, shared)
    return dict(logits=l, p=p, C=C, buf=buf, out=out, shared=shared, y=y, **s)
