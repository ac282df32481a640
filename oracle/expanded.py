"""fp64 oracle of Expanded Drop: capacity-aware inference that re-routes
tokens dropped by a full expert to further experts of their candidate set.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Source: [CAP] "MoE expert capacity factor and token dropping" page
(wiblog.cn).  Its inference section describes Capacity-Aware Inference: token
drop caps the load of overloaded experts and discards the excess, and Expanded
Drop then lets the overflow tokens look at additional experts of their
candidate set, so that the spare capacity of lightly loaded experts is used.
Its failure-modes section names the symptom this targets (a few experts
filled to capacity while most stay nearly empty).

The page states only the idea.  Readings (each is listed in the design notes):
  * the candidate set of token t is its M highest-logit experts, in
    descending logit order with ties to the lower index (the top-K order of
    oracle/routing.py); candidate 0 is the top-1 choice; M >= 1, and M = 1 is
    the top-1 layer;
  * round 0 is the top-1 layer's capacity assignment (capacity C, the
    layer's priority order);
  * round r = 1 .. M-1: every token still without a slot applies to its
    candidate r.  Expert i has C - kept_i free slots; it takes its round-r
    applicants in the layer's priority order (token order: ascending t;
    gate-descending: descending p[t, i], ties to the lower t) and appends them
    after the slots already filled, so earlier rounds keep priority;
  * a re-routed token is processed by the expert that took it, with gate
    p[t, i] (the top-1 gate rule applied to that expert); a token that no
    candidate took passes through, as a dropped top-1 token does;
  * routed_count, f, P and L_aux stay those of the top-1 decisions:
    re-routing happens after routing, at inference.

Parity status: pinned by a sequential slot-filling simulation in pure Python
(tests/bruteforce.py), by the special cases M = 1 and C >= T (both the top-1
layer), by the closed form "M = N and N C >= T drops nothing", by a
hand-worked example (tests/golden/expanded_drop_small.txt) and by invariants.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import TOKEN_ORDER, GATE_DESC, assign_slots, aux_loss, capacity, combine, dispatch, expert_ffn, ffn, \
    router_logits, softmax


def candidates(logits: np.ndarray, M: int) -> np.ndarray:
    """Candidate set [T, M]: the M highest logits per token, descending, ties to the lower index."""
    T, N = logits.shape
    if not 1 <= M <= N:
        raise ValueError("M must be in [1, N]")
    return np.argsort(-logits, axis=1, kind="stable")[:, :M].astype(np.int32)


def assign_expanded(cand: np.ndarray, p: np.ndarray, N: int, C: int, priority: str = TOKEN_ORDER):
    """Round 0: the top-1 assignment; round r: unplaced tokens apply to cand[:, r].

    Returns dict with expert_id [T] (the expert that holds the token; the
    first choice for a token no expert took), gate [T] (p at that expert),
    slot [T] (-1 = dropped), round [T] (-1 = dropped), token_of_slot [N, C],
    kept_count [N], n_dropped, active."""
    if priority not in (TOKEN_ORDER, GATE_DESC):
        raise ValueError(priority)
    T, M = cand.shape
    rows = np.arange(T)
    e0 = cand[:, 0]
    a = assign_slots(e0, p[rows, e0], N, C, priority)
    slot = a["slot"].copy()
    tos = a["token_of_slot"].copy()
    kept = a["kept_count"].copy()
    served = e0.copy()
    gate = p[rows, e0].copy()
    rnd = np.where(slot >= 0, 0, -1).astype(np.int32)
    for r in range(1, M):
        er = cand[:, r]
        unplaced = slot < 0
        for i in range(N):
            toks = np.nonzero(unplaced & (er == i))[0]        # ascending t
            if priority == GATE_DESC and toks.size:
                toks = toks[np.lexsort((toks, -p[toks, i]))]  # primary: -p, secondary: t
            k = min(toks.size, C - int(kept[i]))
            if k <= 0:
                continue
            take = toks[:k]
            s = kept[i] + np.arange(k, dtype=np.int32)
            slot[take] = s
            tos[i, s] = take
            served[take] = i
            gate[take] = p[take, i]
            rnd[take] = r
            kept[i] += k
    return dict(expert_id=served, gate=gate, slot=slot, round=rnd, token_of_slot=tos, kept_count=kept,
                n_dropped=int(T - kept.sum()), active=np.nonzero(kept > 0)[0].astype(np.int32))


def moe_forward_expanded(x, w_gate, bias, w1_of, w2_of, N: int, M: int = 2, capacity_factor: float = 1.0,
                         C: Optional[int] = None, priority: str = TOKEN_ORDER, gate_scale: bool = True,
                         residual_all: bool = False, ws1=None, ws2=None):
    """Top-1 layer forward with Expanded Drop over M candidates, in fp64."""
    T = x.shape[0]
    l = router_logits(x, w_gate, bias)
    p = softmax(l)
    cand = candidates(l, M)
    count, f, P, l_aux = aux_loss(cand[:, 0], p, N)
    if C is None or C == 0:
        C = capacity(T, N, capacity_factor)
    a = assign_expanded(cand, p, N, C, priority)
    buf = dispatch(x, a["token_of_slot"], a["kept_count"])
    out = expert_ffn(buf, a["kept_count"], w1_of, w2_of)
    shared = ffn(x, ws1, ws2) if ws1 is not None else None
    y = combine(out, x, a["expert_id"], a["slot"], a["gate"], gate_scale, residual_all, shared)
    return dict(logits=l, p=p, candidates=cand, first_choice=cand[:, 0].copy(), routed_count=count, f=f, P=P,
                l_aux=l_aux, C=C, buf=buf, out=out, shared=shared, y=y, **a)
