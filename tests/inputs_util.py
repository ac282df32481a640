"""Test-side input conditioning: the routing predicates use the fp64 oracle.

Argmax and the gate-descending order are integer decisions taken from
floating-point values.  The HIP router evaluates them in fp32, the oracle in
fp64.  The inputs are conditioned so that the decision is the same in either
precision:

* top-2 logit margin >= 1e-3 on every row (the fp32 accumulation error of a
  logit is ~1e-5 at d = 768 and ~1e-4 at d = 5120);
* for gate-descending runs: among each expert's C_max + 1 highest-gate tokens,
  adjacent gates differ by a relative 1e-4 (the fp32 gate error is ~1e-5).

Rows that fail are redrawn by the input generator.
"""
import numpy as np

import oracle
import workloads

MARGIN = 1e-3
GATE_GAP = 1e-4


def stored_router(inp):
    dt = inp.wl.dtype
    return oracle.route(oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt), inp.bias)


def margin_bad_rows(inp):
    l, _, _, _ = stored_router(inp)
    if l.shape[1] < 2:
        return np.zeros(0, dtype=np.int64)
    top2 = np.partition(l, -2, axis=1)[:, -2:]
    return np.nonzero(top2[:, 1] - top2[:, 0] < MARGIN)[0]


def gate_gap_bad_rows(c_max, gap=GATE_GAP):
    def bad(inp):
        rows = list(margin_bad_rows(inp))
        l, p, e, g = stored_router(inp)
        for i in np.unique(e):
            toks = np.nonzero(e == i)[0]
            order = toks[np.lexsort((toks, -g[toks]))][: c_max + 1]
            gg = g[order]
            close = (gg[:-1] - gg[1:]) < gap * gg[:-1]
            rows.extend(order[1:][close].tolist())
        return np.array(sorted(set(rows)), dtype=np.int64)
    return bad


def conditioned_inputs(wl, *, weights=True, gate_order_cmax=None, threads=8):
    """Inputs with the margin rule (and the gate-gap rule if gate_order_cmax is set)."""
    pred = margin_bad_rows if gate_order_cmax is None else gate_gap_bad_rows(gate_order_cmax)
    return workloads.make_inputs(wl, weights=weights, bad_rows=pred, threads=threads)


# ---------------------------------------------------------------------------
# routing variants (top-K token choice, expert choice)
# ---------------------------------------------------------------------------
def topk_margin_bad_rows(K):
    """Rows whose top K + 1 logits are not 1e-3 apart (the K choices and their order)."""
    def bad(inp):
        l, _, _, _ = stored_router(inp)
        top = -np.sort(-l, axis=1)[:, : min(K + 1, l.shape[1])]
        return np.nonzero((top[:, :-1] - top[:, 1:] < MARGIN).any(axis=1))[0]
    return bad


def topk_gate_gap_bad_rows(K, c_max, gap=GATE_GAP):
    """Also, for gate-descending slots: inside each expert's assignment list, the
    c_max + 1 highest gates must be a relative `gap` apart."""
    from oracle import routing as orr
    margin = topk_margin_bad_rows(K)

    def bad(inp):
        rows = set(margin(inp).tolist())
        dt = inp.wl.dtype
        _, _, e, g = orr.route_topk(oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt), inp.bias, K)
        T = e.shape[0]
        ev, gv = e.T.ravel(), g.T.ravel()
        for i in np.unique(ev):
            vs = np.nonzero(ev == i)[0]
            vs = vs[np.lexsort((vs, -gv[vs]))][: c_max + 1]
            gg = gv[vs]
            close = (gg[:-1] - gg[1:]) < gap * gg[:-1]
            rows.update((vs[1:][close] % T).tolist())
        return np.array(sorted(rows), dtype=np.int64)
    return bad


def expert_choice_bad_rows(C, gap=GATE_GAP):
    """Expert choice: for every expert, its C + 1 highest probabilities must be a
    relative `gap` apart (which tokens it takes, and their slot order)."""
    def bad(inp):
        rows = set(margin_bad_rows(inp).tolist())
        _, p, _, _ = stored_router(inp)
        T = p.shape[0]
        for i in range(p.shape[1]):
            ts = np.lexsort((np.arange(T), -p[:, i]))[: C + 1]
            pp = p[ts, i]
            close = (pp[:-1] - pp[1:]) < gap * pp[:-1]
            rows.update(ts[1:][close].tolist())
        return np.array(sorted(rows), dtype=np.int64)
    return bad


def expanded_bad_rows(M, C, gate_order, gap=GATE_GAP):
    """Expanded Drop: the top-(M+1) logit margins decide every candidate list
    (topk_margin_bad_rows(M)); with gate order also the first-choice gate gaps of
    the top-1 layer (gate_gap_bad_rows(C)) and, for every expert i and round r >= 1,
    a relative `gap` between all gates p[t, i] of the tokens whose candidate r is i
    (the round's applicants are a subset of them)."""
    from oracle import expanded as ox
    margin = topk_margin_bad_rows(M)
    top1 = gate_gap_bad_rows(C, gap) if gate_order else None

    def bad(inp):
        rows = set(margin(inp).tolist())
        if not gate_order:
            return np.array(sorted(rows), dtype=np.int64)
        rows.update(top1(inp).tolist())
        l, p, _, _ = stored_router(inp)
        cand = ox.candidates(l, M)
        for r in range(1, M):
            for i in np.unique(cand[:, r]):
                ts = np.nonzero(cand[:, r] == i)[0]
                ts = ts[np.lexsort((ts, -p[ts, i]))]
                pp = p[ts, i]
                close = (pp[:-1] - pp[1:]) < gap * pp[:-1]
                rows.update(ts[1:][close].tolist())
        return np.array(sorted(rows), dtype=np.int64)
    return bad
