"""Per-token brute-force evaluation of the Switch top-1 layer, pure Python.

Independent of the oracle: plain loops over Python floats, the softmax via
math.exp, ranks by counting higher-priority tokens pairwise (O(T^2)), and the
expert term in mask form (every expert evaluated on every token, then the
routed one selected).  Only for tiny inputs.
"""
import math


def _dot(a, b):
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def _expert(xrow, w1, w2):
    # w1[k][j] (d x d_ff), w2[j][k] (d_ff x d)
    d = len(xrow)
    dff = len(w1[0])
    h = []
    for j in range(dff):
        s = 0.0
        for k in range(d):
            s += xrow[k] * w1[k][j]
        h.append(s if s > 0.0 else 0.0)
    o = []
    for k in range(d):
        s = 0.0
        for j in range(dff):
            s += h[j] * w2[j][k]
        o.append(s)
    return o


def brute_forward(x, wg, bias, w1, w2, C, priority="token", gate_scale=True, residual_all=False,
                  ws1=None, ws2=None):
    """x: list of T rows; wg: N rows; bias: list or None; w1[i]: d x d_ff; w2[i]: d_ff x d."""
    T = len(x)
    N = len(wg)
    d = len(x[0])
    logits, probs, eid, gate = [], [], [], []
    for t in range(T):
        l = [_dot(wg[i], x[t]) + (bias[i] if bias is not None else 0.0) for i in range(N)]
        best = 0
        for i in range(1, N):
            if l[i] > l[best]:
                best = i
        m = l[best]
        ex = [math.exp(v - m) for v in l]
        z = math.fsum(ex)
        p = [v / z for v in ex]
        logits.append(l)
        probs.append(p)
        eid.append(best)
        gate.append(p[best])

    def before(u, t):
        if priority == "token":
            return u < t
        return gate[u] > gate[t] or (gate[u] == gate[t] and u < t)

    rank = []
    for t in range(T):
        r = 0
        for u in range(T):
            if u != t and eid[u] == eid[t] and before(u, t):
                r += 1
        rank.append(r)
    kept = [r < C for r in rank]

    y = []
    for t in range(T):
        row = [0.0] * d
        for i in range(N):
            sel = 1.0 if (eid[t] == i and kept[t]) else 0.0
            if sel:
                o = _expert(x[t], w1[i], w2[i])
                s = gate[t] if gate_scale else 1.0
                for k in range(d):
                    row[k] += s * o[k]
        if (not kept[t]) or residual_all:
            for k in range(d):
                row[k] += x[t][k]
        if ws1 is not None:
            sh = _expert(x[t], ws1, ws2)
            for k in range(d):
                row[k] += sh[k]
        y.append(row)

    count = [sum(1 for t in range(T) if eid[t] == i) for i in range(N)]
    f = [c / T for c in count]
    P = [math.fsum(probs[t][i] for t in range(T)) / T for i in range(N)]
    l_aux = N * math.fsum(f[i] * P[i] for i in range(N))
    kept_count = [sum(1 for t in range(T) if eid[t] == i and kept[t]) for i in range(N)]
    slot = [rank[t] if kept[t] else -1 for t in range(T)]
    return dict(logits=logits, p=probs, expert_id=eid, gate=gate, rank=rank, slot=slot, y=y,
                routed_count=count, f=f, P=P, l_aux=l_aux, kept_count=kept_count,
                n_dropped=T - sum(kept_count))
