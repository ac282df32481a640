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


def _softmax_row(l):
    m = max(l)
    ex = [math.exp(v - m) for v in l]
    z = math.fsum(ex)
    return [v / z for v in ex]


def brute_forward_topk(x, wg, bias, w1, w2, K, C, priority="token", gate_scale=True, residual_all=False,
                       renorm=False):
    """Top-K token choice: repeated selection of the largest remaining logit per
    token; assignment ranks by pairwise counting over the (choice, token) pairs."""
    T, N, d = len(x), len(wg), len(x[0])
    eid, gate, probs = [], [], []
    for t in range(T):
        l = [_dot(wg[i], x[t]) + (bias[i] if bias is not None else 0.0) for i in range(N)]
        p = _softmax_row(l)
        chosen = []
        for _ in range(K):
            best = None
            for i in range(N):
                if i in chosen:
                    continue
                if best is None or l[i] > l[best]:
                    best = i
            chosen.append(best)
        g = [p[i] for i in chosen]
        if renorm:
            z = math.fsum(g)
            g = [v / z for v in g]
        eid.append(chosen)
        gate.append(g)
        probs.append(p)

    def key_before(a, b):  # a, b = (j, t)
        va, vb = a[0] * T + a[1], b[0] * T + b[1]
        if priority == "token":
            return va < vb
        ga, gb = gate[a[1]][a[0]], gate[b[1]][b[0]]
        return ga > gb or (ga == gb and va < vb)

    pairs = [(j, t) for j in range(K) for t in range(T)]
    slot = [[-1] * K for _ in range(T)]
    for (j, t) in pairs:
        r = 0
        for (j2, t2) in pairs:
            if (j2, t2) != (j, t) and eid[t2][j2] == eid[t][j] and key_before((j2, t2), (j, t)):
                r += 1
        if r < C:
            slot[t][j] = r
    y = []
    for t in range(T):
        row = [0.0] * d
        any_kept = False
        for j in range(K):
            if slot[t][j] < 0:
                continue
            any_kept = True
            o = _expert(x[t], w1[eid[t][j]], w2[eid[t][j]])
            s = gate[t][j] if gate_scale else 1.0
            for k in range(d):
                row[k] += s * o[k]
        if (not any_kept) or residual_all:
            for k in range(d):
                row[k] += x[t][k]
        y.append(row)
    count = [sum(1 for t in range(T) for j in range(K) if eid[t][j] == i) for i in range(N)]
    f = [c / (K * T) for c in count]
    P = [math.fsum(probs[t][i] for t in range(T)) / T for i in range(N)]
    kept_count = [sum(1 for t in range(T) for j in range(K) if eid[t][j] == i and slot[t][j] >= 0)
                  for i in range(N)]
    return dict(expert_ids=eid, gates=gate, p=probs, slot=slot, y=y, routed_count=count, f=f, P=P,
                l_aux=N * math.fsum(f[i] * P[i] for i in range(N)), kept_count=kept_count,
                n_dropped=K * T - sum(kept_count))


def brute_forward_expert_choice(x, wg, bias, w1, w2, C, gate_scale=True, residual_all=False):
    """Expert choice: each expert ranks every token by counting the tokens with a
    higher score (ties to the lower index) and keeps ranks below C."""
    T, N, d = len(x), len(wg), len(x[0])
    probs = []
    for t in range(T):
        l = [_dot(wg[i], x[t]) + (bias[i] if bias is not None else 0.0) for i in range(N)]
        probs.append(_softmax_row(l))
    pick = [[-1] * N for _ in range(T)]
    for i in range(N):
        for t in range(T):
            r = 0
            for u in range(T):
                if u != t and (probs[u][i] > probs[t][i] or (probs[u][i] == probs[t][i] and u < t)):
                    r += 1
            if r < C:
                pick[t][i] = r
    y = []
    for t in range(T):
        row = [0.0] * d
        any_kept = False
        for i in range(N):
            if pick[t][i] < 0:
                continue
            any_kept = True
            o = _expert(x[t], w1[i], w2[i])
            s = probs[t][i] if gate_scale else 1.0
            for k in range(d):
                row[k] += s * o[k]
        if (not any_kept) or residual_all:
            for k in range(d):
                row[k] += x[t][k]
        y.append(row)
    return dict(p=probs, pick=pick, y=y)


def brute_forward_expanded(x, wg, bias, w1, w2, M, C, priority="token", gate_scale=True, residual_all=False):
    """Expanded Drop as a sequential slot-filling simulation: per round, the
    tokens still without a slot are visited one at a time in the priority
    order (ascending t, or descending p at the expert they apply to, ties to the
    lower t) and each takes the next free slot of its candidate for that round
    if there is one.  Candidates by repeated selection of the largest remaining
    logit."""
    T, N, d = len(x), len(wg), len(x[0])
    probs, chosen = [], []
    for t in range(T):
        l = [_dot(wg[i], x[t]) + (bias[i] if bias is not None else 0.0) for i in range(N)]
        probs.append(_softmax_row(l))
        c = []
        for _ in range(M):
            best = None
            for i in range(N):
                if i not in c and (best is None or l[i] > l[best]):
                    best = i
            c.append(best)
        chosen.append(c)
    fill = [0] * N
    slot = [-1] * T
    served = [c[0] for c in chosen]
    gate = [probs[t][chosen[t][0]] for t in range(T)]
    rnd = [-1] * T
    for r in range(M):
        waiting = [t for t in range(T) if slot[t] < 0]
        if priority == "gate":
            waiting.sort(key=lambda t: (-probs[t][chosen[t][r]], t))
        for t in waiting:
            e = chosen[t][r]
            if fill[e] < C:
                slot[t], served[t], gate[t], rnd[t] = fill[e], e, probs[t][e], r
                fill[e] += 1
    y = []
    for t in range(T):
        if slot[t] < 0:
            y.append(list(x[t]))
            continue
        o = _expert(x[t], w1[served[t]], w2[served[t]])
        s = gate[t] if gate_scale else 1.0
        y.append([s * o[k] + (x[t][k] if residual_all else 0.0) for k in range(d)])
    count = [sum(1 for t in range(T) if chosen[t][0] == i) for i in range(N)]  # first choices
    f = [c / T for c in count]
    P = [math.fsum(probs[t][i] for t in range(T)) / T for i in range(N)]
    return dict(candidates=chosen, p=probs, expert_id=served, gate=gate, slot=slot, round=rnd, y=y,
                kept_count=fill, n_dropped=T - sum(fill), routed_count=count, f=f, P=P,
                l_aux=N * math.fsum(f[i] * P[i] for i in range(N)))
