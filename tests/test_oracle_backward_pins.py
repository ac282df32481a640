"""Pins of the fp64 backward oracle against things other than itself (CPU only).

* central finite differences of the (separately pinned) forward oracle, for
  every gradient the backward returns, over the flag and priority variants;
* torch autograd in float64 on the cases that reduce to library routines: a
  single expert with C >= T is a dense ReLU FFN, and the router with fixed
  choices is a softmax whose gradient autograd derives on its own;
* closed forms: exactly uniform routing gives a zero aux-loss gradient, all
  tokens on one expert gives dL/dl_ti = dl_aux (N/T) p_ti ([i = k] - p_tk);
* invariants: per-token softmax gradients sum to zero, inactive experts get
  zero weight gradients, dropped tokens pass dy straight through;
* the ReLU kink option: inside the band the two choices differ by exactly
  the masked terms.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob

EPS = 1e-6


def _draw(seed, T, N, d, dff, bias, shared):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((N, d))
    b = rng.standard_normal(N) if bias else None
    w1 = rng.standard_normal((N, d, dff))
    w2 = rng.standard_normal((N, dff, d))
    ws1 = rng.standard_normal((d, dff + 2)) if shared else None
    ws2 = rng.standard_normal((dff + 2, d)) if shared else None
    dy = rng.standard_normal((T, d))
    return dict(x=x, wg=wg, b=b, w1=w1, w2=w2, ws1=ws1, ws2=ws2, dy=dy)


def _fwd(p, N, C, priority, gate_scale, residual_all):
    w1, w2 = p["w1"], p["w2"]
    return oracle.moe_forward(p["x"], p["wg"], p["b"], lambda e: w1[e], lambda e: w2[e], N, C=C, priority=priority,
                              gate_scale=gate_scale, residual_all=residual_all, ws1=p["ws1"], ws2=p["ws2"])


def _loss(p, N, C, kw, dl_aux):
    r = _fwd(p, N, C, **kw)
    return float(np.sum(p["dy"] * r["y"]) + dl_aux * r["l_aux"]), r


def _decisions(p, r):
    """Everything piecewise constant: choices, slots, ReLU patterns (kept rows and shared)."""
    pats = []
    for t in np.nonzero(r["slot"] >= 0)[0]:
        pats.append(p["x"][t] @ p["w1"][r["expert_id"][t]] > 0)
    if p["ws1"] is not None:
        pats.append((p["x"] @ p["ws1"] > 0).ravel())
    return (r["expert_id"].tolist(), r["slot"].tolist(), np.concatenate(pats).tolist() if pats else [])


def _margins_ok(p, r, N, priority):
    l = r["logits"]
    top2 = np.sort(l, axis=1)[:, -2:] if N > 1 else None
    if top2 is not None and np.min(top2[:, 1] - top2[:, 0]) < 1e-3:
        return False
    zs = [p["x"][t] @ p["w1"][r["expert_id"][t]] for t in range(len(r["slot"]))]
    if p["ws1"] is not None:
        zs.append((p["x"] @ p["ws1"]).ravel())
    if np.min(np.abs(np.concatenate(zs))) < 1e-3:
        return False
    if priority == "gate":
        for i in range(N):
            g = np.sort(r["gate"][r["expert_id"] == i])
            if g.size > 1 and np.min(np.diff(g)) < 1e-3:
                return False
    return True


def _fd_grad(p, name, N, C, kw, dl_aux, base_dec):
    a = p[name]
    g = np.zeros_like(a)
    flat, gflat = a.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        v = flat[i]
        flat[i] = v + EPS
        lp, rp = _loss(p, N, C, kw, dl_aux)
        assert _decisions(p, rp) == base_dec, (name, i)
        flat[i] = v - EPS
        lm, rm = _loss(p, N, C, kw, dl_aux)
        assert _decisions(p, rm) == base_dec, (name, i)
        flat[i] = v
        gflat[i] = (lp - lm) / (2 * EPS)
    return g


def _case(seed0, T, N, d, dff, cf, bias, shared, priority, kw):
    for seed in range(seed0, seed0 + 200):
        p = _draw(seed, T, N, d, dff, bias, shared)
        C = oracle.capacity(T, N, cf)
        r = _fwd(p, N, C, priority=priority, **kw)
        if _margins_ok(p, r, N, priority):
            return p, C, r
    raise AssertionError("no well-conditioned draw")


FD_CASES = [
    # id, seed, T, N, d, dff, cf, bias, shared, priority, gate_scale, residual_all, dl_aux
    ("token-scaled", 100, 14, 3, 4, 5, 1.0, False, False, "token", True, False, 0.0),
    ("token-aux-bias", 200, 12, 4, 3, 4, 0.75, True, False, "token", True, False, 0.7),
    ("gate-order", 300, 13, 3, 3, 4, 0.75, True, False, "gate", True, False, -0.4),
    ("unscaled-residual", 400, 11, 3, 3, 5, 0.6, False, False, "token", False, True, 0.3),
    ("shared-expert", 500, 10, 2, 3, 3, 1.0, True, True, "token", True, False, 0.5),
    ("one-expert", 600, 7, 1, 3, 4, 1.0, False, False, "token", True, False, 1.0),
]


@pytest.mark.parametrize("case", FD_CASES, ids=[c[0] for c in FD_CASES])
def test_backward_matches_finite_differences(case):
    _, seed, T, N, d, dff, cf, bias, shared, priority, gs, ra, dl_aux = case
    kw = dict(priority=priority, gate_scale=gs, residual_all=ra)
    p, C, r = _case(seed, T, N, d, dff, cf, bias, shared, priority, dict(gate_scale=gs, residual_all=ra))
    assert r["n_dropped"] > 0 or N == 1 or cf >= 1.0
    w1, w2 = p["w1"], p["w2"]
    got = ob.moe_backward(r, p["x"], p["wg"], lambda e: w1[e], lambda e: w2[e], N, p["dy"], dl_aux,
                          gate_scale=gs, residual_all=ra, ws1=p["ws1"], ws2=p["ws2"])
    dec = _decisions(p, r)
    names = [("x", "dx"), ("wg", "dw_gate"), ("w1", "dw1"), ("w2", "dw2")]
    if bias:
        names.append(("b", "dbias"))
    if shared:
        names += [("ws1", "dws1"), ("ws2", "dws2")]
    for pn, gn in names:
        fd = _fd_grad(p, pn, N, C, kw, dl_aux, dec)
        scale = max(1.0, float(np.max(np.abs(fd))))
        np.testing.assert_allclose(got[gn], fd, rtol=0, atol=2e-7 * scale, err_msg=gn)


def test_dense_ffn_matches_torch_autograd():
    """N = 1, C >= T: the layer is y = g ReLU(x W1) W2 with g = 1 and a router
    whose softmax over one expert is constant."""
    T, d, dff = 21, 7, 11
    rng = np.random.default_rng(7)
    x, w1, w2 = rng.standard_normal((T, d)), rng.standard_normal((1, d, dff)), rng.standard_normal((1, dff, d))
    wg, b, dy = rng.standard_normal((1, d)), rng.standard_normal(1), rng.standard_normal((T, d))
    r = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], 1, capacity_factor=1.0)
    got = ob.moe_backward(r, x, wg, lambda e: w1[e], lambda e: w2[e], 1, dy, dl_aux=0.9)
    tx = torch.tensor(x, requires_grad=True)
    t1 = torch.tensor(w1[0], requires_grad=True)
    t2 = torch.tensor(w2[0], requires_grad=True)
    y = torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(tx, t1.T)), t2.T)
    y.backward(torch.tensor(dy))
    np.testing.assert_allclose(got["dx"], tx.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["dw1"][0], t1.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["dw2"][0], t2.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert not got["dw_gate"].any() and not got["dbias"].any()


@pytest.mark.parametrize("N,T,d,c_aux", [(5, 17, 6, 0.0), (8, 32, 4, 1.3), (3, 9, 10, -2.0)])
def test_router_matches_torch_autograd(N, T, d, c_aux):
    """gate_t = softmax(x W_g^T + b)[t, e_t] with the choices e held fixed, and
    l_aux = N sum_i f_i mean_t p_ti with f held fixed: torch differentiates it."""
    rng = np.random.default_rng(N * 100 + T)
    x, wg, b = rng.standard_normal((T, d)), rng.standard_normal((N, d)), rng.standard_normal(N)
    a = rng.standard_normal(T)  # upstream gradient of each gate
    l = x @ wg.T + b
    e = np.argmax(l, axis=1)
    p = oracle.softmax(l)
    f = np.bincount(e, minlength=N) / T
    dlog, dwg, db, dx = ob.router_backward(x, wg, p, e.astype(np.int32), a, f, c_aux)
    tx, tw, tb = (torch.tensor(v, requires_grad=True) for v in (x, wg, b))
    tp = torch.softmax(tx @ tw.T + tb, dim=1)
    loss = (torch.tensor(a) * tp[torch.arange(T), torch.tensor(e)]).sum() \
        + c_aux * N * (torch.tensor(f) * tp.mean(dim=0)).sum()
    loss.backward()
    np.testing.assert_allclose(dwg, tw.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dlog.sum(axis=1), 0.0, atol=1e-14)


def test_uniform_routing_gives_zero_aux_gradient():
    """f_i = 1/N for every i: dL_aux/dl_ti = (N/T) p_ti (f_i - sum_j p_tj f_j) = 0."""
    N, reps, d = 8, 4, 8
    rng = np.random.default_rng(2)
    v = rng.standard_normal(N)
    v[5] = v.max() + 0.5
    T = N * reps
    x = np.zeros((T, d))
    x[np.arange(T), np.arange(T) % N] = 1.0
    wg = np.array([[v[(i - j) % N] for j in range(d)] for i in range(N)])
    _, p, e, g = oracle.route(x, wg)
    cnt, f, P, _ = oracle.aux_loss(e, p, N)
    assert cnt.tolist() == [reps] * N
    dlog, dwg, db, dx = ob.router_backward(x, wg, p, e, np.zeros(T), f, 1.0)
    np.testing.assert_allclose(dlog, 0.0, atol=1e-16)
    np.testing.assert_allclose(dwg, 0.0, atol=1e-15)


def test_all_to_one_expert_aux_gradient():
    """Every token on expert k: f = e_k, so dL_aux/dl_ti = dl_aux (N/T) p_ti ([i = k] - p_tk)."""
    T, N, d, k, c = 40, 6, 5, 2, 0.8
    rng = np.random.default_rng(9)
    x, wg = rng.standard_normal((T, d)), 0.1 * rng.standard_normal((N, d))
    b = np.zeros(N)
    b[k] = 2.0
    _, p, e, g = oracle.route(x, wg, b)
    assert (e == k).all()
    _, f, _, _ = oracle.aux_loss(e, p, N)
    dlog, _, db, _ = ob.router_backward(x, wg, p, e, np.zeros(T), f, c)
    want = c * N / T * p * ((np.arange(N) == k)[None, :] - p[:, [k]])
    np.testing.assert_allclose(dlog, want, rtol=1e-13, atol=1e-17)


@pytest.mark.parametrize("priority", ["token", "gate"])
def test_backward_invariants(priority):
    T, N, d, dff = 48, 6, 5, 7
    p = _draw(31, T, N, d, dff, True, False)
    w1, w2 = p["w1"], p["w2"]
    C = 3
    r = oracle.moe_forward(p["x"], p["wg"], p["b"], lambda e: w1[e], lambda e: w2[e], N, C=C, priority=priority)
    # no router gradient at all: gate scaling off and dl_aux = 0
    r0 = oracle.moe_forward(p["x"], p["wg"], p["b"], lambda e: w1[e], lambda e: w2[e], N, C=C, priority=priority,
                            gate_scale=False)
    g0 = ob.moe_backward(r0, p["x"], p["wg"], lambda e: w1[e], lambda e: w2[e], N, p["dy"], 0.0, gate_scale=False)
    drop = r0["slot"] < 0
    assert drop.any()
    np.testing.assert_array_equal(g0["dx"][drop], p["dy"][drop])
    assert not g0["dw_gate"].any() and not g0["dbias"].any()
    # linear in (dy, dl_aux); softmax rows sum to zero; inactive experts untouched
    ga = ob.moe_backward(r, p["x"], p["wg"], lambda e: w1[e], lambda e: w2[e], N, p["dy"], 0.5)
    gb = ob.moe_backward(r, p["x"], p["wg"], lambda e: w1[e], lambda e: w2[e], N, 2 * p["dy"], 1.0)
    for k in ("dx", "dw_gate", "dbias", "dw1", "dw2"):
        np.testing.assert_allclose(gb[k], 2 * ga[k], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ga["dlogits"].sum(axis=1), 0.0, atol=1e-13)
    for i in range(N):
        if r["kept_count"][i] == 0:
            assert not ga["dw1"][i].any() and not ga["dw2"][i].any()


def test_relu_kink_envelope_bounds_every_choice():
    """In-band pre-activations (two of them exactly 0, one tiny): the envelope
    must hold the result of every on/off choice, enumerated by brute force, and
    be attained by the all-negative and all-positive selections."""
    rng = np.random.default_rng(4)
    rows, w1, w2 = rng.standard_normal((4, 5)), rng.standard_normal((5, 6)), rng.standard_normal((6, 5))
    w1[:, 2] = 0.0
    w1[0, 2] = 1.0
    w1[3, 2] = 0.5
    rows[1, 0] = 0.0
    rows[1, 3] = 0.0                 # z[1, 2] = 0 exactly
    rows[3, 0] = -0.5 * rows[3, 3] + 1e-12  # z[3, 2] ~ 1e-12: inside the band, positive
    w1[:, 4] = 0.0
    w1[1, 4] = 1.0
    rows[2, 1] = 0.0                 # z[2, 4] = 0 exactly
    dout = rng.standard_normal((4, 5))
    d_rows, dw1, dw2, h, env = ob.ffn_backward(rows, dout, w1, w2, band_u=2.0 ** -24)
    z = rows @ w1
    inband = [(1, 2), (3, 2), (2, 4)]
    assert all(abs(z[p]) <= ob.sum_band(rows, w1, 2.0 ** -24)[p] for p in inband)
    dh = dout @ w2.T
    base_mask = (z > 0).astype(float)
    for p in inband:
        base_mask[p] = 0.0
    lo_r, hi_r = env["d_rows"]
    lo_w, hi_w = env["dw1"]
    for bits in range(1 << len(inband)):
        m = base_mask.copy()
        for j, p in enumerate(inband):
            if bits >> j & 1:
                m[p] = 1.0
        dz = dh * m
        r, w = dz @ w1.T, rows.T @ dz
        assert np.all(r >= lo_r - 1e-12) and np.all(r <= hi_r + 1e-12)
        assert np.all(w >= lo_w - 1e-12) and np.all(w <= hi_w + 1e-12)
    np.testing.assert_allclose(d_rows, (dh * base_mask) @ w1.T, rtol=1e-14, atol=1e-14)
    # band 0: the plain z > 0 (so the 1e-30 pre-activation counts as active)
    d0 = ob.ffn_backward(rows, dout, w1, w2)
    assert d0[4] is None
    m0 = (z > 0).astype(float)
    np.testing.assert_allclose(d0[0], (dh * m0) @ w1.T, rtol=1e-14, atol=1e-14)
