"""fp64 CPU oracle of the Switch top-1 MoE layer backward pass.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests,
the smoke check and the CPU-baseline leg of the benchmark may call it.

What is differentiated (page title, then section):
  [SWT]  Switch Transformers summary page (personwebsite.pages.dev,
         moe-switch): the Switch-layer passage (the gate value multiplies
         the expert output, which is what lets gradients reach the router)
         and the Eq. 4 passage (f is not differentiable, P is, so the
         auxiliary loss reaches the router through P alone).
  [CAP]  "MoE expert capacity factor and token dropping" (wiblog.cn),
         training-step flowchart: after the task and balance losses,
         backpropagation updates the router and the experts.
  [TOP1] "Top-1 Routing" concept page (compassingai.com), Key parameters
         and compute: each expert is a two-layer FFN without biases.

The forward is y = combine(...) and l_aux from the forward oracle.  Given an
upstream gradient dy [T, d] of y and a scalar dl_aux of l_aux, this returns
the gradient of   L = sum_t <dy_t, y_t> + dl_aux * l_aux   with respect to
x, W_g, b, W1[e], W2[e] (and the shared expert's weights), by the chain rule
written out step by step in fp64:

  combine:  kept t: dO_t = s_t dy_t with s_t = g_t (gate scaling) or 1;
            dg_t = <dy_t, O_t> when gate-scaled, else 0;
            dx_t += dy_t for dropped t and, with the residual flag, kept t.
  expert:   Z = X W1, H = ReLU(Z), O = H W2:
            dW2 = H^T dO;  dH = dO W2^T;  dZ = dH * relu'(Z);
            dW1 = X^T dZ;  dX = dZ W1^T  (scattered back to the tokens).
  router:   dp_{t,i} = [i = e_t] dg_t + dl_aux * N * f_i / T
            (f is held constant: it counts argmax decisions);
            dlogit_t = p_t * (dp_t - <p_t, dp_t>)  (softmax Jacobian);
            dW_g = dlogit^T x;  db = sum_t dlogit_t;  dx += dlogit W_g.
  shared:   S = ReLU(x Ws1) Ws2 for every token: the same three products.

The argmax, the capacity ranks and the ReLU pattern are piecewise constant
in the inputs, so they are taken from the forward and not differentiated.

ReLU at its kink.  relu'(0) is any value in [0, 1].  A GPU kernel decides
the sign of Z from an fp32 sum whose error is bounded by a band around 0
(2 K u sum_k |x_k W1_kf| for K products and unit roundoff u), so for a
pre-activation inside that band either choice is a valid gradient.  With
`kink_band_u` = u the base result takes every in-band pre-activation as
inactive, and the envelope (lo, hi) bounds, element by element, every result
that any on/off choice inside the band gives: each in-band pair (t, f) adds
dH_tf W1[:, f] to dx_t and x_t dH_tf to dW1[:, f] when switched on, and the
envelope adds up the negative parts (lo) and the positive parts (hi) of those
contributions.  kink_band_u = 0 (the default) takes the plain z > 0.

Parity status: pinned by central finite differences of the forward oracle
(every gradient), by torch autograd on the cases that reduce to library
routines (a dense ReLU FFN, the softmax router with fixed choices), and by
closed forms (zero aux gradient under exactly uniform routing, the
all-to-one-expert gradient, per-token softmax gradients summing to zero).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def sum_band(a: np.ndarray, w: np.ndarray, u: float) -> Optional[np.ndarray]:
    """Error band of a floating-point evaluation of a @ w: 2 K u (|a| @ |w|)."""
    if u <= 0:
        return None
    return 2.0 * a.shape[1] * u * (np.abs(a) @ np.abs(w))


def _pos(a):
    return np.maximum(a, 0.0)


def _neg(a):
    return np.minimum(a, 0.0)


def ffn_backward(rows: np.ndarray, d_out: np.ndarray, w1: np.ndarray, w2: np.ndarray, band_u: float = 0.0):
    """Backward of O = ReLU(rows W1) W2 for rows [m, d], d_out = dL/dO [m, d].

    Returns (d_rows [m, d], dW1 [d, d_ff], dW2 [d_ff, d], H [m, d_ff], env) where
    env is None for band_u = 0, else {"d_rows": (lo, hi), "dw1": (lo, hi)}."""
    z = rows @ w1
    h = np.maximum(z, 0.0)
    dw2 = h.T @ d_out
    dh = d_out @ w2.T
    band = sum_band(rows, w1, band_u)
    dz = dh * (z > (0.0 if band is None else band))
    dw1 = rows.T @ dz
    d_rows = dz @ w1.T
    env = None
    if band is not None:
        D = dh * (np.abs(z) <= band)          # contribution of each in-band pair when switched on
        env = {"d_rows": (d_rows + _pos(D) @ _neg(w1).T + _neg(D) @ _pos(w1).T,
                          d_rows + _pos(D) @ _pos(w1).T + _neg(D) @ _neg(w1).T),
               "dw1": (dw1 + _pos(rows).T @ _neg(D) + _neg(rows).T @ _pos(D),
                       dw1 + _pos(rows).T @ _pos(D) + _neg(rows).T @ _neg(D))}
    return d_rows, dw1, dw2, h, env


def combine_backward(dy: np.ndarray, out: np.ndarray, expert_id: np.ndarray, slot: np.ndarray, gate: np.ndarray,
                     gate_scale: bool = True, residual_all: bool = False):
    """Backward of the combine step.

    Returns (d_out [N, C, d] with zeros in empty slots, dg [T], dx_direct [T, d])."""
    T, d = dy.shape
    N, C = out.shape[0], out.shape[1]
    d_out = np.zeros((N, C, d))
    dg = np.zeros(T)
    dx = np.zeros((T, d))
    for t in range(T):
        s = slot[t]
        if s < 0:
            dx[t] = dy[t]
            continue
        e = expert_id[t]
        scale = gate[t] if gate_scale else 1.0
        d_out[e, s] = scale * dy[t]
        if gate_scale:
            dg[t] = float(dy[t] @ out[e, s])
        if residual_all:
            dx[t] = dy[t]
    return d_out, dg, dx


def router_backward(x: np.ndarray, w_gate: np.ndarray, p: np.ndarray, expert_id: np.ndarray, dg: np.ndarray,
                    f: np.ndarray, dl_aux: float):
    """Backward of gate = p[t, e_t] and l_aux = N sum_i f_i P_i through the softmax.

    Returns (dlogits [T, N], dW_g [N, d], db [N], dx_router [T, d])."""
    T, N = p.shape
    dp = np.zeros((T, N))
    dp[np.arange(T), expert_id] = dg
    dp += dl_aux * N * f[None, :] / T
    dlogits = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    return dlogits, dlogits.T @ x, dlogits.sum(axis=0), dlogits @ w_gate


def moe_backward(fwd: dict, x, w_gate, w1_of, w2_of, N: int, dy, dl_aux: float = 0.0, gate_scale: bool = True,
                 residual_all: bool = False, ws1=None, ws2=None, kink_band_u: float = 0.0):
    """Gradient of sum_t <dy_t, y_t> + dl_aux * l_aux for the forward `fwd` (the dict
    of oracle.moe_forward on the same fp64 x and weights).

    Returns a dict: dx [T, d], dw_gate [N, d], dbias [N], dw1 [N, d, d_ff],
    dw2 [N, d_ff, d], dws1 / dws2 (or None), dg [T], dlogits [T, N]; with
    kink_band_u > 0 also the envelopes dx_env, dw1_env, dws1_env as (lo, hi)."""
    T, d = x.shape
    e, slot, g = fwd["expert_id"], fwd["slot"], fwd["gate"]
    d_out, dg, dx = combine_backward(dy, fwd["out"], e, slot, g, gate_scale, residual_all)
    dff = w1_of(0).shape[1]
    dw1 = np.zeros((N, d, dff))
    dw2 = np.zeros((N, dff, d))
    band = kink_band_u > 0
    dx_lo, dx_hi = np.zeros((T, d)), np.zeros((T, d))      # envelope offsets
    dw1_lo, dw1_hi = (np.zeros((N, d, dff)), np.zeros((N, d, dff))) if band else (None, None)
    tos, kept = fwd["token_of_slot"], fwd["kept_count"]
    for i in range(N):
        k = int(kept[i])
        if k == 0:
            continue
        toks = tos[i, :k]
        d_rows, dw1[i], dw2[i], _, env = ffn_backward(x[toks], d_out[i, :k], w1_of(i), w2_of(i), kink_band_u)
        dx[toks] += d_rows
        if band:
            dx_lo[toks] += env["d_rows"][0] - d_rows
            dx_hi[toks] += env["d_rows"][1] - d_rows
            dw1_lo[i], dw1_hi[i] = env["dw1"]
    dws1 = dws2 = dws1_env = None
    if ws1 is not None:
        d_rows, dws1, dws2, _, env = ffn_backward(x, dy, ws1, ws2, kink_band_u)
        dx += d_rows
        if band:
            dx_lo += env["d_rows"][0] - d_rows
            dx_hi += env["d_rows"][1] - d_rows
            dws1_env = env["dw1"]
    dlogits, dwg, db, dx_r = router_backward(x, w_gate, fwd["p"], e, dg, fwd["f"], dl_aux)
    dx += dx_r
    out = dict(dx=dx, dw_gate=dwg, dbias=db, dw1=dw1, dw2=dw2, dws1=dws1, dws2=dws2, dg=dg, dlogits=dlogits)
    if band:
        out.update(dx_env=(dx + dx_lo, dx + dx_hi), dw1_env=(dw1_lo, dw1_hi), dws1_env=dws1_env)
    return out
