"""Pins of the fp64 oracle against things other than itself (CPU only).

* a hand-worked example whose values were derived on paper from the pages'
  definitions (tests/golden/worked_example.json);
* per-token brute force in pure Python on tiny random inputs;
* closed forms: L_aux = 1 under exactly uniform routing, all tokens to one
  expert, a single expert (dense FFN against an einsum);
* the invariants the layer must satisfy at any size.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from tests.bruteforce import brute_forward

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _fr(v):
    return float(Fraction(v)) if isinstance(v, str) else float(v)


def _arr(v):
    return np.array([[_fr(a) for a in row] for row in v]) if isinstance(v[0], list) else np.array([_fr(a) for a in v])


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as fh:
        return json.load(fh)


def _gold_run(gold, **kw):
    N = gold["N"]
    x = np.array(gold["x"], dtype=np.float64)
    wg = math.log(3.0) * np.eye(N)
    w1 = np.array(gold["w1"], dtype=np.float64)
    w2 = np.array(gold["w2"], dtype=np.float64)
    return oracle.moe_forward(x, wg, None, lambda e: w1[e], lambda e: w2[e], N,
                              capacity_factor=gold["capacity_factor"], **kw)


# ---------------------------------------------------------------------------
# hand-worked example
# ---------------------------------------------------------------------------
def test_worked_example_routing(gold):
    r = _gold_run(gold)
    assert r["C"] == gold["C"]
    assert r["expert_id"].tolist() == gold["expert_id"]
    np.testing.assert_allclose(r["gate"], _arr(gold["gate"]), rtol=1e-13)
    np.testing.assert_allclose(r["p"][:, 0], _arr(gold["p_expert0"]), rtol=1e-13)
    assert r["routed_count"].tolist() == gold["routed_count"]
    np.testing.assert_allclose(r["f"], _arr(gold["f"]), rtol=1e-15)
    np.testing.assert_allclose(r["P"], _arr(gold["P"]), rtol=1e-13)
    assert r["l_aux"] == pytest.approx(_fr(gold["l_aux"]), rel=1e-13)


@pytest.mark.parametrize("priority,key", [("token", "token_order"), ("gate", "gate_descending")])
def test_worked_example_slots_and_outputs(gold, priority, key):
    g = gold[key]
    r = _gold_run(gold, priority=priority)
    assert r["slot"].tolist() == g["slot"]
    assert r["kept_count"].tolist() == g["kept_count"]
    assert r["n_dropped"] == g["n_dropped"]
    np.testing.assert_allclose(r["y"], _arr(g["y_gate_scaled"]), rtol=1e-13, atol=1e-14)
    kept = r["slot"] >= 0
    o = r["out"][r["expert_id"][kept], r["slot"][kept]]
    np.testing.assert_allclose(o, _arr(gold["expert_out_unscaled"])[kept], rtol=1e-14)


def test_worked_example_flags(gold):
    t = gold["token_order"]
    r = _gold_run(gold, gate_scale=False)
    np.testing.assert_allclose(r["y"], _arr(t["y_unscaled"]), rtol=1e-14)
    r = _gold_run(gold, residual_all=True)
    np.testing.assert_allclose(r["y"], _arr(t["y_gate_scaled_residual_all"]), rtol=1e-13)


# ---------------------------------------------------------------------------
# brute force on tiny inputs
# ---------------------------------------------------------------------------
def _tiny(seed, T, N, d, dff, bias, ties=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    if ties:  # duplicated rows -> equal gates inside an expert
        x[T // 2:] = x[: T - T // 2]
    wg = rng.standard_normal((N, d))
    b = rng.standard_normal(N) if bias else None
    w1 = rng.standard_normal((N, d, dff))
    w2 = rng.standard_normal((N, dff, d))
    return x, wg, b, w1, w2


CASES = [
    # seed, T, N, d, dff, cf, bias, ties
    (1, 16, 4, 8, 6, 1.0, False, False),
    (2, 24, 3, 5, 7, 0.5, True, False),
    (3, 33, 5, 4, 4, 1.25, True, True),
    (4, 40, 6, 6, 3, 2.0, False, True),
    (5, 7, 8, 3, 5, 1.0, True, False),      # T < N
    (6, 12, 1, 4, 4, 1.0, False, False),    # one expert
    (7, 30, 2, 2, 9, 0.25, True, True),     # heavy dropping
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("priority", ["token", "gate"])
@pytest.mark.parametrize("gate_scale,residual_all", [(True, False), (False, False), (True, True)])
def test_oracle_matches_bruteforce(case, priority, gate_scale, residual_all):
    seed, T, N, d, dff, cf, bias, ties = case
    x, wg, b, w1, w2 = _tiny(seed, T, N, d, dff, bias, ties)
    C = oracle.capacity(T, N, cf)
    r = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, capacity_factor=cf,
                           priority=priority, gate_scale=gate_scale, residual_all=residual_all)
    bf = brute_forward(x.tolist(), wg.tolist(), None if b is None else b.tolist(), w1.tolist(), w2.tolist(),
                       C, priority, gate_scale, residual_all)
    assert r["expert_id"].tolist() == bf["expert_id"]
    assert r["slot"].tolist() == bf["slot"]
    assert r["kept_count"].tolist() == bf["kept_count"]
    assert r["routed_count"].tolist() == bf["routed_count"]
    assert r["n_dropped"] == bf["n_dropped"]
    np.testing.assert_allclose(r["logits"], np.array(bf["logits"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["p"], np.array(bf["p"]), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["gate"], np.array(bf["gate"]), rtol=1e-12)
    np.testing.assert_allclose(r["f"], np.array(bf["f"]), rtol=0, atol=0)
    np.testing.assert_allclose(r["P"], np.array(bf["P"]), rtol=1e-12)
    assert r["l_aux"] == pytest.approx(bf["l_aux"], rel=1e-12)
    np.testing.assert_allclose(r["y"], np.array(bf["y"]), rtol=1e-10, atol=1e-10)


def test_oracle_matches_bruteforce_shared_expert():
    x, wg, b, w1, w2 = _tiny(11, 20, 3, 4, 5, True)
    rng = np.random.default_rng(12)
    ws1, ws2 = rng.standard_normal((4, 6)), rng.standard_normal((6, 4))
    C = oracle.capacity(20, 3, 1.0)
    r = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], 3, capacity_factor=1.0, ws1=ws1, ws2=ws2)
    bf = brute_forward(x.tolist(), wg.tolist(), b.tolist(), w1.tolist(), w2.tolist(), C,
                       ws1=ws1.tolist(), ws2=ws2.tolist())
    np.testing.assert_allclose(r["y"], np.array(bf["y"]), rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,reps,d", [(4, 3, 4), (8, 5, 11), (16, 2, 16)])
def test_uniform_routing_gives_laux_one(N, reps, d):
    """x_t = one-hot(t mod N), circulant W_g: every expert gets T/N tokens and
    P_i = 1/N by symmetry, so f = P = 1/N and L_aux = 1."""
    rng = np.random.default_rng(N)
    v = rng.standard_normal(N)
    v[3 % N] = v.max() + 0.5  # unique maximum
    T = N * reps
    x = np.zeros((T, d))
    x[np.arange(T), np.arange(T) % N] = 1.0
    wg = np.zeros((N, d))
    for i in range(N):
        for j in range(N):
            wg[i, j] = v[(i - j) % N]
    _, p, e, g = oracle.route(x, wg)
    cnt, f, P, l_aux = oracle.aux_loss(e, p, N)
    assert cnt.tolist() == [reps] * N
    np.testing.assert_allclose(f, 1.0 / N, rtol=0, atol=0)
    np.testing.assert_allclose(P, 1.0 / N, rtol=1e-13)
    assert l_aux == pytest.approx(1.0, rel=1e-13)


def test_all_tokens_to_one_expert():
    T, N, d, k = 64, 8, 6, 5
    rng = np.random.default_rng(0)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((N, d)) * 0.1
    b = np.zeros(N)
    b[k] = 50.0
    _, p, e, g = oracle.route(x, wg, b)
    cnt, f, P, l_aux = oracle.aux_loss(e, p, N)
    assert (e == k).all()
    assert f.tolist() == [1.0 if i == k else 0.0 for i in range(N)]
    assert l_aux == pytest.approx(N * P[k], rel=1e-15)
    C = oracle.capacity(T, N, 1.0)
    a = oracle.assign_slots(e, g, N, C)
    assert C == T // N
    assert a["kept_count"].tolist() == [C if i == k else 0 for i in range(N)]
    assert a["n_dropped"] == T - C
    assert a["active"].tolist() == [k]


def test_single_expert_is_dense_ffn():
    T, d, dff = 37, 9, 13
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((1, d))
    w1 = rng.standard_normal((1, d, dff))
    w2 = rng.standard_normal((1, dff, d))
    r = oracle.moe_forward(x, wg, None, lambda e: w1[e], lambda e: w2[e], 1, capacity_factor=1.0)
    assert r["C"] == T and r["n_dropped"] == 0
    np.testing.assert_array_equal(r["gate"], 1.0)
    assert r["f"].tolist() == [1.0] and r["P"].tolist() == [1.0] and r["l_aux"] == 1.0
    h = np.einsum("td,df->tf", x, w1[0])
    dense = np.einsum("tf,fd->td", np.where(h > 0, h, 0.0), w2[0])
    np.testing.assert_allclose(r["y"], dense, rtol=1e-12, atol=1e-12)


def test_softmax_against_library():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 17)) * 5
    np.testing.assert_allclose(oracle.softmax(l), scipy.special.softmax(l, axis=1), rtol=1e-13)
    np.testing.assert_allclose(oracle.softmax(l).sum(1), 1.0, rtol=1e-14)


@pytest.mark.parametrize("T,N,cf,C", [(256, 8, 1.0, 32), (4096, 128, 1.25, 40), (4096, 128, 0.5, 16),
                                      (4096, 128, 2.0, 64), (16384, 128, 1.25, 160), (128, 384, 2.0, 1),
                                      (10, 1, 0.1, 1), (7, 2, 1.0, 4), (0 + 3, 3, 0.0001, 1)])
def test_capacity(T, N, cf, C):
    assert oracle.capacity(T, N, cf) == C


# ---------------------------------------------------------------------------
# invariants at moderate size, for every flag combination
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("priority", ["token", "gate"])
@pytest.mark.parametrize("cf", [0.5, 1.0, 2.0])
def test_invariants(priority, cf):
    T, N, d, dff = 512, 16, 24, 32
    rng = np.random.default_rng(int(cf * 10) + (priority == "gate"))
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((N, d)) * 0.3
    b = -1.5 * np.log(rng.permutation(N) + 1.0)
    w1 = rng.standard_normal((N, d, dff)) / np.sqrt(d)
    w2 = rng.standard_normal((N, dff, d)) / np.sqrt(dff)
    r = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, capacity_factor=cf, priority=priority)
    C, e, g, slot = r["C"], r["expert_id"], r["gate"], r["slot"]
    kept = slot >= 0
    assert r["kept_count"].sum() == T - r["n_dropped"]
    assert (r["kept_count"] <= C).all()
    assert r["f"].sum() == pytest.approx(1.0, abs=1e-15)
    assert r["P"].sum() == pytest.approx(1.0, rel=1e-13)
    assert r["routed_count"].sum() == T
    np.testing.assert_array_equal(r["y"][~kept], x[~kept])  # dropped tokens equal their input
    for i in range(N):
        toks = np.nonzero(e == i)[0]
        kt = toks[kept[toks]]
        dt = toks[~kept[toks]]
        assert sorted(slot[kt].tolist()) == list(range(len(kt)))
        if priority == "token":
            assert (kt == toks[: len(kt)]).all()  # kept set is a prefix in token order
        elif len(kt) and len(dt):
            assert g[kt].min() >= g[dt].max()
        for s in range(len(kt)):
            assert r["token_of_slot"][i, s] in kt
        assert (r["token_of_slot"][i, len(kt):] == -1).all()
    # gate scaling off / residual flag relations
    r0 = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, capacity_factor=cf,
                            priority=priority, gate_scale=False)
    r1 = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, capacity_factor=cf,
                            priority=priority, residual_all=True)
    np.testing.assert_allclose(r["y"][kept], g[kept, None] * r0["y"][kept], rtol=1e-13)
    np.testing.assert_allclose(r1["y"][kept] - x[kept], r["y"][kept], rtol=1e-9, atol=1e-12)


def test_softmax_large_logits_stays_finite():
    """Logits of magnitude ~1e3 (a strongly biased router) must still give a distribution."""
    l = np.array([[1000.0, 999.0, -1000.0], [-800.0, -801.0, -799.0]])
    p = oracle.softmax(l)
    np.testing.assert_allclose(p, scipy.special.softmax(l, axis=1), rtol=1e-13)
    assert np.isfinite(p).all()
