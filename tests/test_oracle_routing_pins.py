"""Pins of the routing-variant oracle (top-K token choice, expert choice), CPU only.

* per-token brute force in pure Python (tests/bruteforce.py) on tiny inputs,
  over both priorities, the flags, renormalised gates and heavy dropping;
* special cases: K = 1 is the top-1 layer (its own pinned oracle); K = N with
  room for every assignment, and expert choice with C = T, are both the dense
  softmax-weighted mixture sum_i p_ti E_i(x_t), checked against an einsum;
* invariants: distinct choices per token with descending logits, kept <= C,
  expert choice keeps min(C, T) per expert and every kept score is at least
  every unkept one.
"""
import numpy as np
import pytest

import oracle
from oracle import routing as orr
from tests.bruteforce import brute_forward_expert_choice, brute_forward_topk


def _tiny(seed, T, N, d, dff, bias, ties=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    if ties:  # duplicated rows: equal scores and gates, so the tie rules decide
        x[T // 2:] = x[: T - T // 2]
    return (x, rng.standard_normal((N, d)), rng.standard_normal(N) if bias else None,
            rng.standard_normal((N, d, dff)), rng.standard_normal((N, dff, d)))


TOPK_CASES = [
    # seed, T, N, d, dff, K, cf, bias, ties
    (1, 16, 4, 5, 6, 2, 1.0, False, False),
    (2, 20, 5, 4, 3, 2, 0.5, True, False),     # heavy dropping
    (3, 9, 6, 3, 4, 3, 1.5, True, False),
    (4, 12, 3, 4, 5, 3, 2.0, False, False),    # K = N
    (5, 7, 8, 3, 3, 2, 1.0, True, False),      # T < N
    (6, 18, 4, 4, 3, 2, 0.6, True, True),      # equal gates
]


@pytest.mark.parametrize("case", TOPK_CASES)
@pytest.mark.parametrize("priority", ["token", "gate"])
@pytest.mark.parametrize("gate_scale,residual_all,renorm", [(True, False, False), (False, True, False),
                                                            (True, False, True)])
def test_topk_matches_bruteforce(case, priority, gate_scale, residual_all, renorm):
    seed, T, N, d, dff, K, cf, bias, ties = case
    x, wg, b, w1, w2 = _tiny(seed, T, N, d, dff, bias, ties)
    C = orr.capacity_topk(T, N, K, cf)
    r = orr.moe_forward_topk(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, K=K, capacity_factor=cf,
                             priority=priority, gate_scale=gate_scale, residual_all=residual_all, renorm=renorm)
    bf = brute_forward_topk(x.tolist(), wg.tolist(), None if b is None else b.tolist(), w1.tolist(), w2.tolist(),
                            K, C, priority, gate_scale, residual_all, renorm)
    assert r["expert_ids"].tolist() == bf["expert_ids"]
    np.testing.assert_allclose(r["gates"], np.array(bf["gates"]), rtol=1e-12)
    assert r["slot"].tolist() == bf["slot"]
    assert r["kept_count"].tolist() == bf["kept_count"]
    assert r["n_dropped"] == bf["n_dropped"]
    assert r["routed_count"].tolist() == bf["routed_count"]
    np.testing.assert_allclose(r["f"], bf["f"], rtol=0, atol=0)
    np.testing.assert_allclose(r["P"], bf["P"], rtol=1e-12)
    assert r["l_aux"] == pytest.approx(bf["l_aux"], rel=1e-12)
    np.testing.assert_allclose(r["y"], np.array(bf["y"]), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("seed,T,N,d,dff,cf,bias,ties", [(11, 16, 4, 5, 6, 1.0, False, False),
                                                          (12, 13, 3, 4, 3, 0.5, True, False),
                                                          (13, 10, 5, 3, 4, 2.0, True, False),
                                                          (14, 5, 8, 3, 3, 1.0, False, False),
                                                          (15, 14, 3, 4, 3, 0.7, True, True)])
@pytest.mark.parametrize("gate_scale,residual_all", [(True, False), (False, True)])
def test_expert_choice_matches_bruteforce(seed, T, N, d, dff, cf, bias, ties, gate_scale, residual_all):
    x, wg, b, w1, w2 = _tiny(seed, T, N, d, dff, bias, ties)
    r = orr.moe_forward_expert_choice(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, capacity_factor=cf,
                                      gate_scale=gate_scale, residual_all=residual_all)
    bf = brute_forward_expert_choice(x.tolist(), wg.tolist(), None if b is None else b.tolist(), w1.tolist(),
                                     w2.tolist(), r["C"], gate_scale, residual_all)
    assert r["pick"].tolist() == bf["pick"]
    np.testing.assert_allclose(r["y"], np.array(bf["y"]), rtol=1e-10, atol=1e-10)


def test_topk_k1_is_the_top1_layer():
    x, wg, b, w1, w2 = _tiny(21, 40, 6, 5, 7, True)
    for pr in ("token", "gate"):
        a = orr.moe_forward_topk(x, wg, b, lambda e: w1[e], lambda e: w2[e], 6, K=1, capacity_factor=0.8,
                                 priority=pr)
        t = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], 6, capacity_factor=0.8, priority=pr)
        assert a["C"] == t["C"]
        assert a["expert_ids"][:, 0].tolist() == t["expert_id"].tolist()
        assert a["slot"][:, 0].tolist() == t["slot"].tolist()
        assert a["token_of_slot"].tolist() == t["token_of_slot"].tolist()
        np.testing.assert_array_equal(a["f"], t["f"])
        np.testing.assert_allclose(a["y"], t["y"], rtol=1e-14, atol=1e-14)


def _dense_mixture(x, wg, b, w1, w2):
    p = oracle.softmax(x @ wg.T + (0 if b is None else b))
    h = np.maximum(np.einsum("td,ndf->ntf", x, w1), 0.0)
    o = np.einsum("ntf,nfd->ntd", h, w2)
    return np.einsum("tn,ntd->td", p, o)


def test_full_topk_and_full_expert_choice_are_the_dense_mixture():
    T, N = 14, 4
    x, wg, b, w1, w2 = _tiny(31, T, N, 5, 6, True)
    want = _dense_mixture(x, wg, b, w1, w2)
    a = orr.moe_forward_topk(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, K=N, C=T)
    assert a["n_dropped"] == 0
    np.testing.assert_allclose(a["y"], want, rtol=1e-12, atol=1e-12)
    c = orr.moe_forward_expert_choice(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, C=T)
    assert (c["pick"] >= 0).all()
    np.testing.assert_allclose(c["y"], want, rtol=1e-12, atol=1e-12)


def test_routing_invariants():
    T, N, K = 300, 12, 2
    x, wg, b, w1, w2 = _tiny(41, T, N, 6, 4, True)
    l, p, e, g = orr.route_topk(x, wg, b, K)
    assert all(len(set(row)) == K for row in e.tolist())
    lv = np.take_along_axis(l, e.astype(np.int64), axis=1)
    assert (lv[:, 0] >= lv[:, 1]).all()
    for pr in ("token", "gate"):
        a = orr.assign_slots_topk(e, g, N, 20, pr)
        assert (a["kept_count"] <= 20).all()
        assert a["kept_count"].sum() == K * T - a["n_dropped"]
        # slots of one expert are 0..kept-1 exactly once
        for i in range(N):
            s = sorted(a["slot"][e == i][a["slot"][e == i] >= 0].tolist())
            assert s == list(range(a["kept_count"][i]))
    s = orr.select_expert_choice(p, 17)
    assert (s["kept_count"] == 17).all()
    for i in range(N):
        kept = s["pick"][:, i] >= 0
        assert p[kept, i].min() >= p[~kept, i].max()
