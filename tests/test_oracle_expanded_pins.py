"""Pins of the Expanded Drop oracle (oracle/expanded.py), CPU only.

* a sequential slot-filling simulation in pure Python (tests/bruteforce.py)
  on tiny inputs, both priorities, the flags, heavy dropping and equal gates;
* the hand-worked example tests/golden/expanded_drop_small.json;
* special cases: M = 1 and C >= T are the top-1 layer (its own pinned
  oracle); M = N with N C >= T drops nothing (a token left without a slot
  would need all N experts full, i.e. N C <= T - 1 kept tokens);
* invariants: kept <= C, slots 0 .. kept-1 filled once per expert, a token
  placed in round r sits at its candidate r with gate p there, a token left
  over finds every candidate full, round-0 placements are the top-1 layer's,
  and more candidates never drop more tokens.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import expanded as ox
from tests.bruteforce import brute_forward_expanded

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "expanded_drop_small.json")


def _tiny(seed, T, N, d, dff, bias, ties=False, skew=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    if ties:  # duplicated rows: equal gates, so the tie rules decide
        x[T // 2:] = x[: T - T // 2]
    b = rng.standard_normal(N) if bias else None
    if skew:
        b = (b if b is not None else np.zeros(N)) - skew * np.log1p(np.arange(N))
    return x, rng.standard_normal((N, d)), b, rng.standard_normal((N, d, dff)), rng.standard_normal((N, dff, d))


CASES = [
    # seed, T, N, d, dff, M, cf, bias, ties, skew
    (1, 16, 4, 5, 6, 2, 1.0, False, False, 0.0),
    (2, 24, 5, 4, 3, 3, 0.5, True, False, 1.5),     # heavy dropping, skewed load
    (3, 9, 6, 3, 4, 4, 0.8, True, False, 0.0),
    (4, 12, 3, 4, 5, 3, 0.7, False, False, 2.0),    # M = N
    (5, 7, 8, 3, 3, 2, 1.0, True, False, 0.0),      # T < N
    (6, 18, 4, 4, 3, 2, 0.6, True, True, 1.0),      # equal gates
    (7, 20, 4, 3, 3, 4, 0.4, False, True, 3.0),     # all candidates, most tokens overflow
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("priority", ["token", "gate"])
@pytest.mark.parametrize("gate_scale,residual_all", [(True, False), (False, True)])
def test_expanded_matches_sequential_simulation(case, priority, gate_scale, residual_all):
    seed, T, N, d, dff, M, cf, bias, ties, skew = case
    x, wg, b, w1, w2 = _tiny(seed, T, N, d, dff, bias, ties, skew)
    r = ox.moe_forward_expanded(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, M=M, capacity_factor=cf,
                                priority=priority, gate_scale=gate_scale, residual_all=residual_all)
    bf = brute_forward_expanded(x.tolist(), wg.tolist(), None if b is None else b.tolist(), w1.tolist(),
                                w2.tolist(), M, r["C"], priority, gate_scale, residual_all)
    assert r["candidates"].tolist() == bf["candidates"]
    assert r["expert_id"].tolist() == bf["expert_id"]
    assert r["slot"].tolist() == bf["slot"]
    assert r["round"].tolist() == bf["round"]
    assert r["kept_count"].tolist() == bf["kept_count"]
    assert r["n_dropped"] == bf["n_dropped"]
    np.testing.assert_allclose(r["gate"], np.array(bf["gate"]), rtol=1e-12)
    np.testing.assert_allclose(r["y"], np.array(bf["y"]), rtol=1e-10, atol=1e-10)
    # the load statistics stay those of the first choices
    assert r["routed_count"].tolist() == bf["routed_count"]
    np.testing.assert_allclose(r["f"], bf["f"], rtol=0, atol=0)
    np.testing.assert_allclose(r["P"], bf["P"], rtol=1e-12)
    assert r["l_aux"] == pytest.approx(bf["l_aux"], rel=1e-12)


def test_cases_reroute_tokens():
    """The parametrised cases do exercise re-routing (and leave some tokens over)."""
    rerouted = dropped = 0
    for seed, T, N, d, dff, M, cf, bias, ties, skew in CASES:
        x, wg, b, w1, w2 = _tiny(seed, T, N, d, dff, bias, ties, skew)
        r = ox.moe_forward_expanded(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, M=M, capacity_factor=cf)
        rerouted += int((r["round"] > 0).sum())
        dropped += r["n_dropped"]
    assert rerouted >= 10 and dropped >= 5


@pytest.mark.parametrize("case", range(5))
def test_golden_small(case):
    g = json.load(open(GOLDEN))
    c = g["cases"][case]
    l = np.array(g["logits"])
    p = oracle.softmax(l)
    a = ox.assign_expanded(ox.candidates(l, c["M"]), p, g["N"], g["C"], c["priority"])
    assert a["expert_id"].tolist() == c["expert_id"]
    assert a["slot"].tolist() == c["slot"]
    assert a["round"].tolist() == c["round"]
    assert a["kept_count"].tolist() == c["kept_count"]
    assert a["n_dropped"] == c["n_dropped"]
    np.testing.assert_array_equal(a["gate"], p[np.arange(len(l)), a["expert_id"]])


@pytest.mark.parametrize("priority", ["token", "gate"])
def test_m1_is_top1_layer(priority):
    x, wg, b, w1, w2 = _tiny(21, 30, 5, 4, 6, True, skew=1.0)
    r = ox.moe_forward_expanded(x, wg, b, lambda e: w1[e], lambda e: w2[e], 5, M=1, capacity_factor=0.6,
                                priority=priority)
    t1 = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], 5, capacity_factor=0.6, priority=priority)
    for k in ("expert_id", "slot", "token_of_slot", "kept_count", "active", "routed_count"):
        np.testing.assert_array_equal(r[k], t1[k], err_msg=k)
    assert r["n_dropped"] == t1["n_dropped"] > 0
    np.testing.assert_array_equal(r["gate"], t1["gate"])
    np.testing.assert_array_equal(r["y"], t1["y"])
    assert r["l_aux"] == t1["l_aux"]


@pytest.mark.parametrize("priority", ["token", "gate"])
def test_room_for_all_is_top1_layer(priority):
    x, wg, b, w1, w2 = _tiny(22, 25, 4, 4, 5, True, skew=1.0)
    r = ox.moe_forward_expanded(x, wg, b, lambda e: w1[e], lambda e: w2[e], 4, M=3, C=25, priority=priority)
    t1 = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], 4, C=25, priority=priority)
    assert r["n_dropped"] == 0 and (r["round"] == 0).all()
    np.testing.assert_array_equal(r["slot"], t1["slot"])
    np.testing.assert_array_equal(r["y"], t1["y"])


@pytest.mark.parametrize("seed,T,N,cf", [(31, 40, 4, 1.0), (32, 64, 8, 1.0), (33, 30, 5, 1.2), (34, 50, 3, 1.0)])
@pytest.mark.parametrize("priority", ["token", "gate"])
def test_all_candidates_drop_nothing(seed, T, N, cf, priority):
    """M = N and N C >= T: every token ends in some expert, however skewed the router."""
    x, wg, b, w1, w2 = _tiny(seed, T, N, 3, 2, True, skew=3.0)
    C = oracle.capacity(T, N, cf)
    assert N * C >= T
    r = ox.moe_forward_expanded(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, M=N, C=C, priority=priority)
    t1 = oracle.moe_forward(x, wg, b, lambda e: w1[e], lambda e: w2[e], N, C=C, priority=priority)
    assert t1["n_dropped"] > 0  # the skew overflows the top-1 layer
    assert r["n_dropped"] == 0 and (r["slot"] >= 0).all()


def _check_invariants(r, N, C, M, priority):
    T = len(r["slot"])
    cand, p = r["candidates"], r["p"]
    kept = r["kept_count"]
    assert (kept <= C).all()
    assert kept.sum() + r["n_dropped"] == T
    for i in range(N):
        toks = r["token_of_slot"][i, :kept[i]]
        assert (toks >= 0).all() and (r["token_of_slot"][i, kept[i]:] == -1).all()
        assert (r["expert_id"][toks] == i).all()
        assert r["slot"][toks].tolist() == list(range(kept[i]))
    placed = np.nonzero(r["slot"] >= 0)[0]
    assert (cand[placed, r["round"][placed]] == r["expert_id"][placed]).all()
    np.testing.assert_array_equal(r["gate"], p[np.arange(T), r["expert_id"]])
    for t in np.nonzero(r["slot"] < 0)[0]:
        assert (kept[cand[t]] == C).all(), f"token {t} left over with a free candidate"
        assert r["expert_id"][t] == cand[t, 0]
    # round 0 is the top-1 assignment
    t1 = oracle.assign_slots(cand[:, 0], p[np.arange(T), cand[:, 0]], N, C, priority)
    np.testing.assert_array_equal(np.nonzero(r["round"] == 0)[0], np.nonzero(t1["slot"] >= 0)[0])
    # inside each expert, the tokens of a later round sit after those of an earlier one
    for i in range(N):
        rr = r["round"][r["token_of_slot"][i, :kept[i]]]
        assert (np.diff(rr) >= 0).all()


@pytest.mark.parametrize("priority", ["token", "gate"])
def test_invariants_medium(priority):
    rng = np.random.default_rng(41)
    T, N, d = 600, 12, 16
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((N, d)) * 0.3
    b = -1.2 * np.log1p(rng.permutation(N))
    drops = []
    for M in range(1, 6):
        r = ox.moe_forward_expanded(x, wg, b, lambda e: np.zeros((d, 1)), lambda e: np.zeros((1, d)), N, M=M,
                                    capacity_factor=0.9, priority=priority)
        _check_invariants(r, N, r["C"], M, priority)
        drops.append(r["n_dropped"])
    assert all(a >= b_ for a, b_ in zip(drops, drops[1:])), drops
    assert drops[0] > drops[-1]


def test_gate_order_prefers_higher_gate_in_later_rounds():
    """Inside a re-route round the free slots go by descending p at that expert,
    not by token index (the golden example's t0/t1 contest, restated on
    shuffled token positions)."""
    g = json.load(open(GOLDEN))
    l = np.array(g["logits"])
    perm = np.array([5, 1, 7, 0, 3, 6, 2, 4])   # new position of each old token
    l2 = np.empty_like(l)
    l2[perm] = l
    p2 = oracle.softmax(l2)
    a = ox.assign_expanded(ox.candidates(l2, 2), p2, 3, 2, "gate")
    c = g["cases"][3]
    assert a["expert_id"][perm].tolist() == c["expert_id"]
    assert a["round"][perm].tolist() == c["round"]
    assert sorted(a["kept_count"].tolist()) == sorted(c["kept_count"])
