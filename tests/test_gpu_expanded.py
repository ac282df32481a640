"""GPU parity of Expanded Drop (switch_moe_forward with desc.expand_choices =
M >= 2) against the fp64 oracle (oracle/expanded.py) on the same seeded inputs.

Bars as for top-1: the serving expert, slots, kept counts, n_dropped,
routed_count bit-exact; gates and P relative 1e-5; f exact; outputs per token
max_k |y - y_ref| / max_k |y_ref| <= 1e-4 (fp32) or 2e-2 (bf16); tokens left
without a slot bit-identical to x.  Inputs are conditioned so that every
candidate list and every gate-order decision is taken by margins far above
fp32 rounding (tests/inputs_util.expanded_bad_rows).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import expanded as ox
from tests import inputs_util
from tests.gpu_util import TOL_OUT, TOL_P, dev, host, host_bits, row_rel

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from switch_top_routed_amd import native


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _custom(name, T, d, dff, N, cf, dtype="bf16", seed=0, **kw):
    return workloads.Workload(name, T, d, dff, N, cf, dtype, 1.0 / math.sqrt(d), seed=40_000 + seed, **kw)


def _devs(inp, dt):
    return dict(x=dev(inp.x, dt), w_gate=dev(inp.w_gate, dt), w1=dev(inp.w1, dt), w2=dev(inp.w2, dt),
                bias=None if inp.bias is None else torch.from_numpy(inp.bias).cuda(),
                ws1=None if inp.ws1 is None else dev(inp.ws1, dt), ws2=None if inp.ws2 is None else dev(inp.ws2, dt))


def _layer(wl, **kw):
    return native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N,
                            dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32,
                            capacity_factor=wl.capacity_factor, priority=wl.priority, gate_scale=wl.gate_scale,
                            residual_all=wl.residual_all, d_ff_shared=wl.d_ff_shared, **kw)


def _run(layer, d):
    out = layer(d["x"], d["w_gate"], d["w1"], d["w2"], bias=d["bias"], ws1=d["ws1"], ws2=d["ws2"])
    torch.cuda.synchronize()
    return out


def _expand_case(wl, M, C=None):
    C = C or oracle.capacity(wl.T, wl.N, wl.capacity_factor)
    _say(f"expanded M={M} {wl.name} T={wl.T} N={wl.N} C={C} {wl.priority} gs={wl.gate_scale} "
         f"res={wl.residual_all} shared={wl.d_ff_shared} {wl.dtype}")
    inp = workloads.make_inputs(wl, bad_rows=inputs_util.expanded_bad_rows(M, C, wl.priority == "gate"))
    d = _devs(inp, wl.dtype)
    layer = _layer(wl, expand=M, C=C)
    out = _run(layer, d)
    dt = wl.dtype
    ws1 = oracle.widen(inp.ws1, dt) if inp.ws1 is not None else None
    ws2 = oracle.widen(inp.ws2, dt) if inp.ws2 is not None else None
    ref = ox.moe_forward_expanded(oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt), inp.bias,
                                  lambda e: oracle.widen(inp.w1[e], dt), lambda e: oracle.widen(inp.w2[e], dt),
                                  wl.N, M=M, C=C, priority=wl.priority, gate_scale=wl.gate_scale,
                                  residual_all=wl.residual_all, ws1=ws1, ws2=ws2)
    assert layer.C == C
    np.testing.assert_array_equal(host(out["expert_id"]), ref["expert_id"])
    np.testing.assert_array_equal(host(out["slot"]), ref["slot"])
    np.testing.assert_array_equal(host(out["kept_count"]), ref["kept_count"])
    assert int(host(out["n_dropped"])[0]) == ref["n_dropped"]
    np.testing.assert_allclose(host(out["gate"]), ref["gate"], rtol=1e-5)
    np.testing.assert_array_equal(host(out["routed_count"]), ref["routed_count"])
    np.testing.assert_array_equal(host(out["f"]), ref["f"].astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(host(out["P"]), ref["P"], rtol=TOL_P, atol=1e-9)
    assert abs(float(host(out["l_aux"])[0]) - ref["l_aux"]) <= 1e-5 * abs(ref["l_aux"])
    y = host(out["y"])
    tol = TOL_OUT[dt]
    left = ref["slot"] < 0
    live = np.nonzero(~left)[0] if wl.d_ff_shared == 0 else np.arange(wl.T)
    if live.size:
        r = row_rel(y[live], ref["y"][live])
        assert r.max() <= tol, f"max row rel err {r.max():.3g} > {tol} (token {live[r.argmax()]})"
    if left.any() and wl.d_ff_shared == 0:
        xs = inp.x.view(np.uint32) if inp.x.dtype == np.float32 else inp.x
        np.testing.assert_array_equal(host_bits(out["y"])[left], xs[left])
    top1_drop = oracle.assign_slots(ref["first_choice"], ref["p"][np.arange(wl.T), ref["first_choice"]], wl.N, C,
                                    wl.priority)["n_dropped"]
    rerouted = int((ref["round"] > 0).sum())
    _say(f"  top-1 drops {top1_drop} -> {ref['n_dropped']} after re-routing {rerouted} tokens")
    return ref, out, layer, d


def test_expanded_tiny_fp32():
    _expand_case(workloads.WORKLOADS["switch-tiny-fp32"].with_(capacity_factor=0.9), 2)


def test_expanded_base_uniform():
    _expand_case(workloads.WORKLOADS["switch-base-uniform"], 2)


@pytest.mark.parametrize("cf,priority,gate_scale,M", [(0.5, "token", True, 2), (1.0, "gate", True, 2),
                                                      (0.5, "gate", False, 4), (1.0, "token", True, 8)])
def test_expanded_skewed(cf, priority, gate_scale, M):
    wl = workloads.WORKLOADS["switch-base-zipf"].with_(capacity_factor=cf, priority=priority, gate_scale=gate_scale)
    ref, *_ = _expand_case(wl, M)
    assert (ref["round"] > 0).sum() > 100  # the skewed router overflows, and re-routing takes many tokens


@pytest.mark.parametrize("M", [2, 8])
def test_expanded_decode(M):
    ref, *_ = _expand_case(workloads.WORKLOADS["switch-decode-384"], M)
    assert (ref["round"] > 0).sum() > 0


EDGE = [
    (_custom("x3-ragged-gate", 1000, 256, 384, 19, 0.8, seed=1, bias_scale=1.0, priority="gate"), 3, None),
    (_custom("x2-residual-shared", 384, 256, 256, 8, 0.9, seed=2, residual_all=True, d_ff_shared=256), 2, None),
    (_custom("x4-f32-odd", 301, 20, 36, 7, 0.7, dtype="f32", seed=3, priority="gate"), 4, None),
    (_custom("x4-all-candidates", 512, 128, 128, 4, 1.0, seed=4, bias_scale=3.0), 4, None),
    (_custom("x2-t1", 1, 128, 256, 4, 1.0, seed=5), 2, None),
    (_custom("x2-c1", 200, 128, 128, 64, 0.1, seed=6, bias_scale=2.0, priority="gate"), 2, None),
    (_custom("x3-big-t", 20000, 128, 128, 16, 0.5, seed=7, bias_scale=2.0), 3, None),
]


@pytest.mark.parametrize("wl,M,C", EDGE, ids=[w.name for w, _, _ in EDGE])
def test_expanded_edge(wl, M, C):
    ref, *_ = _expand_case(wl, M, C)
    if wl.name == "x4-all-candidates":  # M = N and N C >= T: nothing is left over
        assert ref["n_dropped"] == 0


def test_expand_one_is_the_top1_layer():
    """expand_choices = 1 is the Switch layer: bit-identical outputs."""
    wl = workloads.WORKLOADS["switch-base-zipf"].with_(capacity_factor=0.5)
    inp = inputs_util.conditioned_inputs(wl)
    d = _devs(inp, wl.dtype)
    a = {k: v.clone() for k, v in _run(_layer(wl, expand=1), d).items()}
    b = _run(_layer(wl), d)
    for k in a:
        np.testing.assert_array_equal(host_bits(a[k]), host_bits(b[k]), err_msg=k)


def test_expanded_without_overflow_is_the_top1_layer():
    """With C >= T no token overflows, so re-routing changes nothing: bit-identical outputs."""
    wl = _custom("x-no-overflow", 512, 128, 256, 8, 1.0, seed=8)
    inp = workloads.make_inputs(wl, bad_rows=inputs_util.topk_margin_bad_rows(3))
    d = _devs(inp, wl.dtype)
    a = {k: v.clone() for k, v in _run(_layer(wl, expand=3, C=512), d).items()}
    b = _run(_layer(wl, C=512), d)
    for k in a:
        np.testing.assert_array_equal(host_bits(a[k]), host_bits(b[k]), err_msg=k)


def test_expanded_repeat_deterministic():
    wl = workloads.WORKLOADS["switch-base-zipf"].with_(capacity_factor=0.5, priority="gate")
    inp = inputs_util.conditioned_inputs(wl)
    d = _devs(inp, wl.dtype)
    layer = _layer(wl, expand=3)
    a = {k: v.clone() for k, v in _run(layer, d).items()}
    b = _run(layer, d)
    for k in a:
        np.testing.assert_array_equal(host_bits(a[k]), host_bits(b[k]), err_msg=k)
