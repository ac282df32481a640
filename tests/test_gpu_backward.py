"""GPU parity of the layer backward (switch_moe_forward_train +
switch_moe_backward through the C ABI) against the fp64 backward oracle on
the same seeded inputs and the same seeded upstream gradient.

Bars (per row of each gradient, like the forward's outputs):
  max_k dist(g, [lo, hi]) / max_k |ref| <= 1e-4 (fp32) or 2e-2 (bf16),
where [lo, hi] is the oracle's envelope over the ReLU sign choices inside the
fp32 rounding band (lo = hi = ref away from it).  Gradients that must vanish
(experts that kept no token; the router with gate scaling off and no aux
gradient) must be exactly zero.  The forward outputs and the saved slot
tables must equal the plain forward's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import backward as ob
from tests import inputs_util
from tests.gpu_util import TOL_OUT, check_rows, dev, host, host_bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from switch_top_routed_amd import native

U32 = 2.0 ** -24


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _tdt(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def _prepare(wl, gate_cmax=None):
    inp = inputs_util.conditioned_inputs(wl, gate_order_cmax=gate_cmax)
    dt = wl.dtype
    d = dict(x=dev(inp.x, dt), w_gate=dev(inp.w_gate, dt), w1=dev(inp.w1, dt), w2=dev(inp.w2, dt),
             bias=None if inp.bias is None else torch.from_numpy(inp.bias).cuda(),
             ws1=dev(inp.ws1, dt), ws2=dev(inp.ws2, dt))
    dy = workloads.make_upstream(wl)
    return inp, d, dy


def _run(wl, d, dy, dl_aux, C=0):
    layer = native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=_tdt(wl), capacity_factor=wl.capacity_factor,
                             C=C, priority=wl.priority, gate_scale=wl.gate_scale, residual_all=wl.residual_all,
                             d_ff_shared=wl.d_ff_shared, train=True)
    kw = dict(bias=d["bias"], ws1=d["ws1"], ws2=d["ws2"])
    out = {k: v.clone() for k, v in layer.forward_train(d["x"], d["w_gate"], d["w1"], d["w2"], **kw).items()}
    dla = None if dl_aux is None else torch.tensor([dl_aux], dtype=torch.float32, device="cuda")
    g = layer.backward(d["x"], d["w_gate"], d["w1"], d["w2"], dev(dy, wl.dtype), dl_aux=dla, **kw)
    torch.cuda.synchronize()
    return layer, out, g


def _oracle(wl, inp, dy, dl_aux, C=None):
    dt = wl.dtype
    ref = oracle.moe_forward_stored(inp, C=C)
    x, wg = oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt)
    ws1 = oracle.widen(inp.ws1, dt) if inp.ws1 is not None else None
    ws2 = oracle.widen(inp.ws2, dt) if inp.ws2 is not None else None
    g = ob.moe_backward(ref, x, wg, lambda e: oracle.widen(inp.w1[e], dt), lambda e: oracle.widen(inp.w2[e], dt),
                        wl.N, oracle.widen(dy, dt), 0.0 if dl_aux is None else dl_aux, gate_scale=wl.gate_scale,
                        residual_all=wl.residual_all, ws1=ws1, ws2=ws2, kink_band_u=U32)
    return ref, g


def check_backward(wl, inp, dy, dl_aux, out, layer, g, ref, gref):
    tol = TOL_OUT[wl.dtype]
    # forward outputs and saved tables
    np.testing.assert_array_equal(host(out["expert_id"]), ref["expert_id"])
    np.testing.assert_array_equal(host(out["slot"]), ref["slot"])
    np.testing.assert_array_equal(host(out["kept_count"]), ref["kept_count"])
    sv = layer.saved
    np.testing.assert_array_equal(host(sv["token_of_slot"]), ref["token_of_slot"])
    na = int(host(sv["n_active"])[0])
    np.testing.assert_array_equal(host(sv["active"])[:na], ref["active"])
    np.testing.assert_allclose(host(sv["probs"]), ref["p"], rtol=1e-5, atol=1e-9)
    # saved hidden activations of the filled slots
    h = host(sv["h"])
    dt = wl.dtype
    x = oracle.widen(inp.x, dt)
    for e in ref["active"][:8]:
        k = ref["kept_count"][e]
        href = oracle.relu(x[ref["token_of_slot"][e, :k]] @ oracle.widen(inp.w1[e], dt))
        check_rows(f"h[{e}]", h[e, :k], href, tol)
    # gradients
    errs = {}
    errs["dx"] = check_rows("dx", host(g["dx"]), gref["dx"], tol, gref["dx_env"])
    errs["dw_gate"] = check_rows("dw_gate", host(g["dw_gate"]), gref["dw_gate"], tol)
    if inp.bias is not None:
        errs["dbias"] = check_rows("dbias", host(g["dbias"])[None, :], gref["dbias"][None, :], tol)
    errs["dw1"] = check_rows("dw1", host(g["dw1"]), gref["dw1"], tol, gref["dw1_env"])
    errs["dw2"] = check_rows("dw2", host(g["dw2"]), gref["dw2"], tol)
    if wl.d_ff_shared:
        errs["dws1"] = check_rows("dws1", host(g["dws1"]), gref["dws1"], tol, gref["dws1_env"])
        errs["dws2"] = check_rows("dws2", host(g["dws2"]), gref["dws2"], tol)
    _say(f"{wl.name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    return errs


def _case(wl, dl_aux=workloads.DL_AUX, gate_cmax=None, C=None):
    _say(f"{wl.name} T={wl.T} d={wl.d_model} dff={wl.d_ff} N={wl.N} cf={wl.capacity_factor} {wl.priority} "
         f"gs={wl.gate_scale} res={wl.residual_all} shared={wl.d_ff_shared} dl_aux={dl_aux}")
    inp, d, dy = _prepare(wl, gate_cmax)
    layer, out, g = _run(wl, d, dy, dl_aux, C=C or 0)
    ref, gref = _oracle(wl, inp, dy, dl_aux, C=C)
    return check_backward(wl, inp, dy, dl_aux, out, layer, g, ref, gref), (layer, out, g, ref, gref, d, dy)


def _custom(name, T, d, dff, N, cf, dtype="bf16", seed=0, **kw):
    import math
    return workloads.Workload(name, T, d, dff, N, cf, dtype, 1.0 / math.sqrt(d), seed=20_000 + seed, **kw)


# ---------------------------------------------------------------------------
def test_backward_tiny_fp32():
    _case(workloads.WORKLOADS["switch-tiny-fp32"])


def test_backward_tiny_fp32_flags():
    wl = workloads.WORKLOADS["switch-tiny-fp32"].with_(priority="gate", gate_scale=False, residual_all=True,
                                                       bias_scale=1.0)
    _case(wl, gate_cmax=64)


def test_backward_base_uniform():
    _case(workloads.WORKLOADS["switch-base-uniform"])


def test_backward_base_uniform_forward_unchanged():
    """forward_train gives the plain forward's outputs bit for bit."""
    wl = workloads.WORKLOADS["switch-base-uniform"]
    inp, d, dy = _prepare(wl)
    layer, out, g = _run(wl, d, dy, workloads.DL_AUX)
    plain = native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=_tdt(wl), capacity_factor=wl.capacity_factor)
    o2 = plain(d["x"], d["w_gate"], d["w1"], d["w2"])
    torch.cuda.synchronize()
    for k in ("y", "expert_id", "gate", "slot", "routed_count", "kept_count", "n_dropped", "f", "P", "l_aux"):
        np.testing.assert_array_equal(host_bits(out[k]), host_bits(o2[k]), err_msg=k)


def test_backward_deterministic():
    wl = workloads.WORKLOADS["switch-base-uniform"]
    inp, d, dy = _prepare(wl)
    _, _, g1 = _run(wl, d, dy, workloads.DL_AUX)
    g1 = {k: None if v is None else v.clone() for k, v in g1.items()}
    _, _, g2 = _run(wl, d, dy, workloads.DL_AUX)
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v.view(torch.uint8) if v.dtype != torch.float32 else v.view(torch.int32),
                               g2[k].view(torch.uint8) if v.dtype != torch.float32 else g2[k].view(torch.int32)), k


@pytest.mark.parametrize("cf,priority,gate_scale", [(0.5, "gate", True), (1.0, "token", False), (2.0, "gate", False),
                                                    (1.0, "token", True)])
def test_backward_zipf(cf, priority, gate_scale):
    wl = workloads.WORKLOADS["switch-base-zipf"].with_(capacity_factor=cf, priority=priority, gate_scale=gate_scale)
    C = oracle.capacity(wl.T, wl.N, cf)
    _case(wl, gate_cmax=C if priority == "gate" else None)


def test_backward_no_router_gradient_is_exact_zero():
    """Gate scaling off and no aux gradient: dW_g, db and the router part of dx vanish."""
    wl = workloads.WORKLOADS["switch-base-zipf"].with_(capacity_factor=1.0, gate_scale=False)
    errs, (layer, out, g, ref, gref, d, dy) = _case(wl, dl_aux=None)
    assert not torch.any(g["dw_gate"]) and not torch.any(g["dbias"])
    drop = np.nonzero(ref["slot"] < 0)[0]
    np.testing.assert_array_equal(host_bits(g["dx"])[drop], dy[drop])


EDGE = [
    _custom("ragged", 1000, 256, 384, 12, 1.1, seed=1),
    _custom("t1", 1, 128, 256, 4, 1.0, seed=2),
    _custom("n1-dense", 200, 128, 256, 1, 1.0, seed=3),
    _custom("n-not-16", 700, 128, 128, 19, 0.9, seed=4, bias_scale=1.0),
    _custom("f32-odd", 301, 20, 36, 7, 1.3, dtype="f32", seed=5),
    _custom("residual", 512, 256, 256, 8, 0.8, seed=6, residual_all=True),
    _custom("shared", 384, 256, 512, 8, 1.0, seed=7, d_ff_shared=256),
    _custom("shared-dense-tiles", 640, 512, 256, 8, 1.0, seed=14, d_ff_shared=768),
    _custom("shared-generic", 300, 256, 256, 8, 1.0, seed=15, d_ff_shared=256),
    _custom("tiled-c150", 1200, 256, 512, 8, 1.0, seed=13, bias_scale=0.5),
    # C = 154 with skewed routing: the 10-tile fused passes with experts from 16 kept rows
    # to full ones
    _custom("c154-two-classes", 1400, 256, 512, 10, 1.1, seed=16, bias_scale=1.0),
    # the 10-tile fused passes with d and d_ff multiples of 512 (uniform, and skewed with
    # ragged kept counts and full experts)
    _custom("split-c150", 1200, 512, 1024, 8, 1.0, seed=17, bias_scale=0.5),
    _custom("split-c154-skewed", 1400, 512, 1024, 10, 1.1, seed=18, bias_scale=1.0),
]


@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_backward_edge(wl):
    _case(wl)


def check_streaming(wl, inp, dy, dl_aux, g, experts):
    """The backward oracle step by step (combine, each expert, router), checking
    each listed expert's weight gradients as it goes, then dx, dW_g and db; the
    fp64 weight gradients of all experts are never held at once."""
    dt, tol = wl.dtype, TOL_OUT[wl.dtype]
    ref = oracle.moe_forward_stored(inp)
    x, wg = oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt)
    d_out, dg, dx = ob.combine_backward(oracle.widen(dy, dt), ref["out"], ref["expert_id"], ref["slot"],
                                        ref["gate"], wl.gate_scale, wl.residual_all)
    dx_lo, dx_hi = np.zeros_like(dx), np.zeros_like(dx)
    for e in ref["active"]:
        k = int(ref["kept_count"][e])
        toks = ref["token_of_slot"][e, :k]
        d_rows, dw1, dw2, _, env = ob.ffn_backward(x[toks], d_out[e, :k], oracle.widen(inp.w1[e], dt),
                                                   oracle.widen(inp.w2[e], dt), U32)
        dx[toks] += d_rows
        dx_lo[toks] += env["d_rows"][0] - d_rows
        dx_hi[toks] += env["d_rows"][1] - d_rows
        if e in experts:
            check_rows(f"dw1[{e}]", host(g["dw1"][int(e)]), dw1, tol, env["dw1"])
            check_rows(f"dw2[{e}]", host(g["dw2"][int(e)]), dw2, tol)
    _, dwg, db, dx_r = ob.router_backward(x, wg, ref["p"], ref["expert_id"], dg, ref["f"], dl_aux)
    dx += dx_r
    check_rows("dx", host(g["dx"]), dx, tol, (dx + dx_lo, dx + dx_hi))
    check_rows("dw_gate", host(g["dw_gate"]), dwg, tol)
    if inp.bias is not None:
        check_rows("dbias", host(g["dbias"])[None, :], db[None, :], tol)
    return ref


def test_backward_decode():
    """384 experts, C = 1, ~14 experts active: the inactive experts' weight
    gradients must be exactly zero (checked on the device), the active ones and
    every other gradient against the oracle."""
    wl = workloads.WORKLOADS["switch-decode-384"]
    _say(wl.name)
    inp, d, dy = _prepare(wl)
    layer, out, g = _run(wl, d, dy, workloads.DL_AUX)
    ref = check_streaming(wl, inp, dy, workloads.DL_AUX, g, experts=set(range(wl.N)))
    inactive = torch.ones(wl.N, dtype=torch.bool, device="cuda")
    inactive[torch.from_numpy(ref["active"].astype(np.int64)).cuda()] = False
    assert not torch.any(g["dw1"][inactive]) and not torch.any(g["dw2"][inactive])


@pytest.mark.parametrize("name", ["switch-decode-384", "switch-base-uniform", "tiled-c150"])
def test_backward_accumulate_expert_grads(name):
    """SWITCH_ACCUM_EXPERT_GRADS: dw1 / dw2 start from seeded prior gradients R;
    after the backward, every expert that kept a token holds R + its gradient
    (same bar, envelope shifted by R) and every other expert still holds R bit
    for bit; dx, dW_g and db are the plain backward's.  tiled-c150 (C = 150)
    runs the fused passes at their largest row count (10 row tiles)."""
    wl = workloads.WORKLOADS[name] if name in workloads.WORKLOADS else {w.name: w for w in EDGE}[name]
    _say(f"{wl.name} accumulate")
    dt, tol = wl.dtype, TOL_OUT[wl.dtype]
    inp, d, dy = _prepare(wl)
    ref = oracle.moe_forward_stored(inp)
    x = oracle.widen(inp.x, dt)
    d_out, _, _ = ob.combine_backward(oracle.widen(dy, dt), ref["out"], ref["expert_id"], ref["slot"], ref["gate"],
                                      wl.gate_scale, wl.residual_all)
    grads = {}
    for e in ref["active"]:
        k = int(ref["kept_count"][e])
        _, dw1, dw2, _, env = ob.ffn_backward(x[ref["token_of_slot"][e, :k]], d_out[e, :k],
                                              oracle.widen(inp.w1[e], dt), oracle.widen(inp.w2[e], dt), U32)
        grads[int(e)] = (dw1, dw2, env["dw1"])
    # prior gradients: N(0, 1) scaled to the largest gradient magnitude (so both terms count), bf16
    scale = max(max(np.abs(a).max(), np.abs(b).max()) for a, b, _ in grads.values())
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    layer = native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=_tdt(wl), capacity_factor=wl.capacity_factor,
                             priority=wl.priority, gate_scale=wl.gate_scale, residual_all=wl.residual_all,
                             train=True, accumulate_expert_grads=True)
    R1 = (torch.randn(layer.grads["dw1"].shape, generator=gen, device="cuda") * scale).to(_tdt(wl))
    R2 = (torch.randn(layer.grads["dw2"].shape, generator=gen, device="cuda") * scale).to(_tdt(wl))
    layer.grads["dw1"].copy_(R1)
    layer.grads["dw2"].copy_(R2)
    kw = dict(bias=d["bias"])
    layer.forward_train(d["x"], d["w_gate"], d["w1"], d["w2"], **kw)
    dla = torch.tensor([workloads.DL_AUX], dtype=torch.float32, device="cuda")
    g = layer.backward(d["x"], d["w_gate"], d["w1"], d["w2"], dev(dy, dt), dl_aux=dla, **kw)
    torch.cuda.synchronize()
    idle = torch.ones(wl.N, dtype=torch.bool, device="cuda")
    idle[torch.from_numpy(ref["active"].astype(np.int64)).cuda()] = False
    assert torch.equal(g["dw1"][idle].view(torch.int16), R1[idle].view(torch.int16))
    assert torch.equal(g["dw2"][idle].view(torch.int16), R2[idle].view(torch.int16))
    worst = 0.0
    for e, (dw1, dw2, env1) in grads.items():
        r1, r2 = host(R1[e]), host(R2[e])
        worst = max(worst, check_rows(f"dw1[{e}]", host(g["dw1"][e]), r1 + dw1, tol, (r1 + env1[0], r1 + env1[1])))
        worst = max(worst, check_rows(f"dw2[{e}]", host(g["dw2"][e]), r2 + dw2, tol))
    _say(f"{wl.name} accumulate: {len(grads)} active experts, max row rel err {worst:.2e}")
    # the other gradients are the plain backward's
    check_streaming(wl, inp, dy, workloads.DL_AUX, g, experts=set())


def test_backward_accumulate_refused_on_generic_path():
    """The flag needs the fused bf16 expert backward; the fp32 layer is refused before any launch."""
    wl = workloads.WORKLOADS["switch-tiny-fp32"]
    inp, d, dy = _prepare(wl)
    layer = native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=torch.float32, capacity_factor=wl.capacity_factor,
                             train=True, accumulate_expert_grads=True)
    layer.forward_train(d["x"], d["w_gate"], d["w1"], d["w2"])
    with pytest.raises(native.SwitchError) as ei:
        layer.backward(d["x"], d["w_gate"], d["w1"], d["w2"], dev(dy, wl.dtype))
    assert ei.value.status == 3
