"""GPU parity: every stage and the whole layer, through the C ABI, against the
fp64 oracle on the same seeded inputs.

Covers the tiny fp32 layer, the base-scale uniform layer (stage by stage),
the 12-run skewed-routing matrix, the 384-expert decode batch, and edge cases
(ragged T, T = 1, a single expert, all tokens to one expert, N not a multiple
of 16, ~1000 experts, one expert holding more than 8192 tokens under
gate-descending priority, fp32 with odd sizes).  Determinism and
NaN-poisoned buffers/workspace are checked on the base-scale layer.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import inputs_util
from tests.gpu_util import (TOL_OUT, check_output, check_routing, check_slots, dev, host, host_bits, row_rel)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import switch_top_routed_amd as sw
    from switch_top_routed_amd import native


def _say(msg):
    print(f"[case] {msg}", flush=True)


_CACHE = {}


def prepared(wl, gate_cmax=None):
    """(inputs, device tensors) for a workload; cached per process."""
    key = (wl, gate_cmax)
    if key not in _CACHE:
        inp = inputs_util.conditioned_inputs(wl, gate_order_cmax=gate_cmax)
        dt = wl.dtype
        d = dict(x=dev(inp.x, dt), w_gate=dev(inp.w_gate, dt), w1=dev(inp.w1, dt), w2=dev(inp.w2, dt),
                 bias=None if inp.bias is None else torch.from_numpy(inp.bias).cuda(),
                 ws1=dev(inp.ws1, dt), ws2=dev(inp.ws2, dt))
        _CACHE[key] = (inp, d)
    return _CACHE[key]


def run_layer(wl, d, priority=None, gate_scale=None, cf=None, poison=False):
    T, dm, dff, N = wl.T, wl.d_model, wl.d_ff, wl.N
    layer = native.SwitchMoE(T, dm, dff, N, dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32,
                             capacity_factor=wl.capacity_factor if cf is None else cf,
                             priority=wl.priority if priority is None else priority,
                             gate_scale=wl.gate_scale if gate_scale is None else gate_scale,
                             residual_all=wl.residual_all, d_ff_shared=wl.d_ff_shared)
    if poison:
        layer.ws.fill_(255)
        for v in layer.out.values():
            v.view(torch.uint8).fill_(255)
    out = layer(d["x"], d["w_gate"], d["w1"], d["w2"], bias=d["bias"], ws1=d["ws1"], ws2=d["ws2"])
    torch.cuda.synchronize()
    return layer, out


def check_layer(wl, inp, out, ref):
    check_routing(out, ref, wl.N)
    check_slots(out, ref)
    check_output(out["y"], ref, inp.x, wl.dtype, shared=wl.d_ff_shared > 0)


# ---------------------------------------------------------------------------
# tiny fp32 layer
# ---------------------------------------------------------------------------
def test_tiny_fp32_layer():
    wl = workloads.WORKLOADS["switch-tiny-fp32"]
    _say(wl.name)
    inp, d = prepared(wl)
    ref = oracle.moe_forward_stored(inp)
    layer, out = run_layer(wl, d)
    assert layer.C == ref["C"] == 32
    check_layer(wl, inp, out, ref)


def test_tiny_fp32_gate_desc_unscaled():
    wl = workloads.WORKLOADS["switch-tiny-fp32"].with_(priority="gate", gate_scale=False)
    _say(wl.name + " gate-desc unscaled")
    inp, d = prepared(wl, gate_cmax=32)
    ref = oracle.moe_forward_stored(inp)
    _, out = run_layer(wl, d)
    check_layer(wl, inp, out, ref)


# ---------------------------------------------------------------------------
# base-scale uniform layer, stage by stage
# ---------------------------------------------------------------------------
BASE = "switch-base-uniform"


@pytest.fixture(scope="module")
def base():
    wl = workloads.WORKLOADS[BASE]
    inp, d = prepared(wl)
    ref = oracle.moe_forward_stored(inp)
    return wl, inp, d, ref


def test_base_route(base):
    wl, inp, d, ref = base
    _say("base route")
    o = sw.switch_route(d["x"], d["w_gate"], d["bias"])
    torch.cuda.synchronize()
    check_routing(o, ref, wl.N)


@pytest.mark.parametrize("priority", ["token", "gate"])
def test_base_assign(base, priority):
    wl, inp, d, ref0 = base
    _say(f"base assign {priority}")
    gate32 = ref0["gate"].astype(np.float32)
    ref = oracle.assign_slots(ref0["expert_id"], gate32.astype(np.float64), wl.N, ref0["C"], priority)
    o = sw.switch_assign_capacity(torch.from_numpy(ref0["expert_id"]).cuda(), torch.from_numpy(gate32).cuda(), wl.N,
                                  ref0["C"], priority)
    torch.cuda.synchronize()
    check_slots(o, ref)


def test_base_dispatch(base):
    wl, inp, d, ref = base
    _say("base dispatch")
    tos = torch.from_numpy(ref["token_of_slot"]).cuda()
    kept = torch.from_numpy(ref["kept_count"]).cuda()
    buf = torch.full((wl.N, ref["C"], wl.d_model), float("nan"), dtype=torch.bfloat16, device="cuda")
    sw.switch_dispatch(d["x"], tos, kept, wl.N, ref["C"], expert_in=buf)
    torch.cuda.synchronize()
    bits = host_bits(buf)
    for e in range(wl.N):
        k = ref["kept_count"][e]
        np.testing.assert_array_equal(bits[e, :k], inp.x[ref["token_of_slot"][e, :k]])
        assert (bits[e, k:] == 0x7FC0).all()  # empty slots untouched


def _buf_from_ref(ref, x_stored, N, C, d_model, dtype):
    """Stored-dtype [N, C, d] buffer built from the oracle's slot map; empty slots NaN."""
    if dtype == "bf16":
        b = np.full((N, C, d_model), 0x7FC0, dtype=np.uint16)
    else:
        b = np.full((N, C, d_model), np.nan, dtype=np.float32)
    for e in range(N):
        k = ref["kept_count"][e]
        b[e, :k] = x_stored[ref["token_of_slot"][e, :k]]
    return b


def test_base_expert_ffn(base):
    wl, inp, d, ref = base
    _say("base expert ffn")
    C = ref["C"]
    buf = dev(_buf_from_ref(ref, inp.x, wl.N, C, wl.d_model, "bf16"), "bf16")
    out = torch.full_like(buf, float("nan"))
    kept = torch.from_numpy(ref["kept_count"]).cuda()
    act = torch.zeros(wl.N, dtype=torch.int32)
    act[: len(ref["active"])] = torch.from_numpy(ref["active"])
    nact = torch.tensor([len(ref["active"])], dtype=torch.int32)
    sw.switch_expert_ffn(buf, d["w1"], d["w2"], kept, act.cuda(), nact.cuda(), expert_out=out)
    torch.cuda.synchronize()
    o = host(out)
    for e in range(wl.N):
        k = ref["kept_count"][e]
        if k:
            r = row_rel(o[e, :k], ref["out"][e, :k])
            assert r.max() <= TOL_OUT["bf16"], (e, r.max())
        assert np.isnan(o[e, k:]).all()  # rows beyond kept_count are not written


@pytest.mark.parametrize("flags", [native.GATE_SCALE if torch.cuda.is_available() else 1, 0, 3])
def test_base_combine(base, flags):
    wl, inp, d, ref = base
    _say(f"base combine flags={flags}")
    C = ref["C"]
    outb = np.full((wl.N, C, wl.d_model), np.nan)
    for e in range(wl.N):
        k = ref["kept_count"][e]
        outb[e, :k] = ref["out"][e, :k]
    eo = dev(workloads.f32_to_bf16_bits(outb.astype(np.float32)), "bf16")
    y = sw.switch_combine(eo, d["x"], torch.from_numpy(ref["expert_id"]).cuda(), torch.from_numpy(ref["slot"]).cuda(),
                          torch.from_numpy(ref["gate"].astype(np.float32)).cuda(), flags)
    torch.cuda.synchronize()
    x = oracle.widen(inp.x, "bf16")
    yref = oracle.combine(ref["out"], x, ref["expert_id"], ref["slot"], ref["gate"], gate_scale=bool(flags & 1),
                          residual_all=bool(flags & 2))
    check_output(y, dict(slot=ref["slot"], y=yref), inp.x, "bf16")


def test_base_layer(base):
    wl, inp, d, ref = base
    _say("base layer")
    _, out = run_layer(wl, d)
    check_layer(wl, inp, out, ref)


def test_base_layer_deterministic_and_poison_proof(base):
    wl, inp, d, ref = base
    _say("base layer determinism + NaN-poisoned workspace")
    _, o1 = run_layer(wl, d)
    a = {k: host_bits(v).copy() for k, v in o1.items()}
    _, o2 = run_layer(wl, d, poison=True)
    for k, v in o2.items():
        np.testing.assert_array_equal(host_bits(v), a[k], err_msg=k)


def _staged_layer(wl, d, C, priority="token", gate_scale=True):
    """The layer composed from the per-stage entry points (router, assignment,
    dispatch, expert FFN, the shared expert as a one-expert FFN over all tokens,
    combine), for comparison with switch_moe_forward."""
    r = sw.switch_route(d["x"], d["w_gate"], d["bias"])
    a = sw.switch_assign_capacity(r["expert_id"], r["gate"], wl.N, C, priority)
    xin = sw.switch_dispatch(d["x"], a["token_of_slot"], a["kept_count"], wl.N, C)
    xout = sw.switch_expert_ffn(xin, d["w1"], d["w2"], a["kept_count"], a["active"], a["n_active"])
    shared = None
    if wl.d_ff_shared:
        T, dm, fs = wl.T, wl.d_model, wl.d_ff_shared
        one = lambda v: torch.tensor([v], dtype=torch.int32, device="cuda")
        shared = sw.switch_expert_ffn(d["x"].view(1, T, dm), d["ws1"].view(1, dm, fs), d["ws2"].view(1, fs, dm),
                                      one(T), one(0), one(1)).view(T, dm)
    flags = (native.GATE_SCALE if gate_scale else 0) | (native.RESIDUAL_ALL if wl.residual_all else 0)
    y = sw.switch_combine(xout, d["x"], r["expert_id"], a["slot"], r["gate"], flags, shared_out=shared)
    torch.cuda.synchronize()
    return dict(r, **a, y=y)


def test_base_layer_matches_staged_path(base):
    """switch_moe_forward (token order: slots from the router's tiles, GEMM 1
    gathering x rows) is bit-identical to the composition of the per-stage entry
    points (separate assignment kernels and an explicit dispatch copy)."""
    wl, inp, d, ref = base
    _say("base layer vs staged path")
    layer, o = run_layer(wl, d)
    st = _staged_layer(wl, d, layer.C)
    for k in ("y", "expert_id", "gate", "slot", "kept_count", "routed_count", "f", "P", "l_aux", "n_dropped"):
        np.testing.assert_array_equal(host_bits(o[k]), host_bits(st[k]), err_msg=k)


@pytest.mark.parametrize("name", ["ragged", "f32-odd", "n1000", "tiled-c150", "tiled-c150-wide", "f32-many-tiles",
                                  "shared-drops", "shared-residual", "shared-gate-noscale"])
def test_edge_layer_matches_staged_path(name):
    wl = next(w for w in EDGE if w.name == name)
    _say(f"edge layer vs staged path {name}")
    inp, d = prepared(wl)
    layer, o = run_layer(wl, d)
    st = _staged_layer(wl, d, layer.C, priority=wl.priority, gate_scale=wl.gate_scale)
    for k in ("y", "expert_id", "gate", "slot", "kept_count", "routed_count", "f", "P", "l_aux", "n_dropped"):
        np.testing.assert_array_equal(host_bits(o[k]), host_bits(st[k]), err_msg=k)


def test_base_layer_timed_matches_untimed(base):
    """switch_moe_forward_timed: same outputs bit for bit, stage events in order."""
    wl, inp, d, ref = base
    _say("base layer with stage events")
    layer, o1 = run_layer(wl, d)
    a = {k: host_bits(v).copy() for k, v in o1.items()}
    ev = native.StageEvents()
    layer(d["x"], d["w_gate"], d["w1"], d["w2"], bias=d["bias"], stage_events=ev)
    torch.cuda.synchronize()
    for k, v in layer.out.items():
        np.testing.assert_array_equal(host_bits(v), a[k], err_msg=k)
    spans = [ev.ms(i, i + 1) for i in range(ev.N - 1)]
    assert all(s >= 0.0 for s in spans), spans
    assert ev.ms(3, 4) > 0.0  # the routed expert FFN takes time


# ---------------------------------------------------------------------------
# skewed routing: capacity factor x priority x gate scaling
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cf,priority,gate_scale", workloads.ZIPF_MATRIX)
def test_zipf_matrix(cf, priority, gate_scale):
    wl = workloads.WORKLOADS["switch-base-zipf"].with_(capacity_factor=cf, priority=priority, gate_scale=gate_scale)
    _say(f"zipf cf={cf} {priority} scale={gate_scale}")
    base_wl = workloads.WORKLOADS["switch-base-zipf"]
    inp, d = prepared(base_wl, gate_cmax=64)
    inp.wl = wl
    ref = oracle.moe_forward_stored(inp)
    _, out = run_layer(wl, d)
    check_layer(wl, inp, out, ref)
    assert ref["n_dropped"] > 0.5 * wl.T  # the skew really overflows the hot experts


# ---------------------------------------------------------------------------
# decode-shaped layer: 384 experts, 128 tokens, C = 1
# ---------------------------------------------------------------------------
def test_decode_384():
    wl = workloads.WORKLOADS["switch-decode-384"]
    _say(wl.name)
    inp, d = prepared(wl)
    ref = oracle.moe_forward_stored(inp)
    assert ref["C"] == 1
    _, out = run_layer(wl, d)
    check_layer(wl, inp, out, ref)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def _custom(name, T, d, dff, N, cf, dtype="bf16", seed=0, **kw):
    std = 0.1 if dtype == "f32" else 1.0 / np.sqrt(d)
    return workloads.Workload(name, T, d, dff, N, cf, dtype, std, seed=seed, **kw)


EDGE = [
    _custom("ragged", 1000, 256, 384, 16, 1.0, seed=1),
    _custom("one-token", 1, 128, 128, 4, 1.0, seed=2),
    _custom("dense-one-expert", 300, 128, 256, 1, 1.0, seed=3),
    _custom("n37", 2048, 256, 256, 37, 1.25, seed=4, bias_scale=0.5),
    _custom("n1000", 2048, 128, 128, 1000, 2.0, seed=5),
    _custom("f32-odd", 77, 12, 20, 5, 0.8, dtype="f32", seed=6),
    _custom("ragged-gate", 1000, 256, 384, 16, 0.5, seed=7, priority="gate", gate_scale=False),
    _custom("residual", 700, 128, 256, 8, 1.0, seed=8, residual_all=True),
    _custom("tiled-c90", 720, 256, 512, 8, 1.0, seed=15, bias_scale=0.4),      # C = 90: 96 x 256 tiles
    _custom("tiled-c128", 2048, 256, 512, 16, 1.0, seed=11, bias_scale=0.3),   # C > 64: LDS-tiled GEMM, 128 x 256 tiles
    _custom("tiled-c150", 1200, 256, 512, 8, 1.0, seed=13, bias_scale=0.5),     # C = 150: 160 x 512 (GEMM 1), 160 x 256 tiles
    _custom("tiled-c150-wide", 1200, 512, 1536, 8, 1.0, seed=16, bias_scale=0.5),  # C = 150: 160 x 512 tiles on 8 waves, both GEMMs
    _custom("tiled-c180", 1440, 512, 256, 8, 1.0, seed=14, priority="gate"),    # C = 180: two 128-row m-chunks
    _custom("tiled-c200", 1600, 512, 256, 8, 1.0, seed=12, priority="gate"),    # C = 200: two 128-row m-chunks
    # a shared expert on the tiled GEMM: its second GEMM also does the combine (dropped
    # tokens, the residual flag, gate order without gate scaling)
    _custom("shared-drops", 1000, 256, 384, 16, 0.5, seed=21, d_ff_shared=256),
    _custom("shared-residual", 700, 256, 256, 8, 0.5, seed=22, residual_all=True, d_ff_shared=512),
    _custom("shared-gate-noscale", 900, 256, 256, 8, 0.8, seed=23, priority="gate", gate_scale=False,
            d_ff_shared=256),
    # token-order assignment: 1250 router tiles (two LDS chunks of partials), one tile
    # group per expert (N = 1024), tokens in two 16K chunks
    _custom("f32-many-tiles", 20000, 32, 64, 1024, 1.0, dtype="f32", seed=16),
]


@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_edge_layer(wl):
    _say(f"edge {wl.name}")
    C = oracle.capacity(wl.T, wl.N, wl.capacity_factor)
    inp, d = prepared(wl, gate_cmax=C if wl.priority == "gate" else None)
    ref = oracle.moe_forward_stored(inp)
    _, out = run_layer(wl, d)
    check_layer(wl, inp, out, ref)


@pytest.mark.parametrize("priority", ["token", "gate"])
def test_all_tokens_to_one_expert(priority):
    """A +30 router bias sends every token to expert 3.  Every fp32 gate is then
    exactly 1.0 (the other probabilities are ~1e-13), so gate-descending order
    degenerates to token order; the expected slots are taken on the fp32 gates."""
    wl = _custom("all-to-one", 512, 128, 128, 8, 1.0, seed=9, priority=priority)
    _say(f"all-to-one {priority}")
    inp = workloads.make_inputs(wl)
    inp.bias = np.zeros(8, np.float32)
    inp.bias[3] = 30.0
    d = dict(x=dev(inp.x, "bf16"), w_gate=dev(inp.w_gate, "bf16"), w1=dev(inp.w1, "bf16"), w2=dev(inp.w2, "bf16"),
             bias=torch.from_numpy(inp.bias).cuda(), ws1=None, ws2=None)
    ref = oracle.moe_forward_stored(inp)
    g32 = ref["gate"].astype(np.float32)
    assert (g32 == 1.0).all()
    ref.update(oracle.assign_slots(ref["expert_id"], g32.astype(np.float64), 8, ref["C"], priority))
    assert ref["kept_count"].tolist() == [0, 0, 0, 64, 0, 0, 0, 0] and ref["n_dropped"] == 448
    _, out = run_layer(wl, d)
    check_routing(out, ref, wl.N)
    check_slots(out, ref)
    kept = ref["slot"] >= 0
    assert (ref["slot"][kept] == np.arange(64)).all() and kept[:64].all()


@pytest.mark.parametrize("N,bias0", [(1, 0.0), (2, 2.5)])
def test_gate_desc_group_beyond_lds_sort(N, bias0):
    """One expert receives > 8192 tokens: the counting path of the gate-descending
    ranking.  N = 1: all gates are exactly 1 (ties resolve to token order);
    N = 2: gates spread over (0.5, 1), conditioned to relative gaps >= 1e-6."""
    wl = _custom(f"big-group-{N}", 9000, 128, 128, N, 1.0, seed=10, priority="gate")
    _say(f"gate-desc group > 8192, N={N}")
    inp = workloads.make_inputs(wl, weights=False)
    inp.bias = np.array([bias0] + [0.0] * (N - 1), np.float32)
    C = oracle.capacity(wl.T, wl.N, 0.5)
    if N > 1:
        workloads.resample_rows(inp, inputs_util.gate_gap_bad_rows(C, gap=1e-6))
    x = oracle.widen(inp.x, "bf16")
    _, p, e, g = oracle.route(x, oracle.widen(inp.w_gate, "bf16"), inp.bias)
    cnt, f, P, l_aux = oracle.aux_loss(e, p, N)
    ref = dict(expert_id=e, gate=g, routed_count=cnt, f=f, P=P, l_aux=l_aux)
    ref.update(oracle.assign_slots(e, g, N, C, "gate"))
    assert ref["routed_count"][0] > 8192
    o = sw.switch_route(dev(inp.x, "bf16"), dev(inp.w_gate, "bf16"), torch.from_numpy(inp.bias).cuda())
    a = sw.switch_assign_capacity(o["expert_id"], o["gate"], wl.N, C, "gate")
    torch.cuda.synchronize()
    check_routing(o, ref, wl.N)
    check_slots(a, ref)


def test_dense_ffn_matches_numpy():
    """A dense FFN through switch_expert_ffn (N = 1, C = M) against a float64 einsum."""
    _say("dense ffn via expert ffn")
    rng = np.random.default_rng(0)
    M, dm, dff = 1000, 256, 512
    x = workloads.f32_to_bf16_bits(rng.standard_normal((1, M, dm)).astype(np.float32))
    w1 = workloads.f32_to_bf16_bits((rng.standard_normal((1, dm, dff)) / np.sqrt(dm)).astype(np.float32))
    w2 = workloads.f32_to_bf16_bits((rng.standard_normal((1, dff, dm)) / np.sqrt(dff)).astype(np.float32))
    out = sw.switch_expert_ffn(dev(x, "bf16"), dev(w1, "bf16"), dev(w2, "bf16"),
                               torch.tensor([M], dtype=torch.int32, device="cuda"),
                               torch.tensor([0], dtype=torch.int32, device="cuda"),
                               torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    xf, w1f, w2f = (oracle.widen(a, "bf16") for a in (x, w1, w2))
    h = np.einsum("md,df->mf", xf[0], w1f[0])
    ref = np.einsum("mf,fd->md", np.maximum(h, 0), w2f[0])
    r = row_rel(host(out)[0], ref)
    assert r.max() <= TOL_OUT["bf16"], r.max()
