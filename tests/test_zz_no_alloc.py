"""switch_moe_forward_noalloc (the forward on the library's own scratch array,
for callers that cannot allocate) against switch_moe_forward on the same
inputs: every output bit-identical (the same kernels run on a different
workspace), on two calls in a row -- the base-scale layer, then a smaller
skewed layer with gate-descending priority -- and a workspace larger than the
array is refused before anything runs."""
import ctypes

import pytest
import torch

import workloads
from tests import inputs_util
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _pair(wl, gate_cmax=None):
    from switch_top_routed_amd import native
    inp = inputs_util.conditioned_inputs(wl, gate_order_cmax=gate_cmax)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    d = {k: dev(getattr(inp, k), wl.dtype) for k in ("x", "w_gate", "w1", "w2")}
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    mk = lambda: native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=dt,  # noqa: E731
                                  capacity_factor=wl.capacity_factor, priority=wl.priority,
                                  gate_scale=wl.gate_scale)
    a, b = mk(), mk()
    for layer in (a, b):  # poison the outputs: every element must be written
        for v in layer.out.values():
            v.view(torch.uint8).fill_(0xA5)
    a(d["x"], d["w_gate"], d["w1"], d["w2"], bias=bias)
    b(d["x"], d["w_gate"], d["w1"], d["w2"], bias=bias, noalloc=True)
    torch.cuda.synchronize()
    for k in a.out:
        ta, tb = a.out[k], b.out[k]
        assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8)), f"{wl.name}: output {k} differs"
    return a.out


def test_noalloc_matches_forward_two_calls():
    from switch_top_routed_amd import native
    L = native.lib()
    assert L.switch_moe_noalloc_max_bytes() == 64 << 20
    print("[case] noalloc: base-uniform", flush=True)
    wl1 = workloads.WORKLOADS["switch-base-uniform"]
    _pair(wl1)
    print("[case] noalloc: smaller skewed layer, gate-descending", flush=True)
    wl2 = workloads.Workload("noalloc-small", 1000, 256, 512, 24, 1.0, "bf16", 1.0 / 16.0, bias_scale=1.0,
                             priority="gate", seed=31_337)
    out = _pair(wl2, gate_cmax=64)
    assert int(out["n_dropped"].item()) > 0  # the skewed layer drops tokens: the slot path is exercised


def test_noalloc_rejects_large_workspace():
    from switch_top_routed_amd import native
    L = native.lib()
    wl = workloads.WORKLOADS["switch-large-shared"]
    desc = native.SwitchMoeDesc(T=wl.T, d_model=wl.d_model, d_ff=wl.d_ff, N=wl.N, C=0,
                                capacity_factor=wl.capacity_factor, dtype=native.BF16, priority=0,
                                flags=native.GATE_SCALE, d_ff_shared=wl.d_ff_shared, top_k=1, routing=0,
                                weight_format=0, expand_choices=1)
    assert L.switch_moe_workspace_bytes(ctypes.byref(desc)) > L.switch_moe_noalloc_max_bytes()
    # refused on the size alone, before the (NULL) inputs are looked at or anything is enqueued
    rc = L.switch_moe_forward_noalloc(ctypes.byref(desc), None, None, None)
    assert rc == 4, rc  # SWITCH_E_WORKSPACE
    assert b"scratch array" in L.switch_last_error()
