"""GPU parity on the large layer with a shared expert (T=16384, d=5120,
d_ff=8192, N=128, cf=1.25 -> C=160, plus one always-on dense FFN of width
8192).

The routed and shared weights (~22 GB of bf16) are drawn on the device with
torch's seeded generator; x and W_g are drawn on the host and conditioned to a
top-2 logit margin >= 1e-3.  Routing, load statistics, slots and counts are
checked in full against the fp64 oracle; the layer output is checked on every
kept token of a seeded sample of experts and on a sample of dropped tokens,
with the oracle evaluating those tokens one expert at a time from the
weights copied back to the host.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import inputs_util
from tests.gpu_util import TOL_OUT, check_routing, check_slots, dev, host, row_rel

pytestmark = pytest.mark.gpu


def _host_bf16(t):
    return oracle.widen(t.detach().cpu().view(torch.int16).numpy().view(np.uint16), "bf16")


def test_large_shared_layer():
    import switch_top_routed_amd as sw
    from switch_top_routed_amd import native

    wl = workloads.WORKLOADS["switch-large-shared"]
    print("[case] switch-large-shared: inputs", flush=True)
    inp = inputs_util.conditioned_inputs(wl, weights=False)
    W = workloads.make_device_weights(wl)
    x = dev(inp.x, "bf16")
    wg = dev(inp.w_gate, "bf16")
    print("[case] switch-large-shared: layer", flush=True)
    layer = native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=torch.bfloat16,
                             capacity_factor=wl.capacity_factor, d_ff_shared=wl.d_ff_shared)
    out = layer(x, wg, W["w1"], W["w2"], ws1=W["ws1"], ws2=W["ws2"])
    torch.cuda.synchronize()

    print("[case] switch-large-shared: oracle routing", flush=True)
    xf = oracle.widen(inp.x, "bf16")
    _, p, e, g = oracle.route(xf, oracle.widen(inp.w_gate, "bf16"), inp.bias)
    cnt, f, P, l_aux = oracle.aux_loss(e, p, wl.N)
    C = oracle.capacity(wl.T, wl.N, wl.capacity_factor)
    assert layer.C == C == 160
    ref = dict(expert_id=e, gate=g, routed_count=cnt, f=f, P=P, l_aux=l_aux)
    ref.update(oracle.assign_slots(e, g, wl.N, C))
    check_routing(out, ref, wl.N)
    check_slots(out, ref)

    print("[case] switch-large-shared: sampled outputs", flush=True)
    rng = np.random.default_rng(123)
    experts = rng.choice(ref["active"], size=4, replace=False)
    dropped = np.nonzero(ref["slot"] < 0)[0]
    drop_sample = rng.choice(dropped, size=min(32, dropped.size), replace=False) if dropped.size else dropped
    toks = np.concatenate([np.nonzero((e == i) & (ref["slot"] >= 0))[0] for i in experts] + [drop_sample])
    ws1 = _host_bf16(W["ws1"])
    ws2 = _host_bf16(W["ws2"])
    shared = oracle.ffn(xf[toks], ws1, ws2)
    del ws1, ws2
    yref = xf[toks] + shared  # dropped tokens: x + shared term
    for i in experts:
        sel = np.nonzero(e[toks] == i)[0]
        sel = sel[ref["slot"][toks[sel]] >= 0]
        o = oracle.ffn(xf[toks[sel]], _host_bf16(W["w1"][i]), _host_bf16(W["w2"][i]))
        yref[sel] = g[toks[sel], None] * o + shared[sel]
    y = host(out["y"])[toks]
    r = row_rel(y, yref)
    assert r.max() <= TOL_OUT["bf16"], f"max row rel err {r.max():.3g} (token {toks[r.argmax()]})"
