"""GPU parity on the large layer with a shared expert (T=16384, d=5120,
d_ff=8192, N=128, cf=1.25 -> C=160, plus one always-on dense FFN of width
8192).

The routed and shared weights (~22 GB of bf16) are drawn on the device with
torch's seeded generator; x and W_g are drawn on the host and conditioned to a
top-2 logit margin >= 1e-3.  Routing, load statistics, slots and counts are
checked in full against the fp64 oracle; the layer output is checked on the
first and the last kept slot of every one of the 128 experts and on 1024
seeded tokens across the batch (kept or dropped), each including the shared
term, with the oracle evaluating those tokens one expert at a time from the
weights copied back to the host.
"""
from concurrent.futures import ThreadPoolExecutor

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


@pytest.mark.timeout(600)
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
    # every active expert's first and last kept slot, plus 1024 seeded tokens
    # across the batch (kept or dropped), each with the shared term
    slot = ref["slot"]
    tos, kc = ref["token_of_slot"], ref["kept_count"]
    ends = [tos[i, j] for i in ref["active"] for j in {0, int(kc[i]) - 1}]
    rng = np.random.default_rng(123)
    toks = np.unique(np.concatenate([np.asarray(ends, dtype=np.int64),
                                     rng.choice(wl.T, size=1024, replace=False)]))
    assert len(ref["active"]) == wl.N
    y = host(out["y"])[toks]
    yref = xf[toks].copy()  # dropped tokens: x + shared term
    shared = oracle.ffn(xf[toks], _host_bf16(W["ws1"]), _host_bf16(W["ws2"]))
    W1, W2 = W["w1"], W["w2"]

    def one(i):
        sel = np.nonzero((e[toks] == i) & (slot[toks] >= 0))[0]
        if sel.size == 0:
            return sel, None
        w1h = W1[i].detach().cpu().view(torch.int16).numpy().view(np.uint16)
        w2h = W2[i].detach().cpu().view(torch.int16).numpy().view(np.uint16)
        return sel, oracle.ffn(xf[toks[sel]], oracle.widen(w1h, "bf16"), oracle.widen(w2h, "bf16"))

    with ThreadPoolExecutor(8) as ex:
        for sel, o in ex.map(one, range(wl.N)):
            if o is not None:
                yref[sel] = g[toks[sel], None] * o
    yref += shared
    r = row_rel(y, yref)
    assert r.max() <= TOL_OUT["bf16"], f"max row rel err {r.max():.3g} (token {toks[r.argmax()]})"
    print(f"[case] switch-large-shared: {toks.size} tokens checked, max row rel err {r.max():.3g}", flush=True)
