"""The layer forward captured in a HIP graph (torch.cuda.CUDAGraph).

The library allocates nothing, synchronises nothing and records no memset,
so one capture of switch_moe_forward replays the whole layer.  Each replay,
with new token rows copied into the captured x in between (eager work and a
synchronisation between replays), must equal an eager forward of a second
layer object on the same rows, bit for bit, for every output.  The routings
cover the paths the forward takes: per-expert token-order slots, the
gate-descending assignment kernels, top-K, expert choice and Expanded Drop.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import dev, host_bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from switch_top_routed_amd import native

CASES = [
    dict(name="top1-token"),
    dict(name="top1-gate", priority="gate"),
    dict(name="top2-token", top_k=2),
    dict(name="expert-choice", routing="expert"),
    dict(name="expand2", expand=2),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_forward_graph_replays_match_eager(case):
    kw = {k: v for k, v in case.items() if k != "name"}
    wl = workloads.Workload("graph", 1000, 256, 384, 16, 0.8, "bf16", 1.0 / math.sqrt(256), seed=50_001,
                            bias_scale=0.5)
    print(f"[case] graph replay {case['name']}", flush=True)
    inp = workloads.make_inputs(wl)
    wg, w1, w2 = dev(inp.w_gate, "bf16"), dev(inp.w1, "bf16"), dev(inp.w2, "bf16")
    bias = torch.from_numpy(inp.bias).cuda() if inp.bias is not None else None

    def layer():
        return native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, dtype=torch.bfloat16,
                                capacity_factor=wl.capacity_factor, **kw)

    lg, le = layer(), layer()
    x_static = dev(inp.x, "bf16").clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lg(x_static, wg, w1, w2, bias=bias)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lg(x_static, wg, w1, w2, bias=bias)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    for rep in range(3):
        rows = inp.x[rng.permutation(wl.T)]  # new token order: other routes, other slots
        x_new = dev(rows, "bf16")
        x_static.copy_(x_new)
        graph.replay()
        torch.cuda.synchronize()
        got = {k: host_bits(v).copy() for k, v in lg.out.items()}
        ref = le(x_new, wg, w1, w2, bias=bias)
        torch.cuda.synchronize()
        for k, v in ref.items():
            np.testing.assert_array_equal(got[k], host_bits(v), err_msg=f"replay {rep}: {k}")
