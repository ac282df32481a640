"""GPU parity of the router kernels beyond the workload configs, through the C
ABI (switch_route) against the fp64 oracle ("Top-1 Routing" page, Core
mechanism and Load balancing).

* d_model a multiple of 32 but not of 128, at token counts where the router
  would stage a workgroup's rows in LDS (T = 4096): the staging's swizzle
  needs d % 128 == 0, so these shapes must take the streaming path and still
  match;
* the two kernels for many tokens with long rows (>= 2048 elements, N <=
  128): the streaming one (rows staged in LDS chunk by chunk, d % 1024 == 0)
  and the K-sliced one (otherwise), at both tile heights (32 and 64 tokens
  per workgroup), with a ragged last tile and N not a multiple of 16.
Expert ids and counts bit-exact, gate / P / L_aux at the router tolerances.
Plus: the plain forward's top-1 epilogue and the training forward's general
epilogue give bit-identical routing, statistics and outputs on every kernel.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import inputs_util
from tests.gpu_util import check_routing, dev

pytestmark = pytest.mark.gpu

CASES = [
    # (T, d_model, N, bias_scale)
    (4096, 96, 64, 0.0),      # one 16-token tile per workgroup, 3 k-steps
    (4096, 160, 40, 1.0),     # 5 k-steps, N ragged, Zipf-like bias
    (8200, 2048, 100, 0.0),   # streaming (rows staged in LDS chunks), 32 tokens per workgroup, last tile 8
    (16400, 2048, 128, 1.0),  # streaming, 64 tokens per workgroup, last tile 16 tokens, 8 chunks
    (8192, 4096, 128, 0.0),   # streaming, 32 tokens per workgroup, 16 chunks
    (16400, 5120, 128, 0.0),  # streaming, 64 tokens per workgroup, last tile 16 tokens, 20 chunks
    (16512, 3072, 100, 1.0),  # streaming, 64 tokens per workgroup, 12 chunks, N ragged
    (16448, 2048, 72, 0.0),   # streaming, 64 tokens per workgroup, N ragged, 257 workgroups
    (8192, 2560, 96, 1.0),    # K-sliced waves (d % 1024 != 0), 32 tokens per workgroup
    (16400, 2560, 120, 0.0),  # K-sliced waves, 64 tokens per workgroup, last tile 16 tokens
]


@pytest.mark.parametrize("T,d,N,bias_scale", CASES)
def test_route_shapes(T, d, N, bias_scale):
    import switch_top_routed_amd as sw

    wl = workloads.Workload(f"route-{T}x{d}x{N}", T, d, 4 * d, N, 1.0, "bf16", 1.0 / math.sqrt(d),
                            bias_scale=bias_scale, seed=20_000 + T + d + N)
    print(f"[case] route T={T} d={d} N={N} bias={bias_scale}", flush=True)
    inp = inputs_util.conditioned_inputs(wl, weights=False)
    _, p, e, g = inputs_util.stored_router(inp)
    cnt, f, P, l_aux = oracle.aux_loss(e, p, N)
    ref = dict(expert_id=e, gate=g, routed_count=cnt, f=f, P=P, l_aux=l_aux)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    o = sw.switch_route(dev(inp.x, "bf16"), dev(inp.w_gate, "bf16"), bias)
    torch.cuda.synchronize()
    check_routing(o, ref, N)


# (T, d_model, N): the fused kernel with staged rows (16 tokens per workgroup), the
# streaming kernel at 32 and 64 tokens per workgroup, and the K-sliced kernel
EPILOGUE_CASES = [(4096, 768, 128), (4096, 256, 40), (8200, 2048, 100), (16400, 2048, 128), (16400, 2560, 120),
                  (16512, 3072, 100)]


@pytest.mark.parametrize("T,d,N", EPILOGUE_CASES)
def test_top1_epilogues_agree(T, d, N):
    """The plain forward ends the router with the several-lanes-per-token top-1
    epilogue; the training forward (probabilities saved) with the general one.
    Both must give the same expert ids, gates and statistics bit for bit."""
    import switch_top_routed_amd as sw
    from tests.gpu_util import host_bits

    F = 128
    wl = workloads.Workload(f"epi-{T}x{d}x{N}", T, d, F, N, 1.0, "bf16", 1.0 / math.sqrt(d), bias_scale=0.5,
                            seed=30_000 + T + d + N)
    print(f"[case] epilogues T={T} d={d} N={N}", flush=True)
    inp = inputs_util.conditioned_inputs(wl, weights=False)
    rng = np.random.default_rng(wl.seed + 1)
    w1 = torch.from_numpy((rng.standard_normal((N, d, F)) / math.sqrt(d)).astype(np.float32)).cuda().to(torch.bfloat16)
    w2 = torch.from_numpy((rng.standard_normal((N, F, d)) / math.sqrt(F)).astype(np.float32)).cuda().to(torch.bfloat16)
    x, wg = dev(inp.x, "bf16"), dev(inp.w_gate, "bf16")
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    plain = sw.SwitchMoE(T, d, F, N, dtype=torch.bfloat16, capacity_factor=1.0)
    a = {k: v.clone() for k, v in plain(x, wg, w1, w2, bias=bias).items()}
    train = sw.SwitchMoE(T, d, F, N, dtype=torch.bfloat16, capacity_factor=1.0, train=True)
    b = train.forward_train(x, wg, w1, w2, bias=bias)
    torch.cuda.synchronize()
    for k in ("expert_id", "gate", "routed_count", "f", "P", "l_aux", "y"):
        np.testing.assert_array_equal(host_bits(a[k]), host_bits(b[k]), err_msg=k)
