"""GPU parity of MXFP4 expert weights: the quantizer (bit-exact against the
oracle's encoding) and the layer forward with MXFP4 experts against the fp64
oracle run on the oracle's own dequantized weights.

Bars: codes and scales bit-exact; routing, slots and counts bit-exact; outputs
per kept token max_k |y - y_ref| / max_k |y_ref| <= 2e-2 (bf16 activations,
fp32 accumulation; the weights are exact in both), dropped tokens bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import mxfp4 as mx
from tests import inputs_util
from tests.gpu_util import check_output, check_routing, check_slots, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from switch_top_routed_amd import native


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _bf16(a32):
    return workloads.f32_to_bf16_bits(a32.astype(np.float32))


@pytest.mark.parametrize("B,K,Nc,kind", [(3, 128, 96, "normal"), (2, 256, 300, "wide"), (1, 384, 17, "special"),
                                         (4, 128, 64, "ties")])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantizer_bit_exact(B, K, Nc, kind, dtype):
    rng = np.random.default_rng(K + Nc)
    w = rng.standard_normal((B, K, Nc)).astype(np.float32)
    if kind == "wide":
        w *= np.exp2(rng.integers(-40, 40, size=(B, 1, Nc))).astype(np.float32)
    if kind == "special":
        w[0, :32, 0] = 0.0                        # all-zero block
        w[0, 32:64, 1] = -0.0                     # negative zeros
        w[0, :32, 2] = 1e-39                      # subnormal fp32 (bf16 too)
        w[0, :32, 3] = 3.0e38                     # near the top of the range
        w[0, 64:96, 4] = np.float32(2.0 ** -130)  # a subnormal block
        w[0, :, 5] = -w[0, :, 5]
    if kind == "ties":  # every block holds 5 (so X = 1) and the rounding midpoints of both signs
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
        pattern = np.array([5.0] + mids + [-m for m in mids] + [0.0] * 17, dtype=np.float32)  # 32 per block
        w = np.ascontiguousarray(np.broadcast_to(np.tile(pattern, K // 32)[None, :, None], (B, K, Nc)))
    stored = _bf16(w) if dtype == "bf16" else w
    wd = dev(stored, dtype)
    codes, scales = native.switch_quantize_mxfp4(wd)
    torch.cuda.synchronize()
    q, s = mx.quantize(oracle.widen(stored, dtype))
    np.testing.assert_array_equal(codes.cpu().numpy(), q)
    np.testing.assert_array_equal(scales.cpu().numpy(), s)


def _mx_case(wl, **over):
    if over:
        wl = wl.with_(**over)
    _say(f"mxfp4 {wl.name} T={wl.T} d={wl.d_model} dff={wl.d_ff} N={wl.N} cf={wl.capacity_factor} {wl.priority}")
    gate_cmax = oracle.capacity(wl.T, wl.N, wl.capacity_factor) if wl.priority == "gate" else None
    inp = inputs_util.conditioned_inputs(wl, gate_order_cmax=gate_cmax)
    dt = wl.dtype
    x, wg = dev(inp.x, dt), dev(inp.w_gate, dt)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    q1, s1 = native.switch_quantize_mxfp4(dev(inp.w1, dt))
    q2, s2 = native.switch_quantize_mxfp4(dev(inp.w2, dt))
    layer = native.SwitchMoE(wl.T, wl.d_model, wl.d_ff, wl.N, capacity_factor=wl.capacity_factor,
                             priority=wl.priority, gate_scale=wl.gate_scale, weight_format="mxfp4")
    out = layer(x, wg, q1, q2, bias=bias, w1_scale=s1, w2_scale=s2)
    torch.cuda.synchronize()

    def w1_of(e):  # the oracle's own encoding of expert e, decoded exactly
        qq, ss = mx.quantize(oracle.widen(inp.w1[e:e + 1], dt))
        return mx.dequantize(qq, ss)[0]

    def w2_of(e):
        qq, ss = mx.quantize(oracle.widen(inp.w2[e:e + 1], dt))
        return mx.dequantize(qq, ss)[0]

    ref = oracle.moe_forward(oracle.widen(inp.x, dt), oracle.widen(inp.w_gate, dt), inp.bias, w1_of, w2_of, wl.N,
                             capacity_factor=wl.capacity_factor, priority=wl.priority, gate_scale=wl.gate_scale)
    check_routing(out, ref, wl.N)
    check_slots(out, ref)
    y = check_output(out["y"], ref, inp.x, dt)
    kept = ref["slot"] >= 0
    _say(f"  C={ref['C']} active {len(ref['active'])} dropped {ref['n_dropped']}")
    return y


def test_mxfp4_decode_384():
    _mx_case(workloads.WORKLOADS["switch-decode-384"])


def test_mxfp4_base():
    _mx_case(workloads.WORKLOADS["switch-base-uniform"])


@pytest.mark.parametrize("cf,priority", [(0.5, "gate"), (2.0, "token")])
def test_mxfp4_skewed(cf, priority):
    _mx_case(workloads.WORKLOADS["switch-base-zipf"], capacity_factor=cf, priority=priority)


def test_mxfp4_small_layers():
    import math
    for i, (T, d, dff, N, cf) in enumerate([(1, 128, 256, 4, 1.0), (300, 256, 384, 12, 1.3), (200, 128, 128, 1, 0.2)]):
        wl = workloads.Workload(f"mx-small-{i}", T, d, dff, N, cf, "bf16", 1.0 / math.sqrt(d), seed=40_000 + i)
        _mx_case(wl)
