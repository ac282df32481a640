"""Input generator: determinism, bf16 rounding, conditioning (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import inputs_util


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100_000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.0e38, 1e-40], np.float32)])
    mine = workloads.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    back = workloads.bf16_bits_to_f32(mine)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_same_seed_same_bytes():
    wl = workloads.WORKLOADS["switch-tiny-fp32"]
    a = workloads.make_inputs(wl)
    b = workloads.make_inputs(wl)
    for k in ("x", "w_gate", "w1", "w2"):
        assert getattr(a, k).tobytes() == getattr(b, k).tobytes()
    c = workloads.make_inputs(wl.with_(seed=wl.seed + 1), weights=False)
    assert c.x.tobytes() != a.x.tobytes()


def test_shapes_and_distributions():
    wl = workloads.WORKLOADS["switch-base-uniform"]
    inp = workloads.make_inputs(wl, weights=False)
    assert inp.x.shape == (4096, 768) and inp.x.dtype == np.uint16
    x = oracle.widen(inp.x, "bf16")
    assert abs(x.std() - 1.0) < 0.01
    wg = oracle.widen(inp.w_gate, "bf16")
    assert abs(wg.std() * np.sqrt(768) - 1.0) < 0.02
    assert inp.bias is None


def test_zipf_bias():
    wl = workloads.WORKLOADS["switch-base-zipf"]
    b = workloads.router_bias(wl)
    ranks = np.rint(np.exp(-b.astype(np.float64) / 1.5)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 129))


@pytest.mark.parametrize("name", ["switch-tiny-fp32", "switch-base-uniform", "switch-decode-384"])
def test_margin_conditioning(name):
    wl = workloads.WORKLOADS[name]
    inp = inputs_util.conditioned_inputs(wl, weights=False)
    assert inputs_util.margin_bad_rows(inp).size == 0


def test_gate_gap_conditioning():
    wl = workloads.WORKLOADS["switch-base-zipf"]
    inp = inputs_util.conditioned_inputs(wl, weights=False, gate_order_cmax=64)
    assert inputs_util.gate_gap_bad_rows(64)(inp).size == 0
