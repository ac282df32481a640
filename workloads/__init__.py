"""Seeded synthetic inputs for the Switch top-1 MoE layer (forward and backward).

This module is shared by the fp64 oracle side (tests, smoke check, CPU
baseline) and the HIP side (tests, bench).  It holds no part of the
layer's arithmetic: it only draws Gaussian tensors, rounds them to the
storage dtype, and resamples rows that a caller-supplied predicate flags
(the routing-margin and gate-gap predicates are built by the tests from
the oracle, so this module never evaluates a router).

Workloads (shapes and distributions follow the layer definitions on the
pages, see "Top-1 Routing", Key parameters and compute; values are
synthetic Gaussian stand-ins for the C4 / mT5 token activations the
Switch Transformers summary page trains on):

  switch-tiny-fp32      T=256   d=64   d_ff=128  N=8   cf=1.0  fp32
  switch-base-uniform   T=4096  d=768  d_ff=3072 N=128 cf=1.25 bf16
  switch-base-zipf      T=4096  d=768  d_ff=3072 N=128 cf in {0.5,1,2} bf16,
                        router bias b_i = -1.5 ln(rank_i)
  switch-large-shared   T=16384 d=5120 d_ff=8192 N=128 cf=1.25 bf16,
                        plus one always-on shared dense FFN (d_ff_s=8192)
  switch-decode-384     T=128   d=4096 d_ff=2048 N=384 cf=2.0  bf16,
                        router bias b_i = -1.0 ln(rank_i)
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Callable, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    d_ff: int
    N: int
    capacity_factor: float
    dtype: str
    wg_std: float          # router weight std
    bias_scale: float = 0.0  # b_i = -bias_scale * ln(rank_i); 0 = no bias
    d_ff_shared: int = 0
    priority: str = "token"  # "token" | "gate"
    gate_scale: bool = True
    residual_all: bool = False
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "switch-tiny-fp32": Workload("switch-tiny-fp32", 256, 64, 128, 8, 1.0, F32, 0.1, seed=10_000),
    "switch-base-uniform": Workload("switch-base-uniform", 4096, 768, 3072, 128, 1.25, BF16,
                                    1.0 / math.sqrt(768), seed=10_001),
    "switch-base-zipf": Workload("switch-base-zipf", 4096, 768, 3072, 128, 1.0, BF16,
                                 1.0 / math.sqrt(768), bias_scale=1.5, seed=10_002),
    "switch-large-shared": Workload("switch-large-shared", 16384, 5120, 8192, 128, 1.25, BF16,
                                    1.0 / math.sqrt(5120), d_ff_shared=8192, seed=10_003),
    "switch-decode-384": Workload("switch-decode-384", 128, 4096, 2048, 384, 2.0, BF16,
                                  1.0 / math.sqrt(4096), bias_scale=1.0, seed=10_004),
}

# the skewed workload is run over this matrix (capacity factor x priority x gate scaling)
ZIPF_MATRIX = [(cf, pr, gs) for cf in (0.5, 1.0, 2.0) for pr in ("token", "gate") for gs in (True, False)]


# ---------------------------------------------------------------------------
# bf16 storage helpers (bit-level; round to nearest even)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draw -> stored array (float32, or uint16 bf16 bits)."""
    if dtype == F32:
        return np.ascontiguousarray(a32, dtype=np.float32)
    return f32_to_bf16_bits(a32)


# ---------------------------------------------------------------------------
# generation
# ---------------------------------------------------------------------------
STREAMS = ("x", "w_gate", "rank", "w1", "w2", "ws1", "ws2", "resample", "dy")

# upstream gradient of the auxiliary loss for backward runs: the balance-loss
# coefficient alpha = 1e-2 of the Switch Transformers summary page (Eq. 4
# passage), i.e. the gradient l_aux receives from  task + alpha * l_aux
DL_AUX = 1e-2


def _children(seed: int):
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(len(STREAMS))
    return dict(zip(STREAMS, kids))


def _normal(seedseq, shape, std, dtype):
    g = np.random.Generator(np.random.PCG64(seedseq))
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return stored(a, dtype)


def _per_expert(seedseq, N, shape, std, dtype, threads):
    kids = seedseq.spawn(N)
    out_dtype = np.float32 if dtype == F32 else np.uint16
    out = np.empty((N,) + tuple(shape), dtype=out_dtype)

    def one(i):
        out[i] = _normal(kids[i], shape, std, dtype)

    if threads > 1 and N > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(N)))
    else:
        for i in range(N):
            one(i)
    return out


@dataclass
class Inputs:
    """Stored inputs of one layer call (host arrays; bf16 held as uint16 bits)."""
    wl: Workload
    x: np.ndarray                 # [T, d]
    w_gate: np.ndarray            # [N, d]
    bias: Optional[np.ndarray]    # [N] float32 or None
    w1: Optional[np.ndarray] = None   # [N, d, d_ff]
    w2: Optional[np.ndarray] = None   # [N, d_ff, d]
    ws1: Optional[np.ndarray] = None  # [d, d_ff_s]
    ws2: Optional[np.ndarray] = None  # [d_ff_s, d]
    resampled_rows: int = 0
    meta: dict = field(default_factory=dict)


def router_bias(wl: Workload) -> Optional[np.ndarray]:
    """b_i = -s * ln(rank_i), rank a seeded permutation of 1..N (fp64, stored as fp32)."""
    if wl.bias_scale == 0.0:
        return None
    kids = _children(wl.seed)
    g = np.random.Generator(np.random.PCG64(kids["rank"]))
    rank = g.permutation(wl.N) + 1
    return (-wl.bias_scale * np.log(rank.astype(np.float64))).astype(np.float32)


def make_inputs(wl: Workload, *, weights: bool = True, threads: int = 8,
                bad_rows: Optional[Callable[["Inputs"], np.ndarray]] = None,
                max_rounds: int = 50) -> Inputs:
    """Draw the stored inputs of workload `wl` on the host.

    x ~ N(0,1); W_g ~ N(0, wg_std^2); W1 ~ N(0, 1/d); W2 ~ N(0, 1/d_ff);
    shared Ws1 ~ N(0, 1/d), Ws2 ~ N(0, 1/d_ff_s).  Draws are float32 and are
    rounded once to the storage dtype.  If `bad_rows` is given it is called
    with the current inputs and returns token rows to redraw (from a
    separate child stream); this repeats until it returns no rows.
    """
    kids = _children(wl.seed)
    T, d, N, F = wl.T, wl.d_model, wl.N, wl.d_ff
    x = _normal(kids["x"], (T, d), 1.0, wl.dtype)
    w_gate = _normal(kids["w_gate"], (N, d), wl.wg_std, wl.dtype)
    inp = Inputs(wl, x, w_gate, router_bias(wl))
    if weights:
        inp.w1 = _per_expert(kids["w1"], N, (d, F), 1.0 / math.sqrt(d), wl.dtype, threads)
        inp.w2 = _per_expert(kids["w2"], N, (F, d), 1.0 / math.sqrt(F), wl.dtype, threads)
        if wl.d_ff_shared:
            Fs = wl.d_ff_shared
            k1, k2 = kids["ws1"], kids["ws2"]
            inp.ws1 = _normal(k1, (d, Fs), 1.0 / math.sqrt(d), wl.dtype)
            inp.ws2 = _normal(k2, (Fs, d), 1.0 / math.sqrt(Fs), wl.dtype)
    if bad_rows is not None:
        resample_rows(inp, bad_rows, max_rounds=max_rounds)
    return inp


def make_upstream(wl: Workload) -> np.ndarray:
    """Upstream gradient dy [T, d] of the layer output for backward runs:
    N(0, 1) draws rounded once to the storage dtype (own child stream)."""
    return _normal(_children(wl.seed)["dy"], (wl.T, wl.d_model), 1.0, wl.dtype)


def resample_rows(inp: Inputs, bad_rows: Callable[["Inputs"], np.ndarray], max_rounds: int = 50) -> None:
    """Redraw the x rows that `bad_rows` flags until it flags none."""
    kids = _children(inp.wl.seed)
    rs = kids["resample"].spawn(max_rounds)
    for r in range(max_rounds):
        rows = np.unique(np.asarray(bad_rows(inp), dtype=np.int64))
        if rows.size == 0:
            inp.meta["resample_rounds"] = r
            return
        fresh = _normal(rs[r], (rows.size, inp.wl.d_model), 1.0, inp.wl.dtype)
        inp.x[rows] = fresh
        inp.resampled_rows += int(rows.size)
    raise RuntimeError(f"resampling did not converge in {max_rounds} rounds")


# ---------------------------------------------------------------------------
# device-side generation for the largest workload (host generation of 21 GB of
# bf16 weights is slow); uses torch's seeded Philox generator on the device.
# ---------------------------------------------------------------------------
def make_device_weights(wl: Workload, device="cuda"):
    """Draw W1, W2 (and shared Ws1, Ws2) directly on the device, stored bf16.

    Returns a dict of device tensors.  Each expert gets its own torch
    generator seeded from (seed, stream, expert) so that any expert can be
    regenerated alone on the host side via `device_expert_weights`.
    """
    import torch
    assert wl.dtype == BF16
    d, F, N = wl.d_model, wl.d_ff, wl.N
    out = {
        "w1": torch.empty((N, d, F), dtype=torch.bfloat16, device=device),
        "w2": torch.empty((N, F, d), dtype=torch.bfloat16, device=device),
    }
    for e in range(N):
        out["w1"][e].copy_(_dev_normal(wl.seed, 1, e, (d, F), 1.0 / math.sqrt(d), device))
        out["w2"][e].copy_(_dev_normal(wl.seed, 2, e, (F, d), 1.0 / math.sqrt(F), device))
    if wl.d_ff_shared:
        Fs = wl.d_ff_shared
        out["ws1"] = _dev_normal(wl.seed, 3, 0, (d, Fs), 1.0 / math.sqrt(d), device)
        out["ws2"] = _dev_normal(wl.seed, 4, 0, (Fs, d), 1.0 / math.sqrt(Fs), device)
    return out


def _dev_normal(seed, stream, index, shape, std, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream * 10_007 + index) & 0x7FFF_FFFF_FFFF_FFFF)
    a = torch.randn(shape, dtype=torch.float32, device=device, generator=g)
    a.mul_(std)
    return a.to(torch.bfloat16)
