"""Helpers shared by the GPU parity tests: host<->device conversion and the
parity bars.

Parity bars (the layer's published tolerances):
  * integer results (expert_id, slot, token_of_slot, counts, n_dropped,
    active list) and f: bit-exact;
  * P: relative 1e-5 with an absolute floor of 1e-9; L_aux: relative 1e-5;
  * gate (fp32 router): relative 1e-5;
  * outputs: per kept token, max_k |y - y_ref| / max_k |y_ref| <= 1e-4 (fp32)
    or 2e-2 (bf16 storage, fp32 accumulation); dropped tokens bit-exact;
  * gradients: the same bar per row, measured as the distance to the
    oracle's [lo, hi] envelope (check_rows).
"""
import numpy as np
import torch

import oracle

TOL_OUT = {"f32": 1e-4, "bf16": 2e-2}
TOL_P = 1e-5
TOL_LAUX = 1e-5
TOL_GATE = 1e-5


def dev(a: np.ndarray, dtype: str):
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> fp64 numpy (bf16 widened exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.widen(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    return t.numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def row_rel(a: np.ndarray, ref: np.ndarray) -> np.ndarray:
    num = np.abs(a - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-30)


def check_routing(o: dict, ref: dict, N: int):
    np.testing.assert_array_equal(host(o["expert_id"]), ref["expert_id"])
    np.testing.assert_allclose(host(o["gate"]), ref["gate"], rtol=TOL_GATE)
    np.testing.assert_array_equal(host(o["routed_count"]), ref["routed_count"])
    np.testing.assert_array_equal(host(o["f"]), ref["f"].astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(host(o["P"]), ref["P"], rtol=TOL_P, atol=1e-9)
    lg = float(host(o["l_aux"])[0])
    assert abs(lg - ref["l_aux"]) <= TOL_LAUX * abs(ref["l_aux"]), (lg, ref["l_aux"])


def check_slots(o: dict, ref: dict, check_tos=True):
    np.testing.assert_array_equal(host(o["slot"]), ref["slot"])
    np.testing.assert_array_equal(host(o["kept_count"]), ref["kept_count"])
    assert int(host(o["n_dropped"])[0]) == ref["n_dropped"]
    if "n_active" in o:
        na = int(host(o["n_active"])[0])
        assert na == len(ref["active"])
        np.testing.assert_array_equal(host(o["active"])[:na], ref["active"])
    if check_tos and "token_of_slot" in o:
        np.testing.assert_array_equal(host(o["token_of_slot"]), ref["token_of_slot"])


def check_output(y_dev: torch.Tensor, ref: dict, x_stored: np.ndarray, dtype: str, rows=None, shared=False):
    """y parity: kept rows within tolerance; dropped rows bit-exact unless a shared term is added."""
    y = host(y_dev)
    slot = ref["slot"]
    idx = np.arange(len(slot)) if rows is None else np.asarray(rows)
    kept = idx[slot[idx] >= 0]
    drop = idx[slot[idx] < 0]
    tol = TOL_OUT[dtype]
    if kept.size:
        r = row_rel(y[kept], ref["y"][kept])
        assert r.max() <= tol, f"max row rel err {r.max():.3g} > {tol} (token {kept[r.argmax()]})"
    if drop.size:
        if shared:
            r = row_rel(y[drop], ref["y"][drop])
            assert r.max() <= tol, f"dropped rows: max rel err {r.max():.3g}"
        else:
            yb = host_bits(y_dev)[drop]
            xs = x_stored.view(np.uint32) if x_stored.dtype == np.float32 else x_stored
            np.testing.assert_array_equal(yb, xs[drop])
    return y


def check_rows(name, got, ref, tol, env=None, zero_rows_exact=True):
    """Row-wise relative distance to [lo, hi] (or to ref); all-zero reference rows must be zero."""
    got = got.reshape(-1, got.shape[-1])
    ref2 = ref.reshape(-1, ref.shape[-1])
    if env is None:
        lo = hi = ref2
    else:
        lo, hi = (e.reshape(-1, ref.shape[-1]) for e in env)
    dist = np.maximum(np.maximum(got - hi, lo - got), 0.0).max(axis=1)
    den = np.abs(ref2).max(axis=1)
    zero = den == 0
    if zero_rows_exact and zero.any():
        bad = np.nonzero(np.abs(got[zero]).max(axis=1) != 0)[0]
        assert bad.size == 0, f"{name}: {bad.size} rows should be exactly zero"
    r = dist[~zero] / den[~zero]
    if r.size:
        assert r.max() <= tol, f"{name}: max row rel err {r.max():.3g} > {tol} (row {np.nonzero(~zero)[0][r.argmax()]})"
    return float(r.max()) if r.size else 0.0
