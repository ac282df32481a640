"""ctypes binding of libswitch_moe.so (argument marshalling only).

Every entry point of include/switch_moe.h has a Python function of the same
name.  Tensors are torch tensors on the GPU; torch provides device memory and
the stream, all arithmetic runs in the library's HIP kernels.  The library
must have been built (python -m switch_top_routed_amd.build); importing this
module never falls back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libswitch_moe.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "switch_moe.h")

F32, BF16 = 0, 1
TOKEN_ORDER, GATE_DESC = 0, 1
GATE_SCALE, RESIDUAL_ALL, RENORM, ACCUM_EXPERT_GRADS = 1, 2, 4, 8
TOKEN_CHOICE, EXPERT_CHOICE = 0, 1
_ROUTING = {"token": TOKEN_CHOICE, "expert": EXPERT_CHOICE, TOKEN_CHOICE: TOKEN_CHOICE, EXPERT_CHOICE: EXPERT_CHOICE}
_DT = {torch.float32: F32, torch.bfloat16: BF16}
_PRIO = {"token": TOKEN_ORDER, "gate": GATE_DESC, TOKEN_ORDER: TOKEN_ORDER, GATE_DESC: GATE_DESC}

_vp = ctypes.c_void_p
_i32, _i64, _u32, _f64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double, ctypes.c_size_t


class SwitchMoeDesc(ctypes.Structure):
    _fields_ = [("T", _i64), ("d_model", _i32), ("d_ff", _i32), ("N", _i32), ("C", _i32),
                ("capacity_factor", _f64), ("dtype", _i32), ("priority", _i32), ("flags", _u32),
                ("d_ff_shared", _i32), ("top_k", _i32), ("routing", _i32), ("weight_format", _i32),
                ("expand_choices", _i32)]


class SwitchMoeInputs(ctypes.Structure):
    _fields_ = [("x", _vp), ("w_gate", _vp), ("bias", _vp), ("w1", _vp), ("w2", _vp), ("ws1", _vp), ("ws2", _vp),
                ("w1_scale", _vp), ("w2_scale", _vp)]


class SwitchMoeOutputs(ctypes.Structure):
    _fields_ = [("y", _vp), ("expert_id", _vp), ("gate", _vp), ("slot", _vp), ("routed_count", _vp),
                ("kept_count", _vp), ("n_dropped", _vp), ("f", _vp), ("P", _vp), ("l_aux", _vp)]


class SwitchMoeSaved(ctypes.Structure):
    _fields_ = [("probs", _vp), ("token_of_slot", _vp), ("active", _vp), ("n_active", _vp), ("h", _vp),
                ("h_shared", _vp)]


class SwitchMoeGrads(ctypes.Structure):
    _fields_ = [("dx", _vp), ("dw_gate", _vp), ("dbias", _vp), ("dw1", _vp), ("dw2", _vp), ("dws1", _vp),
                ("dws2", _vp)]


_SIGS = {
    "switch_capacity": (_i32, [_i64, _i32, _f64]),
    "switch_route_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "switch_route": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "switch_assign_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "switch_assign_capacity": (_i32, [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "switch_dispatch": (_i32, [_vp, _i32, _i64, _i32, _vp, _vp, _i32, _i32, _vp, _vp]),
    "switch_expert_ffn_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "switch_expert_ffn": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "switch_combine": (_i32, [_vp, _vp, _vp, _i32, _i64, _i32, _vp, _vp, _vp, _i32, _i32, _u32, _vp, _vp]),
    "switch_moe_workspace_bytes": (_sz, [ctypes.POINTER(SwitchMoeDesc)]),
    "switch_moe_forward": (_i32, [ctypes.POINTER(SwitchMoeDesc), ctypes.POINTER(SwitchMoeInputs),
                                  ctypes.POINTER(SwitchMoeOutputs), _vp, _sz, _vp]),
    "switch_moe_forward_timed": (_i32, [ctypes.POINTER(SwitchMoeDesc), ctypes.POINTER(SwitchMoeInputs),
                                        ctypes.POINTER(SwitchMoeOutputs), _vp, _sz, _vp, ctypes.POINTER(_vp)]),
    "switch_moe_forward_noalloc": (_i32, [ctypes.POINTER(SwitchMoeDesc), ctypes.POINTER(SwitchMoeInputs),
                                          ctypes.POINTER(SwitchMoeOutputs), _vp]),
    "switch_moe_noalloc_max_bytes": (_sz, []),
    "switch_moe_forward_train": (_i32, [ctypes.POINTER(SwitchMoeDesc), ctypes.POINTER(SwitchMoeInputs),
                                        ctypes.POINTER(SwitchMoeOutputs), ctypes.POINTER(SwitchMoeSaved), _vp, _sz,
                                        _vp]),
    "switch_moe_backward_workspace_bytes": (_sz, [ctypes.POINTER(SwitchMoeDesc)]),
    "switch_moe_backward": (_i32, [ctypes.POINTER(SwitchMoeDesc), ctypes.POINTER(SwitchMoeInputs),
                                   ctypes.POINTER(SwitchMoeOutputs), ctypes.POINTER(SwitchMoeSaved), _vp, _vp,
                                   ctypes.POINTER(SwitchMoeGrads), _vp, _sz, _vp]),
    "switch_moe_backward_timed": (_i32, [ctypes.POINTER(SwitchMoeDesc), ctypes.POINTER(SwitchMoeInputs),
                                         ctypes.POINTER(SwitchMoeOutputs), ctypes.POINTER(SwitchMoeSaved), _vp, _vp,
                                         ctypes.POINTER(SwitchMoeGrads), _vp, _sz, _vp, ctypes.POINTER(_vp)]),
    "switch_quantize_mxfp4": (_i32, [_vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp]),
    "switch_status_str": (ctypes.c_char_p, [_i32]),
    "switch_last_error": (ctypes.c_char_p, []),
}

_lib = None


def header_functions():
    """Names of the functions declared in include/switch_moe.h."""
    with open(HEADER) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(switch_[a-z0-9_]+)\s*\(", text, re.M)))


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m switch_top_routed_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


class SwitchError(RuntimeError):
    def __init__(self, fn, status):
        L = lib()
        msg = L.switch_last_error().decode()
        super().__init__(f"{fn}: {L.switch_status_str(status).decode()} ({status}): {msg}")
        self.status = status


def _check(fn, status):
    if status != 0:
        raise SwitchError(fn, status)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _empty(shape, dtype, dev):
    return torch.empty(shape, dtype=dtype, device=dev)


def _ws(nbytes, dev, ws=None):
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def switch_capacity(T: int, N: int, capacity_factor: float) -> int:
    return int(lib().switch_capacity(T, N, capacity_factor))


def switch_route(x, w_gate, bias=None, *, ws=None, stream=None):
    """Router + load statistics.  Returns dict(expert_id, gate, routed_count, f, P, l_aux)."""
    for t, n in ((x, "x"), (w_gate, "w_gate")):
        _need(t, n)
    T, d = x.shape
    N = w_gate.shape[0]
    dev = x.device
    o = dict(expert_id=_empty(T, torch.int32, dev), gate=_empty(T, torch.float32, dev),
             routed_count=_empty(N, torch.int32, dev), f=_empty(N, torch.float32, dev),
             P=_empty(N, torch.float32, dev), l_aux=_empty(1, torch.float32, dev))
    L = lib()
    nb = L.switch_route_workspace_bytes(T, d, N, _dtype(x))
    w = _ws(nb, dev, ws)
    _check("switch_route", L.switch_route(_p(x), _p(w_gate), _p(bias), T, d, N, _dtype(x), _p(o["expert_id"]),
                                          _p(o["gate"]), _p(o["routed_count"]), _p(o["f"]), _p(o["P"]),
                                          _p(o["l_aux"]), _p(w), w.numel(), _stream(stream)))
    return o


def switch_assign_capacity(expert_id, gate, N: int, C: int, priority="token", *, ws=None, stream=None):
    """Slots under capacity C.  Returns dict(slot, token_of_slot [N, C], kept_count, n_dropped, active, n_active)."""
    _need(expert_id, "expert_id")
    T = expert_id.shape[0]
    dev = expert_id.device
    pr = _PRIO[priority]
    o = dict(slot=_empty(T, torch.int32, dev), token_of_slot=_empty((N, C), torch.int32, dev),
             kept_count=_empty(N, torch.int32, dev), n_dropped=_empty(1, torch.int32, dev),
             active=_empty(N, torch.int32, dev), n_active=_empty(1, torch.int32, dev))
    L = lib()
    w = _ws(L.switch_assign_workspace_bytes(T, N, C, pr), dev, ws)
    _check("switch_assign_capacity",
           L.switch_assign_capacity(_p(expert_id), _p(gate), T, N, C, pr, _p(o["slot"]), _p(o["token_of_slot"]),
                                    _p(o["kept_count"]), _p(o["n_dropped"]), _p(o["active"]), _p(o["n_active"]),
                                    _p(w), w.numel(), _stream(stream)))
    return o


def switch_dispatch(x, token_of_slot, kept_count, N: int, C: int, *, expert_in=None, stream=None):
    _need(x, "x")
    T, d = x.shape
    if expert_in is None:
        expert_in = torch.zeros((N, C, d), dtype=x.dtype, device=x.device)
    _check("switch_dispatch", lib().switch_dispatch(_p(x), _dtype(x), T, d, _p(token_of_slot), _p(kept_count), N, C,
                                                    _p(expert_in), _stream(stream)))
    return expert_in


def switch_expert_ffn(expert_in, w1, w2, kept_count, active, n_active, *, expert_out=None, ws=None, stream=None):
    for t, n in ((expert_in, "expert_in"), (w1, "w1"), (w2, "w2")):
        _need(t, n)
    N, C, d = expert_in.shape
    dff = w1.shape[2]
    if expert_out is None:
        expert_out = torch.zeros_like(expert_in)
    L = lib()
    w = _ws(L.switch_expert_ffn_workspace_bytes(N, C, d, dff, _dtype(expert_in)), expert_in.device, ws)
    _check("switch_expert_ffn",
           L.switch_expert_ffn(_p(expert_in), _p(w1), _p(w2), _dtype(expert_in), N, C, d, dff, _p(kept_count),
                               _p(active), _p(n_active), _p(expert_out), _p(w), w.numel(), _stream(stream)))
    return expert_out


def switch_combine(expert_out, x, expert_id, slot, gate, flags=GATE_SCALE, *, shared_out=None, y=None, stream=None):
    _need(x, "x")
    N, C, d = expert_out.shape
    T = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    _check("switch_combine", lib().switch_combine(_p(expert_out), _p(x), _p(shared_out), _dtype(x), T, d,
                                                  _p(expert_id), _p(slot), _p(gate), N, C, flags, _p(y),
                                                  _stream(stream)))
    return y


_hip = None


def _hip_runtime():
    """The HIP runtime library (for event handles: create, elapsed time, destroy)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
        _hip.hipEventCreate.restype = ctypes.c_int
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        _hip.hipEventElapsedTime.restype = ctypes.c_int
        _hip.hipEventSynchronize.argtypes = [_vp]
        _hip.hipEventSynchronize.restype = ctypes.c_int
        _hip.hipEventDestroy.argtypes = [_vp]
        _hip.hipEventDestroy.restype = ctypes.c_int
    return _hip


class StageEvents:
    """HIP events at stage boundaries.  Forward (n=7, switch_moe_forward_timed): [0] before route,
    [1] assign, [2] dispatch, [3] routed expert FFN, [4] after it, [5] combine, [6] after combine.
    Backward (n=6, switch_moe_backward_timed): [0] start, [1] pass over w2, [2] pass over w1,
    [3] after it, [4] after the shared expert, [5] end."""

    def __init__(self, which=None, n=7):
        """which: indices of the events to create (default all); the others stay NULL and are not recorded."""
        self.N = n
        h = _hip_runtime()
        self.handles = (_vp * self.N)()
        for i in range(self.N) if which is None else which:
            ev = _vp()
            rc = h.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.handles[i] = ev

    def ms(self, i, j):
        """Milliseconds from event i to event j (both recorded and complete)."""
        h = _hip_runtime()
        if h.hipEventSynchronize(self.handles[j]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        out = ctypes.c_float()
        rc = h.hipEventElapsedTime(ctypes.byref(out), self.handles[i], self.handles[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return out.value

    def __del__(self):
        if _hip is not None:
            for i in range(self.N):
                if self.handles[i]:
                    _hip.hipEventDestroy(self.handles[i])


class SwitchMoE:
    """The whole layer with its outputs and workspace preallocated (one call = switch_moe_forward)."""

    def __init__(self, T, d_model, d_ff, N, *, dtype=torch.bfloat16, capacity_factor=1.0, C=0, priority="token",
                 gate_scale=True, residual_all=False, d_ff_shared=0, device="cuda", train=False, top_k=1,
                 routing="token", renorm=False, weight_format="native", expand=1, accumulate_expert_grads=False):
        """top_k > 1: top-K token choice; routing="expert": expert choice; expand = M >= 2: Expanded
        Drop over each token's M highest-logit experts (see include/switch_moe.h).
        With top-K, out["expert_id"], out["gate"] and out["slot"] are [T, K].
        accumulate_expert_grads: the backward adds the routed experts' weight gradients to
        self.grads["dw1"] / ["dw2"] (SWITCH_ACCUM_EXPERT_GRADS); idle experts are left as they are."""
        self.desc = SwitchMoeDesc(T=T, d_model=d_model, d_ff=d_ff, N=N, C=C, capacity_factor=capacity_factor,
                                  dtype=_DT[dtype], priority=_PRIO[priority],
                                  flags=(GATE_SCALE if gate_scale else 0) | (RESIDUAL_ALL if residual_all else 0)
                                  | (RENORM if renorm else 0) | (ACCUM_EXPERT_GRADS if accumulate_expert_grads else 0),
                                  d_ff_shared=d_ff_shared, top_k=top_k, routing=_ROUTING[routing],
                                  weight_format={"native": 0, "mxfp4": 1}[weight_format],
                                  expand_choices=expand)
        K = max(1, top_k)
        L = lib()
        nb = L.switch_moe_workspace_bytes(ctypes.byref(self.desc))
        if nb == 0:
            raise ValueError("invalid layer description (switch_moe_workspace_bytes returned 0): "
                             + L.switch_last_error().decode())
        self.C = C if C else min(T, switch_capacity(K * T, N, capacity_factor))
        dev = torch.device(device)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        tk = (T, K) if K > 1 else (T,)
        self.out = dict(y=_empty((T, d_model), dtype, dev), expert_id=_empty(tk, torch.int32, dev),
                        gate=_empty(tk, torch.float32, dev), slot=_empty(tk, torch.int32, dev),
                        routed_count=_empty(N, torch.int32, dev), kept_count=_empty(N, torch.int32, dev),
                        n_dropped=_empty(1, torch.int32, dev), f=_empty(N, torch.float32, dev),
                        P=_empty(N, torch.float32, dev), l_aux=_empty(1, torch.float32, dev))
        o = self.out
        self._outs = SwitchMoeOutputs(*[o[k].data_ptr() for k in
                                        ("y", "expert_id", "gate", "slot", "routed_count", "kept_count",
                                         "n_dropped", "f", "P", "l_aux")])
        self.dims = (T, d_model, d_ff, N, d_ff_shared, dtype, dev)
        self.saved = None
        if train:
            C_ = self.C
            sv = dict(probs=_empty((T, N), torch.float32, dev), token_of_slot=_empty((N, C_), torch.int32, dev),
                      active=_empty(N, torch.int32, dev), n_active=_empty(1, torch.int32, dev),
                      h=_empty((N, C_, d_ff), dtype, dev),
                      h_shared=_empty((T, d_ff_shared), dtype, dev) if d_ff_shared else None)
            self.saved = sv
            self._saved = SwitchMoeSaved(*[None if sv[k] is None else sv[k].data_ptr() for k in
                                           ("probs", "token_of_slot", "active", "n_active", "h", "h_shared")])
            self.bws = torch.empty(max(256, L.switch_moe_backward_workspace_bytes(ctypes.byref(self.desc))),
                                   dtype=torch.uint8, device=dev)
            wdt = dtype
            self.grads = dict(dx=_empty((T, d_model), dtype, dev), dw_gate=_empty((N, d_model), torch.float32, dev),
                              dbias=_empty(N, torch.float32, dev), dw1=_empty((N, d_model, d_ff), wdt, dev),
                              dw2=_empty((N, d_ff, d_model), wdt, dev),
                              dws1=_empty((d_model, d_ff_shared), wdt, dev) if d_ff_shared else None,
                              dws2=_empty((d_ff_shared, d_model), wdt, dev) if d_ff_shared else None)

    def __call__(self, x, w_gate, w1, w2, bias=None, ws1=None, ws2=None, stream=None, stage_events=None,
                 w1_scale=None, w2_scale=None, noalloc=False):
        """One layer forward.  stage_events: optional StageEvents (7 HIP events) recorded at the stage
        boundaries (switch_moe_forward_timed).  MXFP4 weights: w1 / w2 are the codes and
        w1_scale / w2_scale the E8M0 scales (switch_quantize_mxfp4).  noalloc: call
        switch_moe_forward_noalloc (the library's own scratch array instead of self.ws)."""
        ins = SwitchMoeInputs(x.data_ptr(), w_gate.data_ptr(), None if bias is None else bias.data_ptr(),
                              w1.data_ptr(), w2.data_ptr(), None if ws1 is None else ws1.data_ptr(),
                              None if ws2 is None else ws2.data_ptr(),
                              None if w1_scale is None else w1_scale.data_ptr(),
                              None if w2_scale is None else w2_scale.data_ptr())
        if noalloc:
            _check("switch_moe_forward_noalloc",
                   lib().switch_moe_forward_noalloc(ctypes.byref(self.desc), ctypes.byref(ins),
                                                    ctypes.byref(self._outs), _stream(stream)))
        elif stage_events is None:
            _check("switch_moe_forward", lib().switch_moe_forward(ctypes.byref(self.desc), ctypes.byref(ins),
                                                                  ctypes.byref(self._outs), _p(self.ws),
                                                                  self.ws.numel(), _stream(stream)))
        else:
            _check("switch_moe_forward_timed",
                   lib().switch_moe_forward_timed(ctypes.byref(self.desc), ctypes.byref(ins), ctypes.byref(self._outs),
                                                  _p(self.ws), self.ws.numel(), _stream(stream),
                                                  stage_events.handles))
        return self.out


    def forward_train(self, x, w_gate, w1, w2, bias=None, ws1=None, ws2=None, stream=None):
        """switch_moe_forward_train: the forward plus the saved tensors (self.saved) the backward reads."""
        if self.saved is None:
            raise RuntimeError("layer was built without train=True")
        ins = SwitchMoeInputs(x.data_ptr(), w_gate.data_ptr(), None if bias is None else bias.data_ptr(),
                              w1.data_ptr(), w2.data_ptr(), None if ws1 is None else ws1.data_ptr(),
                              None if ws2 is None else ws2.data_ptr())
        _check("switch_moe_forward_train",
               lib().switch_moe_forward_train(ctypes.byref(self.desc), ctypes.byref(ins), ctypes.byref(self._outs),
                                              ctypes.byref(self._saved), _p(self.ws), self.ws.numel(),
                                              _stream(stream)))
        return self.out

    def backward(self, x, w_gate, w1, w2, dy, dl_aux=None, bias=None, ws1=None, ws2=None, stream=None,
                 stage_events=None):
        """switch_moe_backward after forward_train on the same inputs; dl_aux: device fp32 [1] or None.
        stage_events: optional StageEvents(n=6) (switch_moe_backward_timed).
        Returns self.grads (dbias is None without a router bias)."""
        if self.saved is None:
            raise RuntimeError("layer was built without train=True")
        _need(dy, "dy")
        ins = SwitchMoeInputs(x.data_ptr(), w_gate.data_ptr(), None if bias is None else bias.data_ptr(),
                              w1.data_ptr(), w2.data_ptr(), None if ws1 is None else ws1.data_ptr(),
                              None if ws2 is None else ws2.data_ptr())
        g = self.grads
        gr = SwitchMoeGrads(g["dx"].data_ptr(), g["dw_gate"].data_ptr(),
                            None if bias is None else g["dbias"].data_ptr(), g["dw1"].data_ptr(), g["dw2"].data_ptr(),
                            None if g["dws1"] is None else g["dws1"].data_ptr(),
                            None if g["dws2"] is None else g["dws2"].data_ptr())
        if stage_events is None:
            _check("switch_moe_backward",
                   lib().switch_moe_backward(ctypes.byref(self.desc), ctypes.byref(ins), ctypes.byref(self._outs),
                                             ctypes.byref(self._saved), _p(dy), _p(dl_aux), ctypes.byref(gr),
                                             _p(self.bws), self.bws.numel(), _stream(stream)))
        else:
            _check("switch_moe_backward_timed",
                   lib().switch_moe_backward_timed(ctypes.byref(self.desc), ctypes.byref(ins),
                                                   ctypes.byref(self._outs), ctypes.byref(self._saved), _p(dy),
                                                   _p(dl_aux), ctypes.byref(gr), _p(self.bws), self.bws.numel(),
                                                   _stream(stream), stage_events.handles))
        out = dict(g)
        if bias is None:
            out["dbias"] = None
        return out


def switch_quantize_mxfp4(w, *, stream=None):
    """MXFP4 along K of w [B, K, Ncols] (bf16 or fp32): returns (codes [B, Ncols, K/2] uint8,
    scales [B, Ncols, K/32] uint8)."""
    _need(w, "w")
    B, K, Nc = w.shape
    codes = torch.empty((B, Nc, K // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((B, Nc, K // 32), dtype=torch.uint8, device=w.device)
    _check("switch_quantize_mxfp4", lib().switch_quantize_mxfp4(_p(w), _dtype(w), B, K, Nc, _p(codes), _p(scales),
                                                                _stream(stream)))
    return codes, scales


def switch_moe_forward_train(layer: "SwitchMoE", x, w_gate, w1, w2, **kw):
    """Training forward on a SwitchMoE built with train=True (outputs in layer.out, saved in layer.saved)."""
    return layer.forward_train(x, w_gate, w1, w2, **kw)


def switch_moe_backward(layer: "SwitchMoE", x, w_gate, w1, w2, dy, dl_aux=None, **kw):
    """Backward of the last forward_train of `layer`; returns the gradient dict."""
    return layer.backward(x, w_gate, w1, w2, dy, dl_aux=dl_aux, **kw)


def switch_moe_forward(x, w_gate, w1, w2, *, bias=None, capacity_factor=1.0, C=0, priority="token",
                       gate_scale=True, residual_all=False, ws1=None, ws2=None, stream=None):
    """One-shot whole-layer forward; returns the output dict (fresh tensors)."""
    T, d = x.shape
    N = w_gate.shape[0]
    dff = w1.shape[2]
    layer = SwitchMoE(T, d, dff, N, dtype=x.dtype, capacity_factor=capacity_factor, C=C, priority=priority,
                      gate_scale=gate_scale, residual_all=residual_all,
                      d_ff_shared=0 if ws1 is None else ws1.shape[1], device=x.device)
    out = layer(x, w_gate, w1, w2, bias=bias, ws1=ws1, ws2=ws2, stream=stream)
    out["C"] = layer.C
    return out
