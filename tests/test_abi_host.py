"""C ABI on the host (no GPU needed): the library loads, exports every function
the header declares, and rejects bad arguments before launching anything."""
import ctypes

import pytest

from switch_top_routed_amd import native

E_NULL, E_SHAPE, E_UNSUP, E_WS, E_ALIGN = 1, 2, 3, 4, 6
FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def L():
    return native.lib()


def test_exports_every_declared_symbol(L):
    names = native.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(native._SIGS)


def test_capacity(L):
    assert L.switch_capacity(4096, 128, 1.25) == 40
    assert L.switch_capacity(256, 8, 1.0) == 32
    assert L.switch_capacity(128, 384, 2.0) == 1
    assert L.switch_capacity(16384, 128, 1.25) == 160
    assert L.switch_capacity(4096, 128, 0.5) == 16
    assert L.switch_capacity(0, 8, 1.0) == -1
    assert L.switch_capacity(10, 8, 0.0) == -1
    assert L.switch_capacity(10, 1, 5.0) == 10  # clamped to T


def test_capacity_decimal_rule_matches_oracle(L):
    """C = max(1, ceil(cf T / N)) on the decimal value of cf, as the oracle
    computes it (exact rationals); double arithmetic would round 1.1 * 100 / 10
    up to 12."""
    import oracle
    from oracle import routing as orr
    assert L.switch_capacity(100, 10, 1.1) == oracle.capacity(100, 10, 1.1) == 11
    assert L.switch_capacity(100, 2, 1.1) == oracle.capacity(100, 2, 1.1) == 55
    assert L.switch_capacity(30, 10, 0.7) == oracle.capacity(30, 10, 0.7) == 3
    cfs = [0.1, 0.2, 0.3, 0.5, 0.7, 0.8, 0.9, 1.0, 1.1, 1.2, 1.25, 1.3, 1.5, 1.7, 2.0, 2.2, 3.3, 0.05, 1.15, 1.35]
    for cf in cfs:
        for T in (1, 7, 10, 30, 100, 128, 1000, 4096, 16384, 100_000):
            for N in (1, 2, 3, 7, 8, 10, 128, 384, 1000):
                want = min(T, oracle.capacity(T, N, cf))
                assert L.switch_capacity(T, N, cf) == want, (T, N, cf)
                assert min(T, orr.capacity_topk(T, N, 1, cf)) == want
    assert L.switch_capacity(10, 8, float("nan")) == -1
    assert L.switch_capacity(10, 8, float("inf")) == -1


def test_status_strings(L):
    for s in range(7):
        assert L.switch_status_str(s)
    assert L.switch_status_str(99) == b"unknown status"


def _route(L, x=FAKE, wg=FAKE, T=64, d=128, N=8, dtype=1, outs=FAKE, ws=FAKE, wsb=1 << 30):
    return L.switch_route(x, wg, None, T, d, N, dtype, outs, outs, outs, outs, outs, outs, ws, wsb, None)


def test_route_validation(L):
    assert _route(L, x=None) == E_NULL
    assert b"x is NULL" in L.switch_last_error()
    assert _route(L, wg=None) == E_NULL
    assert _route(L, outs=None) == E_NULL
    assert _route(L, T=0) == E_SHAPE
    assert _route(L, N=0) == E_SHAPE
    assert _route(L, N=1025) == E_SHAPE
    assert _route(L, d=100) == E_SHAPE  # bf16 needs d % 32 == 0
    assert _route(L, dtype=7) == E_UNSUP
    assert _route(L, x=ctypes.c_void_p((1 << 20) + 2)) == E_ALIGN
    assert _route(L, wsb=0) == E_WS
    assert _route(L, ws=None) == E_NULL


def test_workspace_sizes(L):
    assert L.switch_route_workspace_bytes(4096, 768, 128, 1) > 0
    assert L.switch_assign_workspace_bytes(4096, 128, 40, 1) > L.switch_assign_workspace_bytes(4096, 128, 40, 0)
    assert L.switch_expert_ffn_workspace_bytes(128, 40, 768, 3072, 1) >= 128 * 40 * 3072 * 2
    d = native.SwitchMoeDesc(T=4096, d_model=768, d_ff=3072, N=128, C=0, capacity_factor=1.25, dtype=1,
                             priority=0, flags=1, d_ff_shared=0)
    assert L.switch_moe_workspace_bytes(ctypes.byref(d)) > 0
    d.d_model = 100
    assert L.switch_moe_workspace_bytes(ctypes.byref(d)) == 0


def test_assign_validation(L):
    f = L.switch_assign_capacity
    args = lambda **k: dict(dict(eid=FAKE, gate=FAKE, T=64, N=8, C=8, pr=0), **k)

    def call(**k):
        a = args(**k)
        return f(a["eid"], a["gate"], a["T"], a["N"], a["C"], a["pr"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 1 << 30, None)
    assert call(C=0) == E_SHAPE
    assert call(C=65) == E_SHAPE
    assert call(pr=2) == E_UNSUP
    assert call(eid=None) == E_NULL
    assert call(gate=None, pr=1) == E_NULL


def test_ffn_and_combine_validation(L):
    ffn = L.switch_expert_ffn
    assert ffn(FAKE, FAKE, FAKE, 1, 8, 8, 100, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == E_SHAPE
    assert ffn(FAKE, FAKE, FAKE, 1, 8, 8, 128, 200, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == E_SHAPE
    assert ffn(None, FAKE, FAKE, 1, 8, 8, 128, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == E_NULL
    assert ffn(FAKE, FAKE, FAKE, 1, 8, 8, 128, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == E_WS
    comb = L.switch_combine
    assert comb(FAKE, FAKE, None, 1, 64, 128, FAKE, FAKE, FAKE, 8, 8, 4, FAKE, None) == E_UNSUP
    assert comb(FAKE, FAKE, None, 1, 64, 128, FAKE, FAKE, None, 8, 8, 1, FAKE, None) == E_NULL
    assert comb(FAKE, FAKE, None, 1, 64, 12, FAKE, FAKE, FAKE, 8, 8, 1, FAKE, None) == E_SHAPE
    disp = L.switch_dispatch
    assert disp(FAKE, 1, 64, 12, FAKE, FAKE, 8, 8, FAKE, None) == E_SHAPE
    assert disp(FAKE, 1, 64, 128, FAKE, FAKE, 8, 65, FAKE, None) == E_SHAPE


def test_forward_validation(L):
    d = native.SwitchMoeDesc(T=64, d_model=128, d_ff=128, N=8, C=0, capacity_factor=1.0, dtype=1, priority=0,
                             flags=1, d_ff_shared=0)
    ins = native.SwitchMoeInputs(1 << 20, 1 << 20, None, 1 << 20, 1 << 20, None, None)
    outs = native.SwitchMoeOutputs(*([1 << 20] * 10))
    fwd = L.switch_moe_forward
    assert fwd(None, ctypes.byref(ins), ctypes.byref(outs), FAKE, 1 << 30, None) == E_NULL
    assert fwd(ctypes.byref(d), None, ctypes.byref(outs), FAKE, 1 << 30, None) == E_NULL
    assert fwd(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), FAKE, 16, None) == E_WS
    d.flags = 16  # an unknown flag bit
    assert fwd(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), FAKE, 1 << 30, None) == E_UNSUP
    d.flags = 1
    d.d_ff_shared = 128
    assert fwd(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), FAKE, 1 << 30, None) == E_NULL  # ws1 missing
    d.d_ff_shared = 0
    d.capacity_factor = 0.0
    assert fwd(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), FAKE, 1 << 30, None) == E_SHAPE
    # bf16 rows must be multiples of 128 elements (the kernels' granule); refused before any launch
    d.capacity_factor = 1.0
    for dm, dff in ((776, 3072), (768, 3080), (776, 3080)):
        d.d_model, d.d_ff = dm, dff
        assert fwd(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), FAKE, 1 << 30, None) == E_SHAPE
        assert b"multiple of 128" in L.switch_last_error()
        assert L.switch_moe_workspace_bytes(ctypes.byref(d)) == 0


def test_timed_forward_validation(L):
    d = native.SwitchMoeDesc(T=64, d_model=128, d_ff=256, N=8, C=0, capacity_factor=1.0, dtype=1,
                             priority=0, flags=1, d_ff_shared=0)
    assert L.switch_moe_forward_timed(ctypes.byref(d), None, None, FAKE, 1 << 30, None, None) == E_NULL
    assert b"stage_events" in L.switch_last_error()
    ev = (ctypes.c_void_p * 7)()
    assert L.switch_moe_forward_timed(ctypes.byref(d), None, None, FAKE, 1 << 30, None, ev) == E_NULL
    assert b"inputs is NULL" in L.switch_last_error()


def test_size_limits_for_32bit_offsets(L):
    """One expert's weight matrix must stay addressable with 32-bit buffer offsets."""
    ffn = L.switch_expert_ffn
    assert ffn(FAKE, FAKE, FAKE, 1, 8, 8, 65536, 32768, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 62, None) == E_SHAPE
    assert b"exceeds 2^30" in L.switch_last_error()
    d = native.SwitchMoeDesc(T=64, d_model=65536, d_ff=32768, N=8, C=0, capacity_factor=1.0, dtype=1,
                             priority=0, flags=1, d_ff_shared=0)
    assert L.switch_moe_workspace_bytes(ctypes.byref(d)) == 0
    assert _route(L, d=(1 << 20) + 128) == E_SHAPE


def test_train_forward_and_backward_validation(L):
    d = native.SwitchMoeDesc(T=64, d_model=128, d_ff=128, N=8, C=0, capacity_factor=1.0, dtype=1, priority=0,
                             flags=1, d_ff_shared=0)
    ins = native.SwitchMoeInputs(1 << 20, 1 << 20, None, 1 << 20, 1 << 20, None, None)
    outs = native.SwitchMoeOutputs(*([1 << 20] * 10))
    sv = native.SwitchMoeSaved(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None)
    gr = native.SwitchMoeGrads(1 << 20, 1 << 20, None, 1 << 20, 1 << 20, None, None)
    ftr = L.switch_moe_forward_train
    assert ftr(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), None, FAKE, 1 << 30, None) == E_NULL
    assert b"saved is NULL" in L.switch_last_error()
    sv.h = None
    assert ftr(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), ctypes.byref(sv), FAKE, 1 << 30, None) == E_NULL
    assert b"h is NULL" in L.switch_last_error()
    sv.h = (1 << 20) + 8
    assert ftr(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), ctypes.byref(sv), FAKE, 1 << 30, None) == E_ALIGN
    sv.h = 1 << 20
    # same workspace as the plain forward
    assert L.switch_moe_workspace_bytes(ctypes.byref(d)) > 0
    bwd = L.switch_moe_backward
    nb = L.switch_moe_backward_workspace_bytes(ctypes.byref(d))
    assert nb > 0
    args = lambda **k: [ctypes.byref(d), k.get("ins", ctypes.byref(ins)), k.get("fwd", ctypes.byref(outs)),
                        k.get("sv", ctypes.byref(sv)), k.get("dy", FAKE), None, k.get("gr", ctypes.byref(gr)),
                        FAKE, k.get("wsb", nb), None]
    assert bwd(*args(fwd=None)) == E_NULL
    assert bwd(*args(sv=None)) == E_NULL
    assert bwd(*args(gr=None)) == E_NULL
    assert bwd(*args(dy=None)) == E_NULL
    assert bwd(*args(wsb=nb - 1)) == E_WS
    gr.dw1 = None
    assert bwd(*args()) == E_NULL and b"dw1" in L.switch_last_error()
    gr.dw1 = 1 << 20
    d.d_ff_shared = 128
    assert bwd(*args()) == E_NULL  # shared weights and their gradients missing
    d.d_ff_shared = 0
    d.flags = 16
    assert bwd(*args()) == E_UNSUP
    assert L.switch_moe_backward_workspace_bytes(ctypes.byref(d)) == 0


def test_expanded_drop_validation(L):
    """Expanded Drop: top-1 token choice only, M in [2, min(N, 8)], no RENORM, C <= 8192, inference only."""
    def ws(**kw):
        base = dict(T=1024, d_model=128, d_ff=128, N=8, C=0, capacity_factor=1.0, dtype=1, priority=0, flags=1,
                    d_ff_shared=0, expand_choices=2)
        base.update(kw)
        return L.switch_moe_workspace_bytes(ctypes.byref(native.SwitchMoeDesc(**base)))
    assert ws() > ws(expand_choices=0) == ws(expand_choices=1) > 0
    assert ws(expand_choices=8) > ws(expand_choices=2)
    assert ws(priority=1, expand_choices=4) > 0
    assert ws(expand_choices=9) == 0 and b"expand_choices" in L.switch_last_error()
    assert ws(N=4, expand_choices=5) == 0
    assert ws(top_k=2) == 0 and b"top-1" in L.switch_last_error()
    assert ws(routing=1) == 0
    assert ws(flags=1 | 4) == 0 and b"RENORM" in L.switch_last_error()
    assert ws(T=20000, N=2, C=9000) == 0 and b"Expanded Drop" in L.switch_last_error()
    assert ws(T=20000, N=2, C=8192) > 0
    d = native.SwitchMoeDesc(T=64, d_model=128, d_ff=128, N=8, C=0, capacity_factor=1.0, dtype=1, priority=0,
                             flags=1, d_ff_shared=0, expand_choices=2)
    ins = native.SwitchMoeInputs(1 << 20, 1 << 20, None, 1 << 20, 1 << 20, None, None)
    outs = native.SwitchMoeOutputs(*([1 << 20] * 10))
    sv = native.SwitchMoeSaved(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None)
    assert L.switch_moe_forward_train(ctypes.byref(d), ctypes.byref(ins), ctypes.byref(outs), ctypes.byref(sv),
                                      FAKE, 1 << 30, None) == E_UNSUP
    assert L.switch_moe_backward_workspace_bytes(ctypes.byref(d)) == 0
