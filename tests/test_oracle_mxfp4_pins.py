"""Pins of the MXFP4 weight oracle (CPU only): the element rounding against an
exhaustive nearest-value search, the tie rule, exact round trips of values on
the scaled grid, the block-scale rule on hand-picked blocks, and the byte and
block layout."""
import numpy as np
import pytest

from oracle import mxfp4 as mx

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _nearest(v):
    """Brute force: nearest magnitude by distance (ties to the even mantissa: the
    code with (code & 1) == 0), saturating at 6, sign bit from v."""
    a = abs(v)
    best = None
    for code, m in enumerate(GRID):
        dist = abs(a - m)
        if best is None or dist < best[0] or (dist == best[0] and code % 2 == 0):
            best = (dist, code)
    code = best[1]
    if a > 6.0:
        code = 7
    return code | (8 if np.signbit(v) else 0)


def test_element_rounding_exhaustive():
    vals = np.concatenate([np.linspace(-8, 8, 64001), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 7.999,
                                                         -0.0, 0.0, 1e-9, -1e-9, 100.0, -100.0]])
    got = mx.fp4_encode(vals)
    want = np.array([_nearest(v) for v in vals], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_tie_cases():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, code in ties.items():
        assert int(mx.fp4_encode(np.array([v]))[0]) == code, v
        assert int(mx.fp4_encode(np.array([-v]))[0]) == code | 8, -v


@pytest.mark.parametrize("e", [-127, -30, -2, 0, 7, 120])
def test_scaled_grid_round_trips(e):
    rng = np.random.default_rng(e + 200)
    codes = rng.integers(0, 16, size=(2, 3, 64)).astype(np.uint8)
    codes[..., 0] = 7  # each block's max magnitude is 6 so the scale comes out as 2^e
    codes[..., 32] = 15
    vals = mx.fp4_decode(codes) * np.ldexp(1.0, e)       # [E][Ncols][K]
    w = np.swapaxes(vals, 1, 2)                          # [E][K][Ncols]
    q, s = mx.quantize(w)
    assert (s == e + 127).all()
    np.testing.assert_array_equal(mx.dequantize(q, s), w)


def test_block_scale_rule():
    blocks = np.zeros((5, 32))
    blocks[0, 3] = 1.0      # floor(log2 1) - 2 = -2: 1 / 2^-2 = 4 -> code 6
    blocks[1, 0] = -7.0     # E = 0, 7 saturates to 6
    blocks[2, 5] = 6.0      # E = 0
    blocks[3, 9] = 0.3      # floor(log2 0.3) = -2 -> E = -4: 0.3 * 16 = 4.8 -> 4
    # block 4: all zero -> E = -127
    np.testing.assert_array_equal(mx.block_scale_exp(blocks), [-2, 0, 0, -4, -127])
    w = blocks.T[None]                                   # [1][K=32][Ncols=5]
    q, s = mx.quantize(w)
    d = mx.dequantize(q, s)[0].T
    assert d[0, 3] == 1.0 and d[1, 0] == -6.0 and d[2, 5] == 6.0 and d[3, 9] == 0.25
    assert not d[4].any() and s[0, 4, 0] == 0


def test_layout_nibbles_and_blocks():
    w = np.zeros((1, 64, 2))
    w[0, 0, 0] = 1.0    # column 0, k = 0: low nibble of byte 0
    w[0, 1, 0] = 2.0    # column 0, k = 1: high nibble of byte 0; block max 2 -> E = -1, X = 0.5
    w[0, 40, 1] = -3.0  # column 1, k = 40: second block (max 3 -> E = -1), byte 20, low nibble
    q, s = mx.quantize(w)
    assert q.shape == (1, 2, 32) and s.shape == (1, 2, 2)
    assert s[0, 0, 0] == 126 and q[0, 0, 0] == (4 | (6 << 4))   # 1 / 0.5 = 2 -> code 4; 2 / 0.5 = 4 -> code 6
    assert s[0, 1, 0] == 0 and s[0, 1, 1] == 126                 # an all-zero block takes E = -127
    assert q[0, 1, 20] == 15                                     # -3 / 0.5 = -6 -> sign | 7
    assert q[0, 1, :20].sum() == 0 and q[0, 1, 21:].sum() == 0


def test_error_bound():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((2, 128, 16)) * np.ldexp(1.0, rng.integers(-20, 20, size=(2, 1, 16)))
    q, s = mx.quantize(w)
    d = mx.dequantize(q, s)
    X = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=2).swapaxes(1, 2)  # [E][K][Ncols]
    err = np.abs(w - d)
    inside = np.abs(w) <= 6 * X
    assert (err[inside] <= X[inside]).all()       # half the widest spacing (2 X) of the E2M1 grid
    assert (err[~inside] < 2 * X[~inside]).all()  # saturated: |v| < 8 X rounds to 6 X
