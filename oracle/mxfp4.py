"""fp64 oracle of MXFP4 expert weights (weight-only microscaling quantization).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The pages name the format: an open-MoE routing comparison page (attain.fans,
MarkTechPost translation), TL;DR and the gpt-oss passage, says gpt-oss-120b
ships its MoE weights in MXFP4 so that the model fits one 80 GB GPU.  The
format itself is the published OCP Microscaling Formats (MX) v1.0
specification, restated here from its definitions:
  * a block of 32 consecutive elements (here: along the reduction dimension
    of the expert GEMM) shares one E8M0 scale X = 2^E, E an integer in
    [-127, 127], stored as the byte E + 127;
  * each element is FP4 E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa
    bit): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  * conversion: E = floor(log2(max_i |V_i|)) - 2 (2 = the largest exponent of
    E2M1), clamped to [-127, 127]; each V_i / X is rounded to the nearest E2M1
    value, ties to the even mantissa, and values beyond the largest magnitude
    saturate to +-6.
Readings where the specification leaves a choice: an all-zero block takes
E = -127; the sign bit of an element is the sign of V_i (so a negative value
that rounds to zero keeps its sign); two elements share a byte, the lower
index in the low nibble.

Layout (chosen so that the GEMM's reduction dimension is contiguous): a
weight W [E][K][Ncols] quantized along K becomes codes [E][Ncols][K/2] (bytes)
and scales [E][Ncols][K/32] (E8M0 bytes).

Parity status: pinned by an exhaustive nearest-value search over a dense grid
(tests/test_oracle_mxfp4_pins.py), the tie cases, exact round trips of values
on the scaled grid, and the scale rule on hand-picked blocks.
"""
from __future__ import annotations

import numpy as np

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLOCK = 32


def fp4_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (ties to the even mantissa), saturating at 6; sign bit = sign of v."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    # boundaries between consecutive magnitudes and the code taken on a tie
    mag = np.zeros(a.shape, dtype=np.uint8)
    # (lower code, upper code): midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5
    for lo in range(7):
        mid = 0.5 * (E2M1[lo] + E2M1[lo + 1])
        up = lo + 1
        even = lo if lo % 2 == 0 else up  # mantissa bit = code & 1
        mag = np.where(a > mid, up, np.where(a == mid, np.maximum(mag, even), mag)).astype(np.uint8)
    sign = np.signbit(np.asarray(v, dtype=np.float64)).astype(np.uint8)
    return (sign << 3) | mag


def fp4_decode(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1[code & 7]
    return np.where(code & 8, -mag, mag)


def block_scale_exp(block: np.ndarray) -> np.ndarray:
    """E = clamp(floor(log2(max |v|)) - 2, -127, 127) over the last axis; -127 for all-zero blocks."""
    amax = np.max(np.abs(block), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize(w: np.ndarray):
    """W [E][K][Ncols] (float) -> (codes [E][Ncols][K/2] uint8, scales [E][Ncols][K/32] uint8)."""
    w = np.asarray(w, dtype=np.float64)
    E_, K, Nc = w.shape
    assert K % BLOCK == 0
    wt = np.swapaxes(w, 1, 2).reshape(E_, Nc, K // BLOCK, BLOCK)   # blocks along K
    e = block_scale_exp(wt)                                         # [E][Nc][K/32]
    x = wt / np.ldexp(1.0, e)[..., None]
    c = fp4_encode(x).reshape(E_, Nc, K)
    codes = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse layout: -> W [E][K][Ncols] fp64 (exact)."""
    E_, Nc, K2 = codes.shape
    c = np.empty((E_, Nc, 2 * K2), dtype=np.uint8)
    c[..., 0::2] = codes & 15
    c[..., 1::2] = codes >> 4
    v = fp4_decode(c).reshape(E_, Nc, 2 * K2 // BLOCK, BLOCK)
    v = v * np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    return np.swapaxes(v.reshape(E_, Nc, 2 * K2), 1, 2)
