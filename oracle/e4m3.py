"""E4M3 codec and tile/block quantiser of the oracle (test infrastructure only).

This module is part of the CPU oracle.  It is test infrastructure: only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it.  It
shares no code with the HIP library.

Sources
-------
[RG-FP8]  "DeepSeek-V3 Technical Report" reading guide (xyznot.com, Turkish
          edition "Okuma rehberi" and French edition "Guide de lecture"),
          section "Key ideas" ("Temel fikirler" / "Idees cles"), FP8
          mixed-precision bullet: E4M3 on all tensors, 1x128 tile-wise
          activation scaling, 128x128 block-wise weight scaling.
[OCP-FP8] OCP 8-bit Floating Point Specification (OFP8), the E4M3 encoding
          with no infinities ("FN"): 1 sign bit, 4 exponent bits with bias 7,
          3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; the only
          NaN patterns are S.1111.111; the largest finite value is 448.

The pages name E4M3 and the tile shapes but print neither the variant nor the
scale rule.  Readings taken here (the same readings the GPU side implements):
  * variant: OCP E4M3FN (largest finite 448), the native fp8 of the target;
  * scale of a tile: the smallest power of two 2^k with amax <= 448 * 2^k
    (k >= -126; an all-zero tile has scale 1).  A power-of-two scale is what
    the target's block-scaled matrix instructions apply (an E8M0 exponent),
    and it makes x / scale and code * scale exact;
  * code of x: round-to-nearest-even of x / scale (exact), which lies in
    [-448, 448]; NaN is never produced.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN code, straight from the field definitions [OCP-FP8]."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * man_field * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


# Table of all 256 code values, built code by code from the definition above.
DECODE_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# Non-negative finite values in code order 0x00..0x7E.  For a non-negative
# number the code equals its position here, and the values increase with it.
_POS_VALUES = DECODE_TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Codes (uint8) -> fp64 values."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne(x: np.ndarray) -> np.ndarray:
    """Round finite values to the nearest E4M3FN code, ties to the even code.

    Values are first clamped to [-448, 448], so the result is never NaN.
    The nearest code is found by locating x between its two neighbours in the
    table of representable values; on an exact tie the code whose lowest
    mantissa bit is 0 wins (round-half-to-even).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode_rne: non-finite input")
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # _POS[hi-1] < a <= _POS[hi]
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == _POS_VALUES[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return (code | (sign.astype(np.uint8) << 7)).astype(np.uint8)


def quantize_tiles(x: np.ndarray, tile_rows: int, tile_cols: int):
    """Tile-wise E4M3 quantisation [RG-FP8].

    x: [rows, cols] array of values that are exactly representable in fp32.
    tile_rows x tile_cols tiles (1x128 for activations, 128x128 for weights);
    rows must divide by tile_rows and cols by tile_cols.
    Returns (codes uint8 [rows, cols], scales fp32 [rows/tile_rows, cols/tile_cols]).
    """
    x = np.asarray(x)
    rows, cols = x.shape
    if rows % tile_rows or cols % tile_cols:
        raise ValueError("quantize_tiles: shape not a multiple of the tile")
    x32 = x.astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("quantize_tiles: input not exactly representable in fp32")
    rt, ct = rows // tile_rows, cols // tile_cols
    tiles = x32.reshape(rt, tile_rows, ct, tile_cols).astype(np.float64)
    amax = np.abs(tiles).max(axis=(1, 3))                       # exact
    scale = pow2_scales(amax)
    scaled = tiles / scale[:, None, :, None]                    # exact: a power of two
    codes = e4m3_encode_rne(scaled).reshape(rows, cols)
    return codes, scale.astype(np.float32)


def pow2_scales(amax: np.ndarray) -> np.ndarray:
    """Smallest 2^k (k >= -126) with amax <= 448 * 2^k, elementwise; 1 where amax == 0.

    With amax = m * 2^e (frexp: 0.5 <= m < 1) and 448 = 0.875 * 2^9, the
    condition m * 2^e <= 0.875 * 2^(9 + k) holds first at k = e - 9 when
    m <= 0.875 and at k = e - 8 otherwise."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)
    k = np.where(m <= 0.875, e - 9, e - 8)
    k = np.maximum(k, -126)
    return np.where(amax > 0, np.ldexp(1.0, k), 1.0)


def pow2_scale(amax: float) -> float:
    """The same scale found by search: the first k from -126 up that works."""
    if amax == 0.0:
        return 1.0
    k = -126
    while amax > E4M3_MAX * 2.0 ** k:
        k += 1
    return 2.0 ** k


def dequantize_tiles(codes: np.ndarray, scale: np.ndarray, tile_rows: int, tile_cols: int) -> np.ndarray:
    """codes x scale of their tile, in fp64 (exact: a 4-bit by 24-bit product)."""
    rows, cols = codes.shape
    s = np.repeat(np.repeat(np.asarray(scale, dtype=np.float64), tile_rows, axis=0), tile_cols, axis=1)
    return e4m3_decode(codes) * s[:rows, :cols]
