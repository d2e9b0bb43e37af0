"""FP8 (OCP e4m3fn) codec and per-tile dynamic scaling (test infrastructure only).

The Triton walkthrough page, section 4.1, quantises K with a dynamic scale
taken from the block's largest magnitude, runs the product of the quantised
operands, and multiplies the scores by ``1/(q_scale*k_scale)``.  Its constant
is the int8 range 127 and the epsilon's operator is lost in the page text;
the reading taken here uses the e4m3fn range and guards an all-zero tile:

    amax_t  = max |x| over the tile (64 rows x d columns, exact in float32)
    scale_t = float32(448) / max(amax_t, float32(1e-6))      (IEEE fp32 divide)
    y       = float32(x * scale_t)                            (fp32 multiply, RNE)
    code    = e4m3fn(clamp(y, -448, 448))                     (nearest, ties to even)

Q and K are quantised independently; a partial last tile uses only the
rows present.

e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
infinities, NaN only at exponent and mantissa all ones (codes 0x7F, 0xFF),
largest finite 448, subnormal step 2**-9.  The decoder below follows that
definition bit field by bit field; the encoder picks, among the 127
non-negative finite values, the nearest one, breaking ties towards the even
code, and applies the sign bit of y.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
TILE_ROWS = 64
_EPS = np.float32(1e-6)


def decode_e4m3(codes) -> np.ndarray:
    """Decode e4m3fn byte codes to float64 values (NaN for 0x7F/0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.power(2.0, exp_field - 7)
    subnormal = sign * (man / 8.0) * 2.0 ** -6
    val = np.where(exp_field == 0, subnormal, normal)
    return np.where((exp_field == 0xF) & (man == 0x7), np.nan, val)


# Non-negative finite codes 0x00..0x7E; their values increase with the code.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = decode_e4m3(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0)


def encode_e4m3(y) -> np.ndarray:
    """Encode finite values with |y| <= 448 to e4m3fn codes, round to nearest even.

    ``y`` is taken exactly (float64 holds every float32).  Values outside
    [-448, 448] are rejected: callers clamp first.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("encode_e4m3 expects finite values within [-448, 448]")
    a = np.abs(y)
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, mag | np.uint8(0x80), mag).astype(np.uint8)


def quantize_tiles(x, tile_rows: int = TILE_ROWS):
    """Per-tile dynamic quantisation of ``x [B, H, N, d]`` (float32 values).

    Returns ``(codes uint8 [B,H,N,d], scale float32 [B,H,ceil(N/tile_rows)])``.
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    n_tiles = (N + tile_rows - 1) // tile_rows
    codes = np.empty((B, H, N, d), dtype=np.uint8)
    scale = np.empty((B, H, n_tiles), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for t in range(n_tiles):
                tile = x[b, h, t * tile_rows:(t + 1) * tile_rows]
                amax = np.float32(np.max(np.abs(tile)))
                s = np.float32(E4M3_MAX) / np.maximum(amax, _EPS)
                y = (tile * s).astype(np.float32)
                y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
                codes[b, h, t * tile_rows:(t + 1) * tile_rows] = encode_e4m3(y)
                scale[b, h, t] = s
    return codes, scale


# ---------------------------------------------------------------------------
# Power-of-two scaled e4m3 for the P*V product.  The pages give the dynamic
# per-block scale only for K (and by the same reading Q); for an FP8 P*V they
# name FP8 without details (tag page, excerpt on V3).  The reading taken here
# keeps every scale a power of two, so that scaling is exact and the product's
# dequantisation is the matrix core's own per-block exponent:
#
#   V: for each (b, h), 64-key tile t and column c,
#        e = the largest integer with amax * 2**e <= 448 (amax = max |V| over
#            the tile's keys in column c; e = 0 for an all-zero column),
#        code = e4m3fn(V * 2**e)          (exact scaling, then nearest-even),
#        value = decode(code) * 2**-e.
#   P: each probability tile of one query is scaled the same way from its
#      largest entry inside the kernel; that rounding is not reproduced here
#      (the parity tolerance accounts for it).
# ---------------------------------------------------------------------------

def pow2_exponent(amax) -> np.ndarray:
    """Largest integer e with amax * 2**e <= 448 (0 where amax == 0), clipped to
    [-127, 127] (the range of an 8-bit block exponent), elementwise.

    Exact: amax = m * 2**x with m in [0.5, 1) and 448 = 0.875 * 2**9, so
    e = 9 - x when m <= 0.875 and 8 - x otherwise.
    """
    a = np.asarray(amax, dtype=np.float64)
    m, x = np.frexp(a)
    e = np.where(m <= 0.875, 9 - x, 8 - x)
    return np.clip(np.where(a == 0.0, 0, e), -127, 127).astype(np.int64)


def quantize_v_pow2(v, tile_rows: int = TILE_ROWS):
    """Power-of-two e4m3 quantisation of ``v [B, H, N, d]`` per (64-key tile, column).

    Returns ``(codes uint8 [B,H,N,d], exps int64 [B,H,ceil(N/tile_rows),d])``;
    ``decode_e4m3(codes) * 2**-exps`` (tile-broadcast) gives the values used.
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    B, H, N, d = v.shape
    n_tiles = (N + tile_rows - 1) // tile_rows
    codes = np.empty((B, H, N, d), dtype=np.uint8)
    exps = np.empty((B, H, n_tiles, d), dtype=np.int64)
    for t in range(n_tiles):
        rows = slice(t * tile_rows, min(N, (t + 1) * tile_rows))
        amax = np.abs(v[:, :, rows]).max(axis=2)               # [B, H, d]
        e = pow2_exponent(amax)
        exps[:, :, t] = e
        codes[:, :, rows] = encode_e4m3(np.ldexp(v[:, :, rows], e[:, :, None, :]))
    return codes, exps


def dequantize_v_pow2(codes, exps, tile_rows: int = TILE_ROWS) -> np.ndarray:
    """Values ``decode(code) * 2**-e`` of a power-of-two quantised V (float64)."""
    vals = decode_e4m3(codes)
    N = vals.shape[2]
    e_rows = np.repeat(np.asarray(exps), tile_rows, axis=2)[:, :, :N]
    return np.ldexp(vals, -e_rows)
