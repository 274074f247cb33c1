"""E2M1 (FP4) and E4M3 (FP8) codecs, written from the format definitions.

Test infrastructure only (see ``oracle/__init__.py``).

E2M1 [Notes07 §01 Background]: the pages give the representable set
{0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6} with largest magnitude 6.  Here the
table is built from the bit-level definition (1 sign, 2 exponent bits with
bias 1, 1 mantissa bit, subnormals at exponent 0) and a test checks that it
equals the printed set.  Code layout: bit 3 = sign, bits 2..0 = magnitude
index 0..7.

Rounding to E2M1 is round-to-nearest with ties to the even code and
saturation at 6 (a reading: the pages do not name the rounding mode).

E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals at exponent 0, no infinities, S.1111.111 is NaN, largest finite 448.
The pages only say "fp8" for the block scale ([Notes07 §02 FourOverSix]);
E4M3 is the problem statement's choice.  Rounding is round-to-nearest-even;
a value above 464 (the midpoint between 448 and the first non-finite pattern)
overflows, which is reported to the caller instead of producing a number.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# E2M1
# ---------------------------------------------------------------------------


def _e2m1_mag_from_bits(mag_code: int) -> float:
    """Magnitude of a 3-bit E2M1 magnitude code from the format definition."""
    e = (mag_code >> 1) & 0x3
    m = mag_code & 0x1
    if e == 0:  # subnormal: 2^(1-bias) * (m / 2) with bias 1
        return 0.5 * m
    return float(2.0 ** (e - 1)) * (1.0 + m / 2.0)


#: magnitudes of codes 0..7, ascending
E2M1_MAG_VALUES = np.array([_e2m1_mag_from_bits(c) for c in range(8)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """4-bit codes (bit 3 = sign) -> float64 values.  Negative zero is kept."""
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAG_VALUES[codes & 0x7]
    return np.where((codes & 0x8) != 0, -mag, mag)


def e2m1_round_mag(v) -> np.ndarray:
    """Round non-negative values to the nearest E2M1 magnitude code.

    Nearest in absolute distance; on an exact tie the even code wins; values
    above 6 saturate to code 7 (=6).  ``v`` must be >= 0 and not NaN (+inf is
    allowed and saturates).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)) or np.any(v < 0):
        raise ValueError("e2m1_round_mag expects non-negative, non-NaN input")
    vals = E2M1_MAG_VALUES
    hi = np.searchsorted(vals, v, side="left")  # first table value >= v
    hi_c = np.minimum(hi, 7)
    lo_c = np.maximum(hi - 1, 0)
    with np.errstate(invalid="ignore"):
        d_lo = v - vals[lo_c]
        d_hi = vals[hi_c] - v
    pick_lo = d_lo < d_hi
    tie = d_lo == d_hi
    even_lo = (lo_c % 2) == 0
    out = np.where(pick_lo | (tie & even_lo), lo_c, hi_c)
    # v above the largest value: hi == 8, both indices are 7 (saturation)
    out = np.where(hi >= 8, 7, out)
    # v exactly 0 or below the first value: hi == 0
    out = np.where(hi == 0, 0, out)
    return out.astype(np.uint8)


# ---------------------------------------------------------------------------
# E4M3
# ---------------------------------------------------------------------------


def _e4m3_value_from_bits(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        val = m * 2.0 ** -9  # subnormal: 2^(1-7) * m/8
    else:
        val = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -val if s else val


_E4M3_TABLE = np.array([_e4m3_value_from_bits(c) for c in range(256)], dtype=np.float64)
#: the 127 finite non-negative values, codes 0x00..0x7E, ascending
_E4M3_POS = _E4M3_TABLE[:127].copy()
# Rounding grid used for the encoder: the finite values plus the value the
# next bit pattern would have in an unbounded format (1.875 * 2^8 = 480).  A
# value that rounds to it overflows.
_E4M3_GRID = np.concatenate([_E4M3_POS, [1.875 * 2.0 ** 8]])
E4M3_MAX = 448.0


def e4m3_all_values() -> np.ndarray:
    """Decoded value of each of the 256 bit patterns (NaN for 0x7F, 0xFF)."""
    return _E4M3_TABLE.copy()


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 bit patterns -> float64 values."""
    return _E4M3_TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


def e4m3_encode(u):
    """Round non-negative values to E4M3, round-to-nearest, ties to even.

    Returns ``(codes, overflow)``: uint8 bit patterns and a bool mask that is
    True where the value rounds past 448 (``u > 464``); such codes are set to
    0x7F (the NaN pattern).
    """
    u = np.asarray(u, dtype=np.float64)
    if np.any(np.isnan(u)) or np.any(u < 0):
        raise ValueError("e4m3_encode expects non-negative, non-NaN input")
    g = _E4M3_GRID
    hi = np.searchsorted(g, u, side="left")
    hi_c = np.minimum(hi, len(g) - 1)
    lo_c = np.maximum(hi - 1, 0)
    with np.errstate(invalid="ignore"):
        d_lo = u - g[lo_c]
        d_hi = g[hi_c] - u
    pick_lo = d_lo < d_hi
    tie = d_lo == d_hi
    out = np.where(pick_lo | (tie & ((lo_c % 2) == 0)), lo_c, hi_c)
    out = np.where(hi == 0, 0, out)
    overflow = (out >= 127) | (hi >= len(g))
    out = np.where(overflow, 0x7F, out)
    return out.astype(np.uint8), overflow
