"""FourOverSix NVFP4 weight quantization: the CPU oracle.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix ([Notes07 §01 Background], [Notes07 §02 FourOverSix],
[Recap §1 Quantization and GEMM dispatch]):

* elements are E2M1 (value set {0, +-0.5, ..., +-4, +-6}), one FP8 scale per
  block, 0.5 byte per element;
* standard ("M=6") scaling maps each block's largest magnitude to 6;
* FourOverSix also tries an "M=4" scale, computed as the FP8 rounding of
  1.5 times the M=6 scale, quantizes the block with each scale, and keeps the
  M=4 scale only if its mean squared dequantization error is strictly smaller;
* the stored format is plain NVFP4: the choice itself is not stored.

Contract (C1-C9).  Readings of what the pages leave open are marked [reading].
fl32(.) is one IEEE-754 binary32 operation with round-to-nearest-even.

C1 [reading] amax_t = max |w| over the tensor (or the caller's amax_in).
   s_t = fl32(amax_t / 2688), 2688 = 6 * 448 (FP4 max times E4M3 max); if that
   is 0 (all-zero tensor or underflow), s_t = 1.
C2 [reading] d6 = fl32(6 * s_t).  Per 16-element block: a_b = max |w_i|,
   u6 = min(fl32(a_b / d6), 448), sigma6 = E4M3_RNE(u6).
C3 E4M3_RNE: nearest E4M3 value, ties to even mantissa; above 464 overflows.
C4 [page formula] t = 1.5 * sigma6 (exact in fp32), sigma4 = E4M3_RNE(t).
   [reading] if t overflows (sigma6 >= 320) M=4 is not a candidate, which is
   what the page's comparison does with the NaN of a non-saturating cast.
C5 [reading] per candidate sigma: R = 0 if sigma == 0, else
   R = min(fl32(1 / fl32(sigma * s_t)), FLT_MAX); v_i = fl32(|w_i| * R).
C6 [reading] mag_i = E2M1 round-to-nearest, ties to even code, saturating.
C7 [reading] what_i = sign(w_i) * fl32(fl32(val(mag_i) * sigma) * s_t)
   (the inner product is exact; this equals the fp32 dequantization).
C8 [page rule, reading for the order] e_i = fl32(w_i - what_i),
   q_i = fl32(e_i * e_i), SSE = contiguous balanced pairwise sum of q_0..q_15
   in fp32.  Comparing SSE is comparing the mean (division by 16 is exact).
   Choose M=4 iff M=4 is a candidate and SSE4 < SSE6 (a tie keeps M=6).
C9 [reading] code = (signbit(w) << 3) | mag (a negative value that rounds to
   zero keeps its sign); byte j of a row = code[2j] | code[2j+1] << 4; the
   scale byte is the E4M3 pattern of the chosen sigma; mask byte = 1 for M=4.

Layout: W is [n, k] row-major, blocks are 16 consecutive elements along k
(k % 16 == 0); codes [n, k/2], scales [n, k/16], mask [n, k/16], all uint8.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction
import math

import numpy as np

from .codecs import E2M1_MAG_VALUES, e2m1_round_mag, e4m3_decode, e4m3_encode

F32 = np.float32
BLOCK = 16
E4M3_MAX = F32(448.0)
TENSOR_DIV = F32(6.0 * 448.0)  # FP4 max (M=6) times E4M3 max
FLT_MAX = F32(np.finfo(np.float32).max)


@dataclass
class FosResult:
    codes: np.ndarray  # uint8 [n, k/2]
    scales: np.ndarray  # uint8 [n, k/16] (E4M3 bit patterns)
    m4_mask: np.ndarray  # uint8 [n, k/16] (1 = M=4 chosen)
    tensor_scale: np.float32
    amax: np.float32
    diag: dict = field(default_factory=dict)  # optional per-block diagnostics


def tensor_scale_from_amax(amax) -> np.float32:
    """C1: s_t = fl32(amax / 2688), or 1 when that is zero."""
    s = F32(amax) / TENSOR_DIV
    if s == F32(0.0):
        s = F32(1.0)
    return F32(s)


def _tree16(q: np.ndarray) -> np.ndarray:
    """C8: contiguous balanced pairwise fp32 sum over the last axis (16)."""
    p = q[..., 0::2] + q[..., 1::2]  # (q0+q1), (q2+q3), ...
    p = p[..., 0::2] + p[..., 1::2]
    p = p[..., 0::2] + p[..., 1::2]
    return p[..., 0] + p[..., 1]


def _candidate(wb: np.ndarray, sigma: np.ndarray, s_t: np.float32):
    """C5-C8 for one candidate scale per block.

    wb: float32 [..., 16]; sigma: float32 [...].  Returns (mag uint8 [..., 16],
    SSE float32 [...]).
    """
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        S = sigma * s_t
        R = F32(1.0) / S
        R = np.minimum(R, FLT_MAX)
        R = np.where(sigma == F32(0.0), F32(0.0), R).astype(F32)
        v = np.abs(wb) * R[..., None]
    mag = e2m1_round_mag(v)
    val = E2M1_MAG_VALUES.astype(F32)[mag]
    w_abs = (val * sigma[..., None]) * s_t
    w_hat = np.where(np.signbit(wb), -w_abs, w_abs)
    e = wb - w_hat
    q = e * e
    return mag, _tree16(q)


def quantize_fos(w, amax_in=None, diagnostics: bool = False, row_chunk: int = 512) -> FosResult:
    """FourOverSix quantization of a float32 [n, k] matrix (vectorized numpy).

    ``amax_in`` replaces the tensor amax when given (for example the max over
    all shards of a row-sharded tensor).
    """
    w = np.ascontiguousarray(w, dtype=F32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [n, k]")
    n, k = w.shape
    if k % BLOCK != 0:
        raise ValueError("k must be a multiple of 16")
    if not np.all(np.isfinite(w)):
        raise ValueError("w must be finite")
    if amax_in is None:
        amax = F32(np.max(np.abs(w))) if w.size else F32(0.0)
    else:
        amax = F32(amax_in)
        if not (np.isfinite(amax) and amax >= 0):
            raise ValueError("amax_in must be finite and >= 0")
    s_t = tensor_scale_from_amax(amax)
    d6 = F32(6.0) * s_t

    nb = k // BLOCK
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.zeros((n, nb), dtype=np.uint8)
    mask = np.zeros((n, nb), dtype=np.uint8)
    diag = {}
    if diagnostics:
        for key in ("sigma6", "sigma4", "sse6", "sse4"):
            diag[key] = np.zeros((n, nb), dtype=F32)
        diag["valid4"] = np.zeros((n, nb), dtype=bool)

    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        wb = w[r0:r1].reshape(r1 - r0, nb, BLOCK)
        a_b = np.max(np.abs(wb), axis=-1)
        u6 = np.minimum(a_b / d6, E4M3_MAX)  # C2
        c6, _ = e4m3_encode(u6)
        s6 = e4m3_decode(c6).astype(F32)
        t = F32(1.5) * s6  # C4 (exact)
        c4, ovf4 = e4m3_encode(t)
        valid4 = ~ovf4
        s4 = np.where(valid4, e4m3_decode(c4), 0.0).astype(F32)

        mag6, sse6 = _candidate(wb, s6, s_t)
        mag4, sse4 = _candidate(wb, s4, s_t)
        pick4 = valid4 & (sse4 < sse6)  # C8: strict, tie keeps M=6

        mag = np.where(pick4[..., None], mag4, mag6).astype(np.uint8)
        code = mag | (np.signbit(wb).astype(np.uint8) << 3)  # C9
        code = code.reshape(r1 - r0, k)
        codes[r0:r1] = code[:, 0::2] | (code[:, 1::2] << 4)
        scales[r0:r1] = np.where(pick4, c4, c6)
        mask[r0:r1] = pick4.astype(np.uint8)
        if diagnostics:
            diag["sigma6"][r0:r1] = s6
            diag["sigma4"][r0:r1] = s4
            diag["sse6"][r0:r1] = sse6
            diag["sse4"][r0:r1] = sse4
            diag["valid4"][r0:r1] = valid4
    return FosResult(codes, scales, mask, s_t, amax, diag)


# ---------------------------------------------------------------------------
# Scalar pure-Python path (small inputs only).  It follows the same contract
# with Python floats and exact rationals, and is cross-checked against the
# vectorized path by the tests.
# ---------------------------------------------------------------------------


def _fl32(x: float) -> float:
    """Round a Python float (binary64) to binary32.  For one +,-,*,/ of two
    binary32 operands, the binary64 result rounded again to binary32 is the
    correctly rounded binary32 result (53 >= 2*24 + 2)."""
    with np.errstate(over="ignore"):
        return float(np.float32(x))


def _scalar_e4m3_values():
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        v = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        vals.append(v)
    vals.append(Fraction(15, 8) * 256)  # the overflow slot (480)
    return vals


_SC_E4M3 = _scalar_e4m3_values()
_SC_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]


def _nearest_even(x: Fraction, grid) -> int:
    best, best_d = None, None
    for i, g in enumerate(grid):
        d = abs(x - g)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def _sc_e4m3(u: float):
    """-> (code, value) or (None, None) on overflow."""
    c = _nearest_even(Fraction(u), _SC_E4M3)
    if c == 127:
        return None, None
    return c, float(_SC_E4M3[c])


def _sc_e2m1(v: float) -> int:
    if math.isinf(v):
        return 7
    return _nearest_even(Fraction(v), _SC_E2M1)


def block_sse(block, sigma: float, s_t: float):
    """Scalar C5-C8 for one block and one candidate: (mags, what, SSE)."""
    flt_max = float(FLT_MAX)
    if sigma == 0.0:
        R = 0.0
    else:
        S = _fl32(sigma * s_t)
        R = flt_max if S == 0.0 else min(_fl32(1.0 / S), flt_max)
    mags, what, q = [], [], []
    for x in block:
        v = _fl32(abs(x) * R)
        mag = _sc_e2m1(v)
        w_abs = _fl32(_fl32(float(_SC_E2M1[mag]) * sigma) * s_t)
        wh = -w_abs if math.copysign(1.0, x) < 0 else w_abs
        e = _fl32(x - wh)
        mags.append(mag)
        what.append(wh)
        q.append(_fl32(e * e))
    lvl = q
    while len(lvl) > 1:
        lvl = [_fl32(lvl[i] + lvl[i + 1]) for i in range(0, len(lvl), 2)]
    return mags, what, lvl[0]


def quantize_fos_scalar(w, amax_in=None) -> FosResult:
    """Scalar pure-Python FourOverSix quantizer (use for small matrices)."""
    w = np.ascontiguousarray(w, dtype=F32)
    n, k = w.shape
    if k % BLOCK != 0:
        raise ValueError("k must be a multiple of 16")
    rows = [[float(x) for x in row] for row in w]
    amax = max((abs(x) for row in rows for x in row), default=0.0) if amax_in is None else float(F32(amax_in))
    s_t = _fl32(amax / 2688.0)
    if s_t == 0.0:
        s_t = 1.0
    d6 = _fl32(6.0 * s_t)
    nb = k // BLOCK
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.zeros((n, nb), dtype=np.uint8)
    mask = np.zeros((n, nb), dtype=np.uint8)
    for i, row in enumerate(rows):
        code_row = []
        for b in range(nb):
            blk = row[b * BLOCK:(b + 1) * BLOCK]
            a_b = max(abs(x) for x in blk)
            u6 = min(_fl32(a_b / d6), 448.0)
            c6, s6 = _sc_e4m3(u6)
            c4, s4 = _sc_e4m3(1.5 * s6)
            mags6, _, sse6 = block_sse(blk, s6, s_t)
            pick4 = False
            if c4 is not None:
                mags4, _, sse4 = block_sse(blk, s4, s_t)
                pick4 = sse4 < sse6
            mags = mags4 if pick4 else mags6
            for x, m in zip(blk, mags):
                code_row.append(m | (8 if math.copysign(1.0, x) < 0 else 0))
            scales[i, b] = c4 if pick4 else c6
            mask[i, b] = 1 if pick4 else 0
        for j in range(k // 2):
            codes[i, j] = code_row[2 * j] | (code_row[2 * j + 1] << 4)
    return FosResult(codes, scales, mask, F32(s_t), F32(amax))
