"""GPTQ weight optimisation inside FourOverSix block scales: the CPU oracle.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix ([Notes07 §03 How we integrated it]): the block scale of
every block, and with it the M=6 / M=4 choice, is estimated and fixed first;
GPTQ's weight optimisation iterations then run inside those scales, so that
scale selection and the iterations do not interfere.  [Notes07 §01 Background]
names the route: GPTQ + NVFP4.

GPTQ itself is not on the pages.  It is the published method of Frantar,
Ashkboos, Hoefler and Alistarh, "GPTQ: Accurate Post-Training Quantization for
Generative Pre-trained Transformers" (2022), restated here from that
description: columns are quantized one after another, and each column's
rounding error, scaled by the inverse Hessian, is pushed onto the columns not
yet quantized; with U the upper Cholesky factor of the inverse Hessian
(H^-1 = U^T U) the push of column j onto column l > j is e_j * U[j, l] with
e_j = (w_j - what_j) / U[j, j].

Contract C10 [reading] (fl32 as in oracle/fos.py):
* inputs: W [n, k] fp32, U [k, k] fp32 (upper triangle read; it comes from
  calibration activations X: H = 2 X^T X plus damping, see hessian_factor);
  columns in natural order, no reordering.
* fixed first, from the original W: s_t, each block's sigma (the FourOverSix
  choice, C1-C9) and the mask; R_b = C5's reciprocal for the block's sigma.
* then for j = 0 .. k-1, all rows at once, with b = j // 16:
    mag_j  = E2M1_RNE(fl32(|w_j| * R_b))            (C5/C6, fixed sigma)
    what_j = sign(w_j) * fl32(fl32(val(mag_j) * sigma_b) * s_t)   (C7)
    e_j    = fl32(fl32(w_j - what_j) / U[j, j])
    w_l    = fl32(w_l - fl32(e_j * U[j, l]))  for every l > j
  so each element receives its updates in increasing j, one product and one
  subtraction each (no fused multiply-add).
* codes from mag_j and the sign of the updated w_j (C9); scales and mask are
  those of the first step.
"""

from __future__ import annotations

import numpy as np

from .codecs import E2M1_MAG_VALUES, e2m1_round_mag, e4m3_decode
from .fos import FLT_MAX, FosResult, quantize_fos

F32 = np.float32


def hessian(x, damp: float = 0.01) -> np.ndarray:
    """H = 2 X^T X + damp * mean(diag(2 X^T X)) * I in float64 (GPTQ's damped
    Hessian; the damping keeps H positive definite), x [s, k]."""
    x = np.asarray(x, dtype=np.float64)
    h = 2.0 * (x.T @ x)
    h[np.diag_indices_from(h)] += damp * float(np.mean(np.diag(h))) if h.size else 0.0
    return h


def hessian_factor(x, damp: float = 0.01) -> np.ndarray:
    """U (fp32, upper triangular) with H^-1 = U^T U, H = 2 X^T X + damp *
    mean(diag) * I, from calibration activations x [s, k], computed in float64
    (GPTQ's damped Hessian; the damping keeps H positive definite).  H^-1
    comes from H's own Cholesky factor (LAPACK potrf, then potri), the usual
    route for a symmetric positive definite inverse."""
    from scipy.linalg import lapack

    h = hessian(x, damp)
    c, info = lapack.dpotrf(h, lower=True)
    if info != 0:
        raise np.linalg.LinAlgError(f"H is not positive definite (potrf info {info})")
    hinv, info = lapack.dpotri(c, lower=True)  # lower triangle of H^-1
    if info != 0:
        raise np.linalg.LinAlgError(f"potri info {info}")
    hinv = np.tril(hinv) + np.tril(hinv, -1).T
    lower = np.linalg.cholesky(hinv)  # hinv = L L^T
    return np.ascontiguousarray(lower.T).astype(F32)  # U = L^T: hinv = U^T U


def _fixed_scales(pre: FosResult):
    sigma = e4m3_decode(pre.scales).astype(F32)  # [n, k/16]
    s = sigma * pre.tensor_scale
    with np.errstate(divide="ignore"):
        r = np.where(sigma == 0, F32(0.0), np.minimum(F32(1.0) / s, FLT_MAX)).astype(F32)
    return sigma, r


def gptq_fos(w, u, amax_in=None, dtype=np.float32, return_updated=False):
    """C10.  ``dtype=np.float64`` runs the column loop in float64 (for the
    cross-check against the explicit inverse-Hessian form; not the contract).
    ``return_updated=True`` also returns the weights after the loop (every
    column j holding w_j as it stood when it was quantized), for the pin
    that re-evaluates the fp32 steps in exact arithmetic."""
    w = np.ascontiguousarray(w, dtype=F32)
    n, k = w.shape
    u = np.asarray(u)
    if u.shape != (k, k):
        raise ValueError("u must be [k, k]")
    pre = quantize_fos(w, amax_in)
    sigma, r = _fixed_scales(pre)
    s_t = pre.tensor_scale
    vals = E2M1_MAG_VALUES.astype(F32)
    wk = w.astype(dtype)
    uk = u.astype(dtype)
    code = np.zeros((n, k), dtype=np.uint8)
    for j in range(k):
        b = j // 16
        wj = wk[:, j]
        v = (np.abs(wj) * r[:, b].astype(dtype)).astype(F32)  # C5 (fp32 in the contract)
        mag = e2m1_round_mag(v)
        w_abs = ((vals[mag] * sigma[:, b]) * s_t).astype(dtype)  # C7
        neg = np.signbit(wj)
        what = np.where(neg, -w_abs, w_abs)
        e = (wj - what) / uk[j, j]
        code[:, j] = mag | (neg.astype(np.uint8) << 3)
        if j + 1 < k:
            wk[:, j + 1:] = wk[:, j + 1:] - e[:, None] * uk[j, j + 1:][None, :]
    codes = code[:, 0::2] | (code[:, 1::2] << 4)
    res = FosResult(codes.astype(np.uint8), pre.scales, pre.m4_mask, s_t, pre.amax)
    return (res, wk) if return_updated else res


def gptq_fos_obs(w, hinv, amax_in=None) -> np.ndarray:
    """The same optimisation written with the explicit inverse Hessian, in
    float64 (the form the method is usually first stated in): after column
    j, its error e = (w_j - what_j) / Hinv[j, j] is pushed with row j of
    Hinv, and column j is eliminated from Hinv (Hinv -= Hinv[:, j] Hinv[j, :]
    / Hinv[j, j]).  Returns the packed codes; used only to pin gptq_fos."""
    w = np.ascontiguousarray(w, dtype=F32)
    n, k = w.shape
    pre = quantize_fos(w, amax_in)
    sigma, r = _fixed_scales(pre)
    s_t = pre.tensor_scale
    vals = E2M1_MAG_VALUES.astype(F32)
    wk = w.astype(np.float64)
    hi = np.array(hinv, dtype=np.float64, copy=True)
    code = np.zeros((n, k), dtype=np.uint8)
    for j in range(k):
        b = j // 16
        wj = wk[:, j]
        v = (np.abs(wj) * r[:, b].astype(np.float64)).astype(F32)
        mag = e2m1_round_mag(v)
        w_abs = ((vals[mag] * sigma[:, b]) * s_t).astype(np.float64)
        neg = np.signbit(wj)
        what = np.where(neg, -w_abs, w_abs)
        e = (wj - what) / hi[j, j]
        code[:, j] = mag | (neg.astype(np.uint8) << 3)
        wk[:, j + 1:] -= e[:, None] * hi[j, j + 1:][None, :]
        hi -= np.outer(hi[:, j], hi[j, :]) / hi[j, j]
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
