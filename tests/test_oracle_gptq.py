"""Pins of the GPTQ-within-FourOverSix oracle (oracle/gptq.py) against
things other than itself:

* with U = I (and with any diagonal Hessian) no error is pushed to other
  columns, so the codes are exactly the FourOverSix round-to-nearest codes of
  oracle.quantize_fos (an independent, separately pinned routine);
* the Cholesky form (U) and the explicit inverse-Hessian form (column
  elimination on H^-1), both in float64, give the same codes - this pins the
  indices and transposition of the U update against the textbook form;
* hessian_factor: U is upper triangular with a positive diagonal and
  U^T U = H^-1 for H = 2 X^T X + damping (closed form);
* the point of the method: the calibration loss ||X (W - W_hat)^T|| is
  lower than with round-to-nearest, on every seed tried;
* the scales and mask are the FourOverSix pre-selection's, unchanged;
* the fp32 column loop, re-evaluated step by step in exact rational
  arithmetic with one correctly rounded binary32 result per operation (the
  C10 order: product, then subtraction; no fused multiply-add), gives the
  same codes and the same updated weights bit for bit.
"""

import numpy as np
import pytest

import oracle
import synth


def _problem(seed, n=48, k=128, s=384):
    rng = np.random.default_rng(seed)
    w = synth.student_t_weights(n, k, 100 + seed)
    x = rng.standard_normal((s, k)) * (1.0 + rng.random(k))  # uneven channel scales
    return w, x


def _deq(res):
    return oracle.dequant(res.codes, res.scales, res.tensor_scale, "f32").astype(np.float64)


def test_identity_hessian_is_round_to_nearest():
    w, _ = _problem(1)
    rtn = oracle.quantize_fos(w)
    g = oracle.gptq_fos(w, np.eye(w.shape[1], dtype=np.float32))
    assert np.array_equal(g.codes, rtn.codes)
    assert np.array_equal(g.scales, rtn.scales) and np.array_equal(g.m4_mask, rtn.m4_mask)


def test_diagonal_hessian_is_round_to_nearest():
    w, _ = _problem(2)
    k = w.shape[1]
    d = np.random.default_rng(2).random(k) + 0.5
    u = np.diag(1.0 / np.sqrt(d)).astype(np.float32)  # H = diag(d): H^-1 = U^T U
    assert np.array_equal(oracle.gptq_fos(w, u).codes, oracle.quantize_fos(w).codes)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_cholesky_form_equals_inverse_hessian_form(seed):
    w, x = _problem(seed)
    k = w.shape[1]
    h = 2.0 * x.T @ x
    h += 0.01 * np.mean(np.diag(h)) * np.eye(k)
    hinv = np.linalg.inv(h)
    u64 = np.linalg.cholesky(hinv).T
    chol = oracle.gptq_fos(w, u64, dtype=np.float64).codes
    obs = oracle.gptq_fos_obs(w, hinv)
    assert np.array_equal(chol, obs)


def test_hessian_factor_closed_form():
    _, x = _problem(6)
    u = oracle.hessian_factor(x).astype(np.float64)
    k = u.shape[0]
    assert np.allclose(np.tril(u, -1), 0.0) and np.all(np.diag(u) > 0)
    h = 2.0 * x.T @ x
    h += 0.01 * np.mean(np.diag(h)) * np.eye(k)
    rel = np.linalg.norm(u.T @ u @ h - np.eye(k)) / np.sqrt(k)
    assert rel < 1e-3  # fp32 rounding of U


@pytest.mark.parametrize("seed", [7, 8, 9, 10])
def test_lowers_calibration_loss(seed):
    w, x = _problem(seed)
    u = oracle.hessian_factor(x)
    rtn = oracle.quantize_fos(w)
    g = oracle.gptq_fos(w, u)
    loss_rtn = np.linalg.norm(x @ (w - _deq(rtn)).T)
    loss_g = np.linalg.norm(x @ (w - _deq(g)).T)
    assert loss_g < loss_rtn
    assert np.array_equal(g.scales, rtn.scales) and np.array_equal(g.m4_mask, rtn.m4_mask)


def test_fp32_contract_close_to_float64():
    w, x = _problem(11)
    u = oracle.hessian_factor(x)
    a = oracle.gptq_fos(w, u).codes
    b = oracle.gptq_fos(w, u.astype(np.float64), dtype=np.float64).codes
    assert np.mean(a != b) < 0.01  # only near-ties of the rounding can differ


# ---------------------------------------------------------------------------
# Exact re-evaluation of C10's fp32 steps.  Every value is a Fraction; rnd32
# rounds an exact rational to the nearest binary32 value (ties to even,
# subnormals included), written from the format's definition, so nothing
# here shares numpy's float32 arithmetic with the oracle.
# ---------------------------------------------------------------------------
from fractions import Fraction as Q  # noqa: E402


def _rnd32(q):
    if q == 0:
        return Q(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+1) after the fix-up
    if Q(2) ** e > a:
        e -= 1
    elif Q(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)  # below 2^-126 the spacing stays 2^-149
    quantum = Q(2) ** (e - 23)
    t = a / quantum
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Q(1, 2) or (rem == Q(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    assert r < Q(2) ** 128, "overflow not expected in this case"
    return sign * r


def _e4m3_value(byte):
    e, m = (byte >> 3) & 0xF, byte & 0x7
    return Q(m, 8) * Q(2) ** -6 if e == 0 else (1 + Q(m, 8)) * Q(2) ** (e - 7)


_E2M1 = [Q(0), Q(1, 2), Q(1), Q(3, 2), Q(2), Q(3), Q(4), Q(6)]


def _e2m1_nearest(v):
    """Index of the E2M1 magnitude nearest to v >= 0, ties to the even index,
    6 above the range."""
    best = 0
    for i in range(1, 8):
        d, db = abs(v - _E2M1[i]), abs(v - _E2M1[best])
        if d < db or (d == db and i % 2 == 0):
            best = i
    return best


def _gptq_exact(w, u, scales, s_t):
    n, k = w.shape
    wq = [[Q(float(w[i, j])) for j in range(k)] for i in range(n)]
    uq = [[Q(float(u[a, b])) for b in range(k)] for a in range(k)]
    st = Q(float(s_t))
    flt_max = (2 - Q(2) ** -23) * Q(2) ** 127
    codes = np.zeros((n, k), dtype=np.uint8)
    for i in range(n):
        row = wq[i]
        for j in range(k):
            sigma = _e4m3_value(int(scales[i, j // 16]))
            r = Q(0) if sigma == 0 else min(_rnd32(1 / _rnd32(sigma * st)), flt_max)
            wj = row[j]
            mag = _e2m1_nearest(_rnd32(abs(wj) * r))
            # no input is -0, and an update that lands on zero gives +0 (round to
            # nearest), so a zero here is +0, as in the fp32 loop
            neg = wj < 0
            w_abs = _rnd32(_rnd32(_E2M1[mag] * sigma) * st)
            what = -w_abs if neg else w_abs
            e = _rnd32(_rnd32(wj - what) / uq[j][j])
            codes[i, j] = mag | (int(neg) << 3)
            for l in range(j + 1, k):
                row[l] = _rnd32(row[l] - _rnd32(e * uq[j][l]))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    upd = np.array([[float(v) for v in r] for r in wq], dtype=np.float32)
    return packed, upd


@pytest.mark.parametrize("seed", [11, 12])
def test_fp32_column_loop_matches_exact_rational_evaluation(seed):
    """C10 in exact arithmetic: 3 rows x 48 columns (three blocks), a dense
    upper-triangular U from a real calibration Hessian, so every element
    receives up to 47 trailing updates in order."""
    rng = np.random.default_rng(seed)
    n, k = 3, 48
    w = synth.student_t_weights(n, k, 200 + seed)
    x = rng.standard_normal((4 * k, k)) * (1.0 + rng.random(k))
    u = oracle.hessian_factor(x)
    res, upd = oracle.gptq_fos(w, u, return_updated=True)
    codes_q, upd_q = _gptq_exact(w, u, res.scales, res.tensor_scale)
    assert np.array_equal(upd.view(np.uint32), upd_q.view(np.uint32))
    assert np.array_equal(res.codes, codes_q)


def test_exact_evaluation_sees_a_fused_update():
    """The pin is sharp: the same loop with the product and subtraction
    fused (one rounding) changes some updated weight bits."""
    rng = np.random.default_rng(13)
    n, k = 2, 32
    w = synth.student_t_weights(n, k, 213)
    x = rng.standard_normal((4 * k, k)) * (1.0 + rng.random(k))
    u = oracle.hessian_factor(x)
    _, upd = oracle.gptq_fos(w, u, return_updated=True)
    # fused variant, evaluated exactly: w_l = rnd32(w_l - e u) (one rounding)
    res = oracle.quantize_fos(w)
    st = Q(float(res.tensor_scale))
    flt_max = (2 - Q(2) ** -23) * Q(2) ** 127
    differs = False
    for i in range(n):
        row = [Q(float(v)) for v in w[i]]
        for j in range(k):
            sigma = _e4m3_value(int(res.scales[i, j // 16]))
            r = Q(0) if sigma == 0 else min(_rnd32(1 / _rnd32(sigma * st)), flt_max)
            wj = row[j]
            mag = _e2m1_nearest(_rnd32(abs(wj) * r))
            w_abs = _rnd32(_rnd32(_E2M1[mag] * sigma) * st)
            e = _rnd32(_rnd32(wj - (-w_abs if wj < 0 else w_abs)) / Q(float(u[j, j])))
            for l in range(j + 1, k):
                row[l] = _rnd32(row[l] - e * Q(float(u[j, l])))
        differs |= any(np.float32(float(a)).view(np.uint32) != b.view(np.uint32) for a, b in zip(row, upd[i]))
    assert differs


def test_hessian_is_the_damped_gram_matrix_exactly():
    """oracle.hessian against its definition written out in exact rationals
    on small integers and halves (every float64 operation exact here):
    H_ij = 2 sum_s x_si x_sj, plus damp * mean_i(H_ii) on the diagonal."""
    x = np.array([[1, -2, 0.5], [3, 0, -1], [0.5, 1.5, 2], [-1, 1, 1], [2, -0.5, 0]], dtype=np.float64)
    damp = 0.25
    s, k = x.shape
    g = [[2 * sum(Q(float(x[t, i])) * Q(float(x[t, j])) for t in range(s)) for j in range(k)] for i in range(k)]
    lam = Q(1, 4) * sum(g[i][i] for i in range(k)) / k
    want = np.array([[float(g[i][j] + (lam if i == j else 0)) for j in range(k)] for i in range(k)])
    assert np.array_equal(oracle.hessian(x, damp), want)
    assert np.array_equal(oracle.hessian(x, 0.0), np.array([[float(g[i][j]) for j in range(k)] for i in range(k)]))
