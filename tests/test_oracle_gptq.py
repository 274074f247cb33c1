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
* the scales and mask are the FourOverSix pre-selection's, unchanged.
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
