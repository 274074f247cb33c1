"""Pins of the QAT oracle (oracle/qat.py) against things other than itself:

* the input gradient is the derivative of the forward pass: y is linear in
  x, so for every coordinate direction e_j the exact difference
  <dy, y(x + e_j) - y(x)> equals dx[:, j] (rational arithmetic);
* one-hot upstream gradients pick rows of W_hat (indices and orientation);
* an exact rational triple loop on a tiny case;
* STE: the weight gradient is the plain linear layer's, dy^T x, whatever the
  quantization (a closed form, checked by the same directional identity).
"""

from fractions import Fraction

import numpy as np
import torch

import oracle
import synth
from test_oracle_gemm import _decode_independent


def _layer(n, k, seed):
    w = synth.student_t_weights(n, k, seed)
    return oracle.quantize_fos(w)


def test_input_grad_is_the_forward_derivative():
    q = _layer(6, 32, 41)
    x = synth.activations(3, 32, 42)
    dy = synth.activations(3, 6, 43)
    dx = oracle.qat_input_grad(dy, q.codes, q.scales, q.tensor_scale)
    y0 = oracle.qat_forward(x, q.codes, q.scales, q.tensor_scale)
    dyf = dy.float().numpy().astype(np.float64)
    for i in range(3):
        for j in range(32):
            xp = x.clone()
            xp[i, j] = 0.0  # the step -x[i, j] is exact
            step = -float(x[i, j])
            y1 = oracle.qat_forward(xp, q.codes, q.scales, q.tensor_scale)
            d = sum(Fraction(float(dyf[i, c])) * (Fraction(float(y1[i, c])) - Fraction(float(y0[i, c])))
                    for c in range(6))
            scale = max(1.0, float(np.abs(dyf[i]).sum() * np.abs(y0[i]).max()))
            assert abs(float(d) - dx[i, j] * step) <= 1e-12 * scale


def test_one_hot_upstream_picks_weight_rows():
    q = _layer(48, 128, 44)
    rows = [0, 7, 31, 47]
    dy = torch.zeros((len(rows), 48), dtype=torch.bfloat16)
    for i, r in enumerate(rows):
        dy[i, r] = 1.0
    dx = oracle.qat_input_grad(dy, q.codes, q.scales, q.tensor_scale)
    wd = oracle.dequant_f64(q.codes, q.scales, q.tensor_scale)
    for i, r in enumerate(rows):
        assert np.array_equal(dx[i], wd[r])


def test_input_grad_equals_exact_triple_loop():
    q = _layer(5, 32, 45)
    dy = synth.activations(2, 5, 46)
    we = _decode_independent(q.codes, q.scales, q.tensor_scale)
    dx = oracle.qat_input_grad(dy, q.codes, q.scales, q.tensor_scale)
    d = dy.float().numpy()
    for i in range(2):
        for j in range(32):
            exact = sum((Fraction(float(d[i, r])) * we[r][j] for r in range(5)), Fraction(0))
            assert abs(Fraction(float(dx[i, j])) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**80)


def test_weight_grad_is_straight_through():
    x = synth.activations(4, 16, 47)
    dy = synth.activations(4, 3, 48)
    dw = oracle.qat_weight_grad(dy, x)
    xf, df = x.float().numpy().astype(np.float64), dy.float().numpy().astype(np.float64)
    # <dy, (W + e_rc) x^T> - <dy, W x^T> = sum_m dy[m, r] x[m, c], for every (r, c)
    for r in range(3):
        for c in range(16):
            assert dw[r, c] == sum(df[m, r] * xf[m, c] for m in range(4)) or \
                abs(dw[r, c] - sum(df[m, r] * xf[m, c] for m in range(4))) <= 1e-12
