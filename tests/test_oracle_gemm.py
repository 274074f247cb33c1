"""Pins for the oracle's dequantization and float64 GEMM (CPU only)."""

from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import dequant, dequant_f64, gemm_ref, quantize_fos

F32 = np.float32


def _decode_independent(codes, scales, s_t):
    """Exact W_hat from the bit-level formats, using torch's fp8 decode for
    the scales and the E2M1 bit formula for the codes (Fractions)."""
    n, half = codes.shape
    sig = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).float().numpy()
    out = [[None] * (2 * half) for _ in range(n)]
    for i in range(n):
        for j in range(2 * half):
            byte = int(codes[i, j // 2])
            c = (byte >> 4) if j % 2 else (byte & 0xF)
            s, e, m = c >> 3, (c >> 1) & 3, c & 1
            mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
            v = mag * Fraction(float(sig[i, j // 16])) * Fraction(float(s_t))
            out[i][j] = -v if s else v
    return out


def test_dequant_f64_exact_and_f32_single_rounding():
    w = synth.student_t_weights(16, 128, seed=4)
    r = quantize_fos(w)
    exact = _decode_independent(r.codes, r.scales, r.tensor_scale)
    d64 = dequant_f64(r.codes, r.scales, r.tensor_scale)
    assert all(Fraction(float(d64[i, j])) == exact[i][j] for i in range(16) for j in range(128))
    d32 = dequant(r.codes, r.scales, r.tensor_scale, "f32")
    # one rounding of the exact value to float32 (nearest even), zeros signed
    want = np.array([[float(x) for x in row] for row in exact]).astype(F32)
    assert np.array_equal(np.abs(d32), np.abs(want))
    nz = want != 0
    assert np.array_equal(np.signbit(d32)[nz], np.signbit(want)[nz])
    bf = dequant(r.codes, r.scales, r.tensor_scale, "bf16")
    assert torch.equal(bf, torch.from_numpy(want).to(torch.bfloat16))


def test_gemm_ref_matches_naive_triple_loop():
    w = synth.normal_weights(5, 32, seed=8)
    r = quantize_fos(w)
    x = synth.activations(3, 32, seed=9)
    y = gemm_ref(x, r.codes, r.scales, r.tensor_scale)
    wh = _decode_independent(r.codes, r.scales, r.tensor_scale)
    xf = [[Fraction(float(v)) for v in row] for row in x.float().numpy()]
    for m in range(3):
        for n in range(5):
            acc = sum(xf[m][k] * wh[n][k] for k in range(32))
            assert abs(Fraction(float(y[m, n])) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_gemm_ref_one_hot_picks_columns_exactly():
    w = synth.student_t_weights(24, 64, seed=10)
    r = quantize_fos(w)
    wh = dequant_f64(r.codes, r.scales, r.tensor_scale)
    x = torch.zeros(64, 64, dtype=torch.bfloat16)
    x[torch.arange(64), torch.arange(64)] = 1.0
    y = gemm_ref(x, r.codes, r.scales, r.tensor_scale)
    assert np.array_equal(y, wh.T)
