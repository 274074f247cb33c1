"""Pins of the W4A4 oracle (oracle/w4a4.py) against things other than itself:

* on every block where the FourOverSix quantizer keeps the M=6 scale, the
  activation quantizer's scale and codes are exactly the FourOverSix ones
  (oracle.quantize_fos, separately pinned);
* each block scale is the E4M3 value nearest to the block amax over 6 s_t
  (brute force over torch's float8_e4m3fn table), each code magnitude the
  E2M1 value nearest to |x| R (brute force over the printed value set);
* a hand-derived block (ties of every kind) and a small-amax block;
* one-hot activations reproduce the dequantized weight columns; the float64
  reference equals an exact rational triple loop on a tiny case;
* the block-scaled activations are bf16-representable and equal xhat / s_t.
"""

from fractions import Fraction

import numpy as np
import torch

import oracle
import synth
from oracle.w4a4 import act_blockscaled, quantize_act, w4a4_gemm_ref
from test_oracle_gemm import _decode_independent

F32 = np.float32
E2M1_PRINTED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the pages' value set


def _act(m, k, seed):
    return synth.activations(m, k, seed)


def test_matches_fourosix_where_m6_is_kept():
    x = _act(64, 512, 3)
    a = quantize_act(x)
    f = oracle.quantize_fos(x.float().numpy())
    assert a.tensor_scale == f.tensor_scale and a.amax == f.amax
    keep6 = f.m4_mask == 0
    assert keep6.mean() > 0.4
    assert np.array_equal(a.scales[keep6], f.scales[keep6])
    ac = a.codes.reshape(64, -1, 8)
    fc = f.codes.reshape(64, -1, 8)
    assert np.array_equal(ac[keep6], fc[keep6])


def test_scales_and_codes_are_nearest_by_brute_force():
    x = _act(16, 256, 5)
    xf = x.float().numpy()
    a = quantize_act(x)
    table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    fin = table[np.isfinite(table) & (table >= 0)]
    s_t = F32(a.tensor_scale)
    d6 = F32(6.0) * s_t
    sig = torch.from_numpy(a.scales).view(torch.float8_e4m3fn).float().numpy()
    xb = xf.reshape(16, -1, 16)
    u = np.minimum(np.max(np.abs(xb), axis=-1) / d6, F32(448.0)).astype(np.float64)
    dist = np.abs(u[..., None] - fin[None, None, :])
    best = dist.min(axis=-1)
    assert np.all(np.abs(u - sig) == best)
    # codes: nearest E2M1 value to |x| R, R = 1 / fl32(sigma s_t)
    c = np.zeros((16, 256), dtype=np.uint8)
    c[:, 0::2] = a.codes & 0xF
    c[:, 1::2] = a.codes >> 4
    R = (F32(1.0) / (sig.astype(F32) * s_t)).astype(F32)
    v = (np.abs(xb) * R[..., None]).astype(np.float64).reshape(16, 256)
    vals = np.array(E2M1_PRINTED)
    got = vals[c & 7]
    d = np.abs(v[..., None] - vals)
    assert np.all(np.abs(v - got) == d.min(axis=-1))
    assert np.array_equal((c >> 3).astype(bool), np.signbit(xf))


def test_hand_derived_blocks():
    # amax_in 2688 gives s_t = 1 and d6 = 6.  Block 0 has amax 6 (sigma 1,
    # R 1): exact grid values, and every kind of tie (5, 2.5, 0.25, 0.75,
    # 1.25, 1.75, 3.5 go to the even code).  Block 1 has amax 3: sigma 0.5,
    # R 2, so 3 -> 6 (code 7).
    b0 = [6, -4, 3, 2, 1.5, 1, 0.5, 0, -6, 5, 2.5, 0.25, 0.75, -1.25, 1.75, 3.5]
    b1 = [3] + [0] * 15
    x = torch.tensor([b0 + b1], dtype=torch.bfloat16)
    a = quantize_act(x, amax_in=2688.0)
    assert a.tensor_scale == F32(1.0)
    assert a.scales.tolist() == [[0x38, 0x30]]  # E4M3 1.0 and 0.5
    want = [0xE7, 0x45, 0x23, 0x01, 0x6F, 0x04, 0xA2, 0x64, 0x07, 0, 0, 0, 0, 0, 0, 0]
    assert a.codes.tolist() == [want]
    # a caller amax far below the true one: u6 = a / d6 > 448 clamps to 448
    # (E4M3 0x7E), and |x| R saturates at 6
    a = quantize_act(x, amax_in=2.688)
    assert a.scales.tolist() == [[0x7E, 0x7E]]
    assert a.codes[0, 0] == 0xF7 and a.codes[0, 8] == 0x07


def test_one_hot_rows_give_weight_columns():
    w = synth.student_t_weights(48, 128, 8)
    q = oracle.quantize_fos(w)
    cols = [0, 5, 17, 64, 127]
    x = torch.zeros((len(cols), 128), dtype=torch.bfloat16)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = w4a4_gemm_ref(x, q.codes, q.scales, q.tensor_scale)
    wd = oracle.dequant_f64(q.codes, q.scales, q.tensor_scale)
    s_t = float(F32(1.0) / F32(2688.0))
    for i, c in enumerate(cols):
        # the one-hot value quantizes to 6 * 448 * s_t = 1 + O(2^-24)
        np.testing.assert_allclose(y[i], wd[:, c] * (2688.0 * s_t), rtol=0, atol=0)


def test_reference_equals_exact_triple_loop():
    x = _act(3, 32, 11)
    w = synth.student_t_weights(4, 32, 12)
    q = oracle.quantize_fos(w)
    a = quantize_act(x)
    xe = _decode_independent(a.codes, a.scales, a.tensor_scale)
    we = _decode_independent(q.codes, q.scales, q.tensor_scale)
    y = w4a4_gemm_ref(x, q.codes, q.scales, q.tensor_scale)
    for i in range(3):
        for j in range(4):
            exact = sum((xe[i][t] * we[j][t] for t in range(32)), Fraction(0))
            assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**80)


def test_blockscaled_is_bf16_exact():
    x = _act(8, 256, 13)
    a = quantize_act(x)
    xs = act_blockscaled(a)
    assert np.array_equal(torch.from_numpy(xs).to(torch.bfloat16).float().numpy(), xs)
    xhat = oracle.dequant_f64(a.codes, a.scales, a.tensor_scale)
    np.testing.assert_array_equal(xs.astype(np.float64) * float(a.tensor_scale), xhat)
