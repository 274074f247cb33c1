"""Pins for the oracle's E2M1 and E4M3 codecs (CPU only).

Each check compares the oracle with something other than itself: the value
set the pages print, torch's float8_e4m3fn cast (a library routine), a
brute-force nearest search in exact rational arithmetic, or the closed-form
threshold form of round-to-nearest-even on the E2M1 grid.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_brute(v: float) -> int:
    """Nearest of the 16 codes by exact distance to the decoded value, ties to
    the even code; negative codes only tie with positive ones at zero, where
    the positive (sign bit clear) code is taken."""
    best, best_d = None, None
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
        val = -mag if s else mag
        d = abs(Fraction(v) - val)
        if best is None or d < best_d or (d == best_d and (c % 2 == 0) and best % 2 == 1):
            best, best_d = c, d
    return best & 7


def test_e2m1_value_set_matches_page():
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        printed = sorted(float(x) for x in f.read().split("\n") if x and not x.startswith("#"))
    decoded = sorted(set(float(v) for v in codecs.e2m1_decode(np.arange(16))))
    assert sorted(set(printed)) == sorted(set(decoded))
    assert max(abs(v) for v in decoded) == 6.0
    assert list(codecs.E2M1_MAG_VALUES) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _e2m1_probe_values():
    f32 = np.float32
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    pts = list(codecs.E2M1_MAG_VALUES) + mids + [6.5, 7.0, 100.0, 1e30]
    out = []
    for p in pts:
        p32 = f32(p)
        out += [p32, np.nextafter(p32, f32(0)), np.nextafter(p32, f32(np.inf))]
    out += list(np.linspace(0, 8, 4001, dtype=np.float32))
    out += [f32(1e-45), f32(1e-38)]
    return np.array(out, dtype=np.float32)


def test_e2m1_round_matches_bruteforce():
    v = _e2m1_probe_values()
    got = codecs.e2m1_round_mag(v)
    want = np.array([_e2m1_brute(float(x)) for x in v], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e2m1_round_matches_threshold_closed_form():
    # RNE on the grid {0,.5,1,1.5,2,3,4,6} with saturation is, in closed form,
    # the count of crossed midpoints; a tie goes to the even code, so the
    # comparison is ">" at midpoints below an odd code and ">=" below an even one.
    v = _e2m1_probe_values().astype(np.float64)
    closed = ((v > 0.25).astype(int) + (v >= 0.75) + (v > 1.25) + (v >= 1.75)
              + (v > 2.5) + (v >= 3.5) + (v > 5.0))
    assert np.array_equal(codecs.e2m1_round_mag(v), closed.astype(np.uint8))


def test_e2m1_exact_roundtrip_and_saturation():
    for c, val in enumerate(codecs.E2M1_MAG_VALUES):
        assert codecs.e2m1_round_mag(np.array([val]))[0] == c
    assert codecs.e2m1_round_mag(np.array([np.inf]))[0] == 7
    assert codecs.e2m1_round_mag(np.array([6.0001]))[0] == 7


def test_e4m3_decode_matches_torch():
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = bits.view(torch.float8_e4m3fn).float().double().numpy()
    ours = codecs.e4m3_all_values()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.nanmax(ours) == 448.0


def _e4m3_probe_values():
    rng = np.random.default_rng(123)
    f32 = np.float32
    pos = codecs.e4m3_all_values()[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids, [456.0, 460.0, 464.0, 463.99, 464.01, 470.0, 479.0, 480.0, 500.0, 1e6]])
    out = []
    for p in pts:
        p32 = f32(p)
        out += [p32, np.nextafter(p32, f32(0)), np.nextafter(p32, f32(np.inf))]
    out += list((np.exp(rng.uniform(np.log(1e-6), np.log(470), 200000))).astype(np.float32))
    out += [f32(0), f32(1e-45), f32(2.0 ** -10), f32(2.0 ** -10 * 1.5)]
    return np.array(out, dtype=np.float32)


def test_e4m3_encode_matches_torch_cast():
    u = _e4m3_probe_values()
    codes, ovf = codecs.e4m3_encode(u)
    t = torch.from_numpy(u).to(torch.float8_e4m3fn)
    tnan = torch.isnan(t.float()).numpy()
    tbits = t.view(torch.uint8).numpy()
    assert np.array_equal(ovf, tnan)
    assert np.array_equal(codes[~ovf], tbits[~ovf])
    assert not ovf[u <= 464.0].any()
    assert ovf[u > 464.0].all()


def test_e4m3_roundtrip_and_ties():
    pos = codecs.e4m3_all_values()[:127]
    codes, ovf = codecs.e4m3_encode(pos)
    assert not ovf.any() and np.array_equal(codes, np.arange(127))
    # every midpoint between consecutive finite values goes to the even pattern
    mids = (pos[:-1] + pos[1:]) / 2
    mcodes, _ = codecs.e4m3_encode(mids)
    lo = np.arange(126)
    assert np.array_equal(mcodes, np.where(lo % 2 == 0, lo, lo + 1))


def test_e4m3_rejects_negative_and_nan():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([-1.0]))
    with pytest.raises(ValueError):
        codecs.e2m1_round_mag(np.array([np.nan]))
