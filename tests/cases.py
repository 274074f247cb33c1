"""Named test inputs shared by the CPU and GPU tests (no method arithmetic)."""

import os
from fractions import Fraction

import numpy as np

import synth

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_blocks():
    """The 1 x 112 tensor of tests/golden/fos_blocks.txt and its expectations."""
    blocks, expects = [], []
    with open(os.path.join(GOLDEN, "fos_blocks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            tag, rest = line.split(None, 1)
            if tag == "block":
                vals = [F32(float(Fraction(t))) if "/" in t else F32(float(t)) for t in rest.split()]
                assert len(vals) == 16
                blocks.append(vals)
            elif tag == "expect":
                kv = dict(p.split("=") for p in rest.split()[:2])
                bytes_ = [int(b, 16) for b in rest.split("bytes=")[1].split()]
                expects.append((int(kv["scale"], 16), int(kv["m4"]), bytes_))
    assert len(blocks) == len(expects)
    return np.array(blocks, dtype=F32).reshape(1, -1), expects


def all_sigma6_tensor():
    """Block 0 holds the tensor amax 2.625 (s_t = 2^-10); block i+1 has amax
    6 * e4m3_value(i) * s_t, so every non-negative E4M3 value is a sigma6."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    vals += [(8 + m) / 8 * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)][:127 - 8]
    w = np.zeros((1, 16 * 128), dtype=F32)
    w[0, 0] = F32(2688 * 2.0 ** -10)
    for i, s in enumerate(vals):
        w[0, 16 * (i + 1)] = F32(6 * s * 2.0 ** -10)
        w[0, 16 * (i + 1) + 1] = F32(-2.5 * s * 2.0 ** -10)  # an E2M1 midpoint under M=6
    return w


def midpoint_tensor(seed=3):
    """Blocks whose elements sit exactly on E2M1 grid points and midpoints (and
    one float32 ulp either side) for their own M=6 scale: s_t = 2^-10 and each
    block holds a 6*sigma element, so v = |w| / (sigma s_t) lands on the
    probe values up to the rounding of the reciprocal."""
    rng = np.random.default_rng(seed)
    probes = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6], dtype=np.float64)
    s_t = 2.0 ** -10
    rows = []
    sig = [1.0, 1.5, 2.0, 3.25, 0.125, 448.0 / 8, 7.0 / 512]
    for r in range(32):
        row = []
        for b in range(16):
            sigma = sig[(r + b) % len(sig)]
            vals = rng.choice(probes, size=16) * sigma * s_t
            vals[rng.integers(16)] = 6 * sigma * s_t
            vals = vals.astype(F32)
            nudge = rng.integers(-1, 2, size=16)
            vals = np.where(nudge > 0, np.nextafter(vals, F32(np.inf)), np.where(nudge < 0, np.nextafter(vals, F32(0)), vals))
            vals = np.where(rng.integers(0, 2, 16) == 1, -vals, vals)
            row.append(vals)
        rows.append(np.concatenate(row))
    w = np.array(rows, dtype=F32)
    w[0, 0:16] = 0.0
    w[0, 0] = F32(2688 * s_t)
    return w


QUANT_SHAPES = [(1, 16), (3, 48), (5, 80), (17, 272), (64, 4096), (33, 1040)]


def quant_inputs():
    """(name, w) pairs covering tails, edges and the pages' regime."""
    out = [("tiny", synth.tiny(0)[0]), ("edge", synth.edge_weights()), ("golden", golden_blocks()[0]),
           ("sigma6_sweep", all_sigma6_tensor()), ("midpoints", midpoint_tensor())]
    for i, (n, k) in enumerate(QUANT_SHAPES):
        out.append((f"student_t_{n}x{k}", synth.student_t_weights(n, k, seed=100 + i)))
    return out
