"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

Holds no arithmetic of the method (no scaling, rounding to FP4/FP8, or GEMM):
only random draws, and rounding of activations to bfloat16 by torch's cast.

The pages measure on MiniCPM-SALA's real weights and unnamed evaluation tasks
([Notes07 §04 Measured results]); neither is available, so these decoder-shaped
synthetic layers stand in for them.

Weight recipe ("student_t"): float64 draws from a Student-t with 5 degrees of
freedom, scaled to population std 0.02 (divide by sqrt(5/3)); then
round(0.001 * n * k) distinct flat positions, drawn without replacement from
the same generator, are multiplied by 20 (outliers); cast to float32.
Weight recipe ("normal"): 0.02 * N(0, 1), float32.
Activations: N(0, 1) float64 draws rounded to bfloat16.

All weight matrices are [n, k] row-major with k the reduction dimension.  A
layer written "K x N" (e.g. up/gate 4096 x 14336) has k = K, n = N.
"""

from __future__ import annotations

import numpy as np
import torch

HIDDEN = 4096
MLP = 14336


def normal_weights(n: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, k)) * 0.02).astype(np.float32)


def student_t_weights(n: int, k: int, seed: int, rng=None) -> np.ndarray:
    rng = np.random.default_rng(seed) if rng is None else rng
    w = rng.standard_t(5.0, size=(n, k)) * (0.02 / np.sqrt(5.0 / 3.0))
    n_out = int(round(0.001 * n * k))
    if n_out:
        idx = rng.choice(n * k, size=n_out, replace=False)
        w.reshape(-1)[idx] *= 20.0
    return w.astype(np.float32)


def student_t_weights_device(n: int, k: int, seed: int, device) -> torch.Tensor:
    """fp32 [n, k] on `device`, drawn there from the same distribution as
    student_t_weights (Student-t, nu = 5, as z / sqrt(chi2_5 / 5) from six
    normal draws; std 0.02; round(0.001 n k) distinct positions x 20) with
    a torch generator seeded by `seed` -- not the same values as the numpy
    draw.  For whole-model timing runs, where drawing billions of values on
    the host would take minutes."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    chi2 = torch.zeros((n, k), device=device, dtype=torch.float32)
    for _ in range(5):
        chi2.addcmul_(e := torch.randn((n, k), generator=g, device=device, dtype=torch.float32), e)
    w = z.div_(chi2.div_(5.0).sqrt_()).mul_(0.02 / float(np.sqrt(5.0 / 3.0)))
    n_out = int(round(0.001 * n * k))
    if n_out:
        idx = torch.randperm(n * k, generator=g, device=device)[:n_out]
        w.view(-1)[idx] *= 20.0
    return w


def activations(m: int, k: int, seed: int) -> torch.Tensor:
    """bf16 [m, k] CPU tensor of N(0, 1) draws."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k))
    return torch.from_numpy(x).to(torch.bfloat16)


def calibration_activations(s: int, k: int, seed: int) -> np.ndarray:
    """float64 [s, k] calibration inputs: N(0, 1) draws with a per-channel
    scale drawn from U(1, 2), so the Hessian X^T X is far from diagonal in
    relative terms (uneven channel energies, random correlations)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((s, k))
    return x * (1.0 + rng.random(k))


def tiny(seed: int = 0):
    """256 x 256 weights ~ 0.02 N(0,1) and one activation row, one generator."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((1, 256))).to(torch.bfloat16)
    return w, x


# Workload table: name -> list of (layer name, n, k, weight seed) and the M
# values run on it.
SINGLE_LAYER = {"layers": [("w4096x4096", HIDDEN, HIDDEN, 2)], "m": [1, 8, 16, 32, 48]}
MLP_SET = {
    "layers": [("up", MLP, HIDDEN, 30), ("gate", MLP, HIDDEN, 31), ("down", HIDDEN, MLP, 32)],
    "m": [1, 4, 16, 48],
}
LARGE_M = {"layers": [("w4096x4096", HIDDEN, HIDDEN, 40), ("up", MLP, HIDDEN, 41)], "m": [64, 256, 1024, 4096]}


def decoder_layer_shapes():
    """Per-layer matrices of the 32-layer synthetic decoder: q, k, v, o are
    hidden x hidden (multi-head, equal widths: the attention shapes are not
    given), then gate, up (n = MLP width) and down (k = MLP width)."""
    return [("q", HIDDEN, HIDDEN), ("k", HIDDEN, HIDDEN), ("v", HIDDEN, HIDDEN), ("o", HIDDEN, HIDDEN),
            ("gate", MLP, HIDDEN), ("up", MLP, HIDDEN), ("down", HIDDEN, MLP)]


def decoder_weight_seed(layer: int, j: int) -> int:
    return 5000 + 8 * layer + j


def activation_seed(m: int) -> int:
    return 9000 + m


def edge_weights(seed: int = 7) -> np.ndarray:
    """A 64 x 256 matrix whose blocks exercise the rare cases: all-zero blocks,
    blocks far below the tensor amax (subnormal or zero scales), blocks whose
    amax is near the tensor amax (M=4 overflow), negative values that round to
    zero, and blocks holding exact midpoints of the FP4 grid."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[0, :] = 0.0  # all-zero row
    w[1, 0:16] = 0.0  # all-zero block
    w[2, :] *= np.float32(1e-6)  # tiny blocks -> subnormal / zero scales
    w[3, :] *= np.float32(1e-9)
    w[4, 0] = np.float32(1.0)  # tensor amax
    w[5, 0:16] = np.float32(0.9) * np.sign(rng.standard_normal(16)).astype(np.float32)
    w[6, 0:16] = np.float32(-1e-7)  # negative values that round to zero
    w[6, 15] = np.float32(0.3)
    # exact grid points / midpoints for a block whose amax maps to sigma 1 in
    # units of the tensor scale: values k/8 * a for small integers k
    grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6],
                    dtype=np.float32)
    w[7, 0:16] = grid * np.float32(1.0 / 6.0)
    w[8, 16:32] = -grid * np.float32(1.0 / 64.0)
    return w
