"""Dequantization and the float64 W4A16 GEMM reference.

Test infrastructure only (see ``oracle/__init__.py``).

The pages' scheme keeps the standard NVFP4 format, so the GEMM reads codes and
block scales only and never the M=4/M=6 choice ([Notes07 §02 FourOverSix],
its list of benefits).  The W4A16 GEMM of [Recap §1 Quantization and GEMM
dispatch] multiplies 16-bit activations with the dequantized 4-bit weights.

Shapes: x [m, k] (bf16 values), weights [n, k] as codes [n, k/2] and scales
[n, k/16]; y[m, n] = sum_k x[m, k] * W_hat[n, k].

W_hat[n, k] = val(code) * sigma * s_t.  val * sigma has at most 6 significant
bits and s_t 24, so W_hat is exact in float64 and the reference is a plain
float64 matmul (numpy's) of exactly represented operands.
"""

from __future__ import annotations

import numpy as np
import torch

from .codecs import E2M1_MAG_VALUES, e4m3_decode

F32 = np.float32


def _unpack(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    n, half = codes.shape
    out = np.empty((n, 2 * half), dtype=np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def dequant(codes, scales, s_t, out: str = "f32") -> np.ndarray:
    """W_hat as float32 (C7: sign * fl32(fl32(val * sigma) * s_t)) or bf16.

    ``out='bf16'`` returns a torch.bfloat16 CPU tensor: the float32 value
    rounded to nearest-even bfloat16 by torch's cast.
    """
    c = _unpack(codes)
    mag = E2M1_MAG_VALUES.astype(F32)[c & 7]
    sigma = np.repeat(e4m3_decode(scales).astype(F32), 16, axis=1)
    w_abs = (mag * sigma) * F32(s_t)
    w = np.where((c & 8) != 0, -w_abs, w_abs).astype(F32)
    if out == "f32":
        return w
    if out == "bf16":
        return torch.from_numpy(w).to(torch.bfloat16)
    raise ValueError(out)


def dequant_f64(codes, scales, s_t) -> np.ndarray:
    """W_hat exactly, in float64."""
    c = _unpack(codes)
    mag = E2M1_MAG_VALUES[c & 7]
    sigma = np.repeat(e4m3_decode(scales), 16, axis=1)
    w = mag * sigma * float(F32(s_t))
    return np.where((c & 8) != 0, -w, w)


def gemm_ref(x, codes, scales, s_t) -> np.ndarray:
    """y = x @ W_hat^T in float64.  ``x`` holds bf16 values (torch bf16 tensor
    or a float array whose entries are bf16-representable)."""
    if isinstance(x, torch.Tensor):
        x = x.float().numpy()
    x64 = np.asarray(x, dtype=np.float64)
    return x64 @ dequant_f64(codes, scales, s_t).T
