"""W4A4: activations quantized to NVFP4 on the fly, then the product of two
NVFP4 operands: the CPU oracle.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix ([Recap §1 Quantization and GEMM dispatch]): above about
48 tokens the GEMM switches from the W4A16 kernel to a W4A4 one whose
activations are NVFP4 as well, so that both operands feed an NVFP4 matrix
instruction.  Nothing else about the activation side is on the pages.

Contract (A1-A3), all [reading]; fl32 and C1-C9 as in ``oracle/fos.py``:

A1 The activations are the W4A16 path's input, bf16 [m, k] (k % 16 == 0);
   their values are taken exactly as fp32.
A2 They are quantized to the same NVFP4 format as the weights, with the
   standard block scale only: C1 (tensor scale from the activation tensor's
   own amax, or the caller's amax_in), C2 (sigma = sigma6, the block amax
   mapped to 6), C5, C6, C9.  No FourOverSix choice: the pages describe it for
   the offline weight quantization, and an online M=4 trial would double the
   activation pass.
A3 y[i, j] = sum_k xhat[i, k] * what[j, k], both operands dequantized as C7
   (exact in float64, so the reference is a float64 matmul); the GPU may
   accumulate in any order, within the GEMM tolerance.

The block-scaled activations xs = val * sigma (without the tensor scale; at
most 6 significant bits, so exact in bf16) are what a bf16 matrix unit can
multiply exactly; they are returned for the parity tests.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .codecs import E2M1_MAG_VALUES, e4m3_decode, e4m3_encode
from .fos import BLOCK, E4M3_MAX, _candidate, tensor_scale_from_amax
from .gemm import dequant_f64, _unpack

F32 = np.float32


@dataclass
class ActResult:
    codes: np.ndarray  # uint8 [m, k/2]
    scales: np.ndarray  # uint8 [m, k/16] (E4M3 bit patterns)
    tensor_scale: np.float32
    amax: np.float32


def _as_f32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        if x.dtype != torch.bfloat16:
            raise ValueError("activations must be bf16")
        return x.float().numpy()
    return np.ascontiguousarray(x, dtype=F32)


def quantize_act(x, amax_in=None) -> ActResult:
    """A1-A2: NVFP4 with the standard (M=6) block scale."""
    x = _as_f32(x)
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("x must be [m, k] with k % 16 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("x must be finite")
    m, k = x.shape
    amax = (F32(np.max(np.abs(x))) if x.size else F32(0.0)) if amax_in is None else F32(amax_in)
    s_t = tensor_scale_from_amax(amax)  # C1
    d6 = F32(6.0) * s_t
    xb = x.reshape(m, k // BLOCK, BLOCK)
    a_b = np.max(np.abs(xb), axis=-1) if x.size else np.zeros((m, 0), F32)
    u6 = np.minimum(a_b / d6, E4M3_MAX)  # C2
    c6, _ = e4m3_encode(u6)
    s6 = e4m3_decode(c6).astype(F32)
    mag, _ = _candidate(xb, s6, s_t)  # C5, C6
    code = (mag | (np.signbit(xb).astype(np.uint8) << 3)).reshape(m, k)  # C9
    codes = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return ActResult(codes, c6.astype(np.uint8), s_t, amax)


def act_blockscaled(res: ActResult) -> np.ndarray:
    """xs = sign * val * sigma as float32 (exact; bf16-representable)."""
    c = _unpack(res.codes)
    mag = E2M1_MAG_VALUES.astype(F32)[c & 7]
    sigma = np.repeat(e4m3_decode(res.scales).astype(F32), 16, axis=1)
    v = mag * sigma
    return np.where((c & 8) != 0, -v, v).astype(F32)


def w4a4_gemm_ref(x, codes, scales, s_t, amax_in=None) -> np.ndarray:
    """A3: y = xhat @ what^T in float64, xhat from quantize_act(x)."""
    a = quantize_act(x, amax_in)
    xhat = dequant_f64(a.codes, a.scales, a.tensor_scale)
    return xhat @ dequant_f64(codes, scales, s_t).T
