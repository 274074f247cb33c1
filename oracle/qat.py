"""NVFP4 quantization-aware training of a linear layer: the CPU oracle.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix ([Recap] "SOAR 2026 Recap: From Compute Limits to the
Open-Source Ecosystem", section "3. EAGLE-3 speculative decoding and hybrid
architecture adaptation", its "Draft training" part, the NVFP4 QAT item):
the forward pass runs the GEMM on the FP4 weights themselves (not a
simulated fake quantization), and the backward pass hands the gradient
straight through to the BF16 master weights (the straight-through
estimator, STE).

Contract (Q1-Q3), [reading] where the pages are silent:

Q1 Forward: W_hat = FourOverSix NVFP4 of the master weights W (C1-C9, this
   step's W), y = x @ W_hat^T, as the W4A16 GEMM (x bf16; W4A16 because the
   pages' inference path for the draft's decode token counts is W4A16).
Q2 Backward, input gradient: dx = dy @ W_hat (the GEMM's transpose on the
   same FP4 weights; dy bf16), exact in float64 here; the GPU may sum in any
   order within the GEMM tolerance.
Q3 Backward, weight gradient (STE: d W_hat / d W taken as the identity):
   dW = dy^T @ x, the plain linear layer's weight gradient; a plain bf16
   GEMM with no NVFP4 operand, left to the training framework.
"""

from __future__ import annotations

import numpy as np
import torch

from .gemm import dequant_f64


def _f64(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        return a.float().numpy().astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def qat_forward(x, codes, scales, s_t) -> np.ndarray:
    """Q1: y = x @ W_hat^T (float64)."""
    return _f64(x) @ dequant_f64(codes, scales, s_t).T


def qat_input_grad(dy, codes, scales, s_t) -> np.ndarray:
    """Q2: dx = dy @ W_hat (float64), dy [m, n], W_hat [n, k]."""
    return _f64(dy) @ dequant_f64(codes, scales, s_t)


def qat_weight_grad(dy, x) -> np.ndarray:
    """Q3 (STE): dW = dy^T @ x (float64), [n, k]."""
    return _f64(dy).T @ _f64(x)
