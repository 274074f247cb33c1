"""Per-element error bounds for the W4A16 GEMM against the float64 oracle.

The relative Frobenius bar (2e-3 for bf16 output) is an average: at
hundreds of thousands of outputs a single wrong element can hide under the
bf16 rounding floor.  These bounds hold for every element.

With u = 2^-24 and T[m, n] = sum_k |x[m, k] * w_hat[n, k]| (float64):
* the products x * w_hat are exact in fp32 (bf16 x bf16), so an fp32
  accumulation of them in any order differs from the exact sum by far less
  than A = 4 sqrt(k) u T (a random-sign sum of k terms accumulates about
  sqrt(k) roundings of its partial sums, each below u T); measured on the
  host with the oracle on a 512 x 4096 layer at M = 48, removing one
  16-element block from one output breaks the bound at 99 % of random
  positions (96 % with bf16 output: the block's signed sum is sometimes
  tiny), while a real fp32 accumulation stays below 1 % of it;
* bf16 output adds one rounding of the fp32 result, at most 2^-8 of its
  magnitude: |y - ref| <= 2^-8 (|ref| + A) + A.
"""

import numpy as np
import torch

U32 = 2.0 ** -24


def assert_gemm_elementwise(y, x, w_hat, ref, out_dtype, what=""):
    """y: GPU result [m, n] (any dtype), x: bf16 [m, k] (CPU), w_hat: float64
    [n, k] (the oracle's exact dequantization), ref: float64 [m, n]."""
    y = y.double().cpu().numpy() if isinstance(y, torch.Tensor) else np.asarray(y, dtype=np.float64)
    xa = np.abs(np.asarray(x.float().numpy(), dtype=np.float64))
    t = xa @ np.abs(w_hat).T
    k = w_hat.shape[1]
    a = 4.0 * np.sqrt(max(k, 1)) * U32 * t
    bound = a if out_dtype == torch.float32 else 2.0 ** -8 * (np.abs(ref) + a) + a
    err = np.abs(y - ref)
    bad = err > bound
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs beyond the per-element bound; first at "
                             f"[{i}, {j}]: y={y[i, j]!r} ref={ref[i, j]!r} bound={bound[i, j]!r}")
    return float((err / np.maximum(bound, 1e-300)).max())
