"""Plain, slow, obviously-correct CPU oracle for NVFP4 FourOverSix quantization
and the W4A16 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding under ``bit_gemm_amd/``) may import, call or link anything in
this package.  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg use it.  It shares no code, tables or constants with the
HIP path.

Sources (web pages; cited by title and section only):

* [Notes07] "SOAR Weekly Champion Notes 07 | Vanilla Xiao Zhang: NVFP4
  Quantization Improvements and Speculative Decoding in Practice",
  sections "01 Background: Where standard NVFP4 quantization error comes from",
  "02 FourOverSix: Adaptively choosing between M=6 and M=4" and "03 How we
  integrated it" (FourOverSix scales fixed before GPTQ).
* [Recap] "SOAR 2026 Recap: From Compute Limits to the Open-Source Ecosystem",
  section "1. Quantization and GEMM dispatch".

The pages fix the E2M1 value set, the M=6 convention, the M=4 scale formula
and the strict MSE comparison.  The block size (16), the FP8 flavour (E4M3) and
the FP32 per-tensor scale are not on the pages; they come from the task's
problem statement.  Every step the pages leave open is a stated reading (see
the contract in ``oracle/fos.py``).

Modules
-------
codecs  E2M1 and E4M3 encode/decode written from the format definitions.
fos     FourOverSix quantizer: vectorized numpy path and a scalar pure-Python
        path (the two are cross-checked by the tests).
gemm    Dequantization and the float64 GEMM reference.
gptq    GPTQ column updates inside the FourOverSix scales (fixed first), the
        inverse-Hessian factor from calibration activations, and the
        explicit inverse-Hessian form used to pin it.
w4a4    Activation quantization to NVFP4 (standard M=6 block scale) and the
        float64 reference of the W4A4 product.
qat     Quantization-aware training of a linear layer: forward on the FP4
        weights, input gradient through the same weights, STE weight
        gradient.

Parity status: every function here is pinned by ``-m "not gpu"`` tests against
something other than itself (the pages' printed value set, torch's
float8_e4m3fn cast, brute force, exact rational arithmetic, closed forms,
hand-derived golden blocks).  The M=4 block share the pages report (40-43%,
measured with GPTQ on real weights) is context only: "parity unpinned".
"""

from .codecs import (  # noqa: F401
    E2M1_MAG_VALUES,
    e2m1_decode,
    e2m1_round_mag,
    e4m3_decode,
    e4m3_encode,
    e4m3_all_values,
)
from .fos import quantize_fos, quantize_fos_scalar, FosResult, block_sse  # noqa: F401
from .gemm import dequant, dequant_f64, gemm_ref  # noqa: F401
from .gptq import gptq_fos, gptq_fos_obs, hessian, hessian_factor  # noqa: F401
from .w4a4 import ActResult, act_blockscaled, quantize_act, w4a4_gemm_ref  # noqa: F401
from .qat import qat_forward, qat_input_grad, qat_weight_grad  # noqa: F401
