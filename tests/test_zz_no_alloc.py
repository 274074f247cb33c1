"""nvfp4_w4a16_gemm_noalloc (no workspace argument, split-K partials in the
library's fixed per-GPU scratch) through the C ABI, against the existing
nvfp4_w4a16_gemm with a caller workspace: two calls in a row, the second on
a smaller input, each bit-identical to the workspace entry point (the same
kernels) and within the GEMM bars of the float64 oracle; a plan larger than
the scratch is rejected without a launch."""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}


def _noalloc(x, q, out):
    m, k = x.shape
    n = q.codes.shape[0]
    code = nv.F32 if out.dtype == torch.float32 else nv.BF16
    return nv.lib().nvfp4_w4a16_gemm_noalloc(x.data_ptr(), q.codes.data_ptr(), q.scales.data_ptr(),
                                             q.tensor_scale.data_ptr(), out.data_ptr(), m, n, k, code,
                                             torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_workspace_entry_point():
    # (m, n, k, seed): both split K (the streaming kernel, then the reduction
    # reading the scratch): more than 256 row tiles, then k > 4096, where the
    # single-launch full-K kernel does not apply; the second is smaller
    cases = [(48, 14336, 4096, 2), (17, 1000, 4608, 3)]
    scratch = nv.lib().nvfp4_noalloc_scratch_bytes()
    for m, n, k, seed in cases:
        need = nv.workspace_size(m, n, k)
        assert 0 < need <= scratch, (m, n, k, need)
        print("noalloc", m, n, k, "split-K scratch bytes", need, flush=True)
        w = synth.student_t_weights(n, k, seed)
        q = nv.quantize_fos(torch.from_numpy(w).cuda())
        r = oracle.quantize_fos(w)
        x = synth.activations(m, k, synth.activation_seed(m))
        ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
        xd = x.cuda()
        for dt in (torch.bfloat16, torch.float32):
            y0 = torch.full((m, n), float("nan"), dtype=dt, device="cuda")
            assert _noalloc(xd, q, y0) == nv.NVFP4_OK, nv.lib().nvfp4_last_error()
            y1 = nv.w4a16_gemm(xd, q, out_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(y0, y1), (m, n, k, dt)
            yd = y0.double().cpu().numpy()
            err = np.linalg.norm(yd - ref) / np.linalg.norm(ref)
            assert err <= TOL[dt], (m, n, k, dt, err)


def test_noalloc_without_split_and_oversized_plan():
    n, k = 512, 4096
    w = synth.student_t_weights(n, k, 5)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    x = synth.activations(1, k, synth.activation_seed(1)).cuda()
    assert nv.workspace_size(1, n, k) == 0  # one token: the full-K kernel, no scratch
    y0 = torch.empty((1, n), dtype=torch.float32, device="cuda")
    assert _noalloc(x, q, y0) == nv.NVFP4_OK
    torch.cuda.synchronize()
    assert torch.equal(y0, nv.w4a16_gemm(x, q, out_dtype=torch.float32))
    # 64 tokens on a 14336 x 14336 matrix: 38.5 MB of partials > 32 MiB
    m, n, k = 64, 14336, 14336
    assert nv.workspace_size(m, n, k) > nv.lib().nvfp4_noalloc_scratch_bytes()
    big = nv.NVFP4Weight(codes=torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda"),
                         scales=torch.zeros((n, k // 16), dtype=torch.uint8, device="cuda"),
                         tensor_scale=torch.ones(1, dtype=torch.float32, device="cuda"),
                         amax=torch.ones(1, dtype=torch.float32, device="cuda"), m4_mask=None)
    xb = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
    yb = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
    assert _noalloc(xb, big, yb) == 4  # NVFP4_ERR_WORKSPACE_TOO_SMALL
    assert "no-allocation" in nv.lib().nvfp4_last_error().decode()
    torch.cuda.synchronize()
    assert bool((yb == 7.0).all())  # nothing was launched
