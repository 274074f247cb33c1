"""GPU parity: the input-gradient GEMM of quantization-aware training,
dx = dy @ W_hat, against the float64 oracle (relative Frobenius error
<= 2e-3 with bf16 output, <= 1e-5 with fp32 output), and its adjoint
relation to the forward W4A16 GEMM on the same packed weights.
"""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu


def _rel(y, ref):
    return float(np.linalg.norm(np.asarray(y, dtype=np.float64) - ref) / np.linalg.norm(ref))


# (m, n, k): one tile, ragged tiles everywhere, n not a multiple of 8 (the
# unaligned dy rows), k not a multiple of 128, a long reduction.  n % 64 == 0
# and k % 128 == 0 take the kernel with transposing LDS reads ((1, 64, 128),
# (128, 256, 256), (64, 4096, 4096) split 16 ways, (257, 14336, 512), (200,
# 1024, 384) split 4 ways), the others the kernel with transposed stores
# ((64, 4100, 512): its reduction split 13 ways).
SHAPES = [(1, 64, 128), (17, 100, 48), (128, 256, 256), (300, 1001, 1040), (64, 4096, 4096),
          (257, 14336, 512), (200, 1024, 384), (64, 4100, 512)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_input_grad_matches_reference(m, n, k):
    print("dx case", m, n, k, flush=True)
    w = synth.student_t_weights(n, k, 700 + n)
    r = oracle.quantize_fos(w)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    assert np.array_equal(q.codes.cpu().numpy(), r.codes)
    dy = synth.activations(m, n, 7100 + m)
    ref = oracle.qat_input_grad(dy, r.codes, r.scales, r.tensor_scale)
    dyd = dy.cuda()
    e16 = _rel(nv.w4a16_gemm_dx(dyd, q).float().cpu().numpy(), ref)
    e32 = _rel(nv.w4a16_gemm_dx(dyd, q, out_dtype=torch.float32).cpu().numpy(), ref)
    print(f"  rel err bf16 {e16:.3e} fp32 {e32:.3e}")
    assert e16 <= 2e-3 and e32 <= 1e-5


def test_one_hot_upstream_gives_weight_rows_exactly():
    n, k = 96, 320
    w = synth.student_t_weights(n, k, 71)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    rows = [0, 1, 31, 32, 63, 95]
    dy = torch.zeros((len(rows), n), dtype=torch.bfloat16)
    for i, r in enumerate(rows):
        dy[i, r] = 1.0
    dx = nv.w4a16_gemm_dx(dy.cuda(), q, out_dtype=torch.float32).cpu().numpy()
    wd = nv.dequant(q, torch.float32).cpu().numpy()
    for i, r in enumerate(rows):
        assert np.array_equal(dx[i], wd[r]), r


def test_adjoint_of_the_forward_gemm():
    # <dy, x W^T> = <dy W, x>: the backward kernel is the forward kernel's
    # transpose on the same packed weights
    m, n, k = 200, 1024, 768
    w = synth.student_t_weights(n, k, 72)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    x = synth.activations(m, k, 73).cuda()
    dy = synth.activations(m, n, 74).cuda()
    y = nv.w4a16_gemm(x, q, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    dx = nv.w4a16_gemm_dx(dy, q, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    lhs = float((dy.float().cpu().numpy().astype(np.float64) * y).sum())
    rhs = float((dx * x.float().cpu().numpy().astype(np.float64)).sum())
    scale = float(np.abs(dy.float().cpu().numpy()).astype(np.float64).ravel() @ np.abs(y).ravel())
    assert abs(lhs - rhs) <= 1e-5 * scale


def test_full_size_sampled_rows_and_empty():
    n = k = m = 4096
    w = synth.student_t_weights(n, k, 2)
    r = oracle.quantize_fos(w)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    dy = synth.activations(m, n, 7300)
    dx = nv.w4a16_gemm_dx(dy.cuda(), q, out_dtype=torch.float32).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 127, 128, 4095], np.random.default_rng(4).choice(m, 12, replace=False)]))
    ref = oracle.qat_input_grad(dy[torch.from_numpy(rows)], r.codes, r.scales, r.tensor_scale)
    assert _rel(dx[rows], ref) <= 1e-5
    # no weight rows: the product is zero (k = 128 would otherwise select the
    # kernel with transposing reads, which needs at least one 64-row step)
    for k0 in (64, 128):
        q0 = nv.quantize_fos(torch.zeros((0, k0), dtype=torch.float32, device="cuda"))
        z = nv.w4a16_gemm_dx(torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda"), q0, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert z.shape == (5, k0) and float(z.abs().sum()) == 0.0
