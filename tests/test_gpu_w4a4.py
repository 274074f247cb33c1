"""GPU parity: activation quantization and the W4A4 product vs the CPU oracle.

Activation codes, scales, tensor scale, amax and the block-scaled bf16 values
must be bit-exact with oracle.quantize_act; the W4A4 GEMM must be within the
GEMM tolerance of the float64 W4A4 reference (relative Frobenius error
<= 2e-3 with bf16 output, <= 1e-5 with fp32 output).
"""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu


def _assert_act_same(a, r, what):
    assert np.array_equal(a.codes.cpu().numpy(), r.codes), what
    assert np.array_equal(a.scales.cpu().numpy(), r.scales), what
    assert a.tensor_scale.cpu().numpy()[0].view(np.uint32) == np.float32(r.tensor_scale).view(np.uint32), what
    assert a.amax.cpu().numpy()[0].view(np.uint32) == np.float32(r.amax).view(np.uint32), what
    xs = oracle.act_blockscaled(r)
    got = a.blockscaled.float().cpu().numpy()
    assert np.array_equal(got, xs) and np.array_equal(np.signbit(got), np.signbit(xs)), what


def _edge_acts():
    x = synth.activations(7, 256, 71).float()
    x[1] = 0.0  # an all-zero row
    x[2, 16:32] = 0.0  # a zero block
    x[3, 5] = 3.0e4  # an outlier that sets the tensor scale
    x[4, :16] = -1.0e-30  # tiny negatives: sigma 0, codes keep the sign
    x[5, 32:48] = torch.tensor([6.0, -4.0, 3.0, 2.0, 1.5, 1.0, 0.5, 0.0, -6.0, 5.0, 2.5, 0.25, 0.75, -1.25, 1.75, 3.5])
    return x.to(torch.bfloat16)


ACT_SHAPES = [(1, 16), (5, 64), (48, 4096), (300, 1040), (129, 14336)]


@pytest.mark.parametrize("m,k", ACT_SHAPES)
def test_quantize_act_bit_exact(m, k):
    print("act case", m, k, flush=True)
    x = synth.activations(m, k, 7000 + m)
    a = nv.quantize_act(x.cuda())
    torch.cuda.synchronize()
    _assert_act_same(a, oracle.quantize_act(x), f"{m}x{k}")


def test_quantize_act_edges_and_amax_in():
    x = _edge_acts()
    for amax in (None, 2688.0, 0.5):
        a = nv.quantize_act(x.cuda(), None if amax is None else torch.tensor([amax], device="cuda"))
        torch.cuda.synchronize()
        _assert_act_same(a, oracle.quantize_act(x, amax_in=amax), f"edges amax={amax}")
    z = torch.zeros((3, 32), dtype=torch.bfloat16)
    a = nv.quantize_act(z.cuda())
    torch.cuda.synchronize()
    _assert_act_same(a, oracle.quantize_act(z), "zeros")


def _rel(y, ref):
    return float(np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref))


# (m, n, k): both GEMM paths, ragged tiles, odd n, K not a multiple of 64
GEMM_SHAPES = [(1, 128, 256), (49, 256, 512), (64, 1001, 192), (130, 600, 4096), (300, 512, 1040),
               (1024, 4096, 4096)]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_w4a4_gemm_matches_reference(m, n, k):
    print("w4a4 case", m, n, k, flush=True)
    w = synth.student_t_weights(n, k, 800 + n)
    x = synth.activations(m, k, 8100 + m)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    r = oracle.quantize_fos(w)
    assert np.array_equal(q.codes.cpu().numpy(), r.codes)
    xd = x.cuda()
    ref = oracle.w4a4_gemm_ref(x, r.codes, r.scales, r.tensor_scale)
    y = nv.w4a4_gemm(xd, q).float().cpu().numpy()
    e = _rel(y, ref)
    y32 = nv.w4a4_gemm(xd, q, out_dtype=torch.float32).cpu().numpy()
    e32 = _rel(y32, ref)
    print(f"  rel err bf16 {e:.3e} fp32 {e32:.3e}")
    assert e <= 2e-3 and e32 <= 1e-5
    # the same product through the W4A16 entry point on the block-scaled
    # activations, scaled by the activation tensor scale
    a = nv.quantize_act(xd)
    y16 = nv.w4a16_gemm(a.blockscaled, q, out_dtype=torch.float32).cpu().numpy()
    y16 = y16.astype(np.float64) * float(a.tensor_scale.cpu()[0])
    assert _rel(y32, y16) <= 1e-6


def test_w4a4_full_size_sampled_rows():
    # the 4096 x 4096 layer at M = 4096; rows of the product depend on the
    # whole activation tensor only through its amax
    n = k = m = 4096
    w = synth.student_t_weights(n, k, 2)
    x = synth.activations(m, k, 8200)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    y = nv.w4a4_gemm(x.cuda(), q, out_dtype=torch.float32).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095], np.random.default_rng(3).choice(m, 11, replace=False)]))
    amax = float(x.float().abs().max())
    r = oracle.quantize_fos(w)
    ref = oracle.w4a4_gemm_ref(x[torch.from_numpy(rows)], r.codes, r.scales, r.tensor_scale, amax_in=amax)
    assert _rel(y[rows], ref) <= 1e-5


def test_w4a4_errors_and_empty():
    q = nv.quantize_fos(torch.zeros((32, 64), dtype=torch.float32, device="cuda"))
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    need = nv.w4a4_workspace_size(8, 32, 64)
    with pytest.raises(nv.NVFP4Error, match="WORKSPACE_TOO_SMALL"):
        nv.w4a4_gemm(x, q, workspace=torch.empty(need - 256, dtype=torch.uint8, device="cuda"))
    y = nv.w4a4_gemm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), q)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)
    y = nv.w4a4_gemm(x, q)
    torch.cuda.synchronize()
    assert float(y.float().abs().sum()) == 0.0
