"""GPU parity beyond 2^31 elements (64-bit index arithmetic in every kernel).

The largest sizes the boundary accepts are bounded by 2^31 per dimension and
2^40 elements; these tests cross 2^31 elements in the weight matrix and in
the GEMM output.  Inputs are seeded and drawn on the GPU (host generation of
2 G values would take minutes); the oracle checks sampled rows, including
the rows on either side of element 2^31.
"""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu


def _rows_of_interest(n, k):
    r = (1 << 31) // k
    return sorted({0, 1, r - 1, r, min(r + 1, n - 1), n - 2, n - 1})


def test_quantize_gemm_dequant_beyond_2e31_elements():
    n, k = 32784, 65536  # 2.148e9 elements, 8.6 GB of fp32
    g = torch.Generator(device="cuda").manual_seed(31)
    w = torch.randn((n, k), generator=g, device="cuda", dtype=torch.float32) * 0.02
    q = nv.quantize_fos(w)
    amax = float(w.abs().max().item())
    torch.cuda.synchronize()
    assert float(q.amax.item()) == amax
    rows = _rows_of_interest(n, k)
    print("rows", rows, flush=True)
    wr = w[rows].cpu().numpy()
    r = oracle.quantize_fos(wr, amax_in=np.float32(amax))
    assert np.array_equal(q.codes[rows].cpu().numpy(), r.codes)
    assert np.array_equal(q.scales[rows].cpu().numpy(), r.scales)
    assert np.array_equal(q.m4_mask[rows].cpu().numpy(), r.m4_mask)
    # GEMM at one token (full-K kernel) and 48 tokens (pipelined split-K)
    for m in (1, 48):
        x = synth.activations(m, k, synth.activation_seed(m))
        y = nv.w4a16_gemm(x.cuda(), q, out_dtype=torch.float32)
        ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
        got = y[:, rows].double().cpu().numpy()
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-5, m
        del y
    # dequant: the last rows sit past element 2^31 of the output
    out = nv.dequant(q, torch.bfloat16)
    want = oracle.dequant(r.codes, r.scales, r.tensor_scale, "bf16")
    assert torch.equal(out[rows].cpu().view(torch.int16), want.view(torch.int16))


def test_tiled_gemm_output_beyond_2e31_elements():
    m, n, k = 65552, 32784, 128  # y has 2.149e9 elements
    g = torch.Generator(device="cuda").manual_seed(32)
    codes = torch.randint(0, 256, (n, k // 2), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    scales = torch.randint(0, 0x7F, (n, k // 16), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    s_t = torch.tensor([2.0 ** -9], dtype=torch.float32, device="cuda")
    q = nv.NVFP4Weight(codes, scales, s_t, s_t.clone(), None)
    x = (torch.randn((m, k), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    assert nv.gemm_path(m, n, k) == nv.PATH_TILED
    y = nv.w4a16_gemm(x, q, out_dtype=torch.float32)  # 8.6 GB; fp32 so that a small sample has a tight bound
    torch.cuda.synchronize()
    rows_m = sorted({0, (1 << 31) // n, (1 << 31) // n + 1, m - 1})
    cols = [0, 1, n // 2, n - 2, n - 1]
    ref = oracle.gemm_ref(x[rows_m].cpu(), codes[cols].cpu().numpy(), scales[cols].cpu().numpy(), np.float32(2.0 ** -9))
    got = y[rows_m][:, cols].double().cpu().numpy()
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) <= 1e-5
    # the output element past 2^31 was written by this call
    flat = (1 << 31) + 5
    mi, ni = flat // n, flat % n
    one = oracle.gemm_ref(x[mi:mi + 1].cpu(), codes[ni:ni + 1].cpu().numpy(), scales[ni:ni + 1].cpu().numpy(),
                          np.float32(2.0 ** -9))
    assert abs(float(y[mi, ni].item()) - float(one[0, 0])) <= 1e-4 * max(1.0, abs(float(one[0, 0])))


def test_activation_quantizer_beyond_2e31_elements():
    # bf16 activations of 2.148e9 elements (4.3 GB): codes, scales and the
    # block-scaled values on rows either side of element 2^31
    m, k = 32784, 65536
    g = torch.Generator(device="cuda").manual_seed(33)
    x = torch.randn((m, k), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    a = nv.quantize_act(x)
    amax = float(x.float().abs().max().item())
    torch.cuda.synchronize()
    assert float(a.amax.item()) == amax
    rows = _rows_of_interest(m, k)
    print("rows", rows, flush=True)
    r = oracle.quantize_act(x[rows].cpu(), amax_in=amax)
    assert np.array_equal(a.codes[rows].cpu().numpy(), r.codes)
    assert np.array_equal(a.scales[rows].cpu().numpy(), r.scales)
    assert np.array_equal(a.blockscaled[rows].float().cpu().numpy(), oracle.act_blockscaled(r))


def test_input_grad_output_beyond_2e31_elements():
    # dx = dy @ W_hat with 2.149e9 output elements (fp32, 8.6 GB)
    m, n, k = 65552, 128, 32784
    g = torch.Generator(device="cuda").manual_seed(34)
    codes = torch.randint(0, 256, (n, k // 2), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    scales = torch.randint(0, 0x7F, (n, k // 16), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    s_t = torch.tensor([2.0 ** -9], dtype=torch.float32, device="cuda")
    q = nv.NVFP4Weight(codes, scales, s_t, s_t.clone(), None)
    dy = (torch.randn((m, n), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    dx = nv.w4a16_gemm_dx(dy, q, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows_m = sorted({0, (1 << 31) // k, (1 << 31) // k + 1, m - 1})
    cols = [0, 1, k // 2, k - 2, k - 1]
    ref = oracle.qat_input_grad(dy[rows_m].cpu(), codes.cpu().numpy(), scales.cpu().numpy(), np.float32(2.0 ** -9))
    got = dx[rows_m][:, cols].double().cpu().numpy()
    assert np.linalg.norm(got - ref[:, cols]) / np.linalg.norm(ref[:, cols]) <= 1e-5
