"""GPU parity: GPTQ inside fixed FourOverSix scales vs the CPU oracle.

The column updates are fully specified in fp32 (each element gets its
updates in increasing column order, one product and one subtraction each),
so codes, scales, mask, tensor scale and amax must be bit-exact with
oracle.gptq_fos.  U comes from oracle.hessian_factor of seeded synthetic
calibration activations.
"""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu


def _run(w, u, amax=None):
    wd = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    ud = torch.from_numpy(np.ascontiguousarray(u, dtype=np.float32)).cuda()
    a = None if amax is None else torch.tensor([amax], dtype=torch.float32, device="cuda")
    q = nv.quantize_fos_gptq(wd, ud, amax=a)
    torch.cuda.synchronize()
    return q


def _assert_same(q, r, what):
    codes = q.codes.cpu().numpy()
    bad = np.argwhere(codes != r.codes)
    assert bad.size == 0, f"{what}: {len(bad)} of {codes.size} code bytes differ, first {bad[:5].tolist()}"
    assert np.array_equal(q.scales.cpu().numpy(), r.scales), what
    assert np.array_equal(q.m4_mask.cpu().numpy(), r.m4_mask), what
    assert q.tensor_scale.cpu().numpy()[0].view(np.uint32) == np.float32(r.tensor_scale).view(np.uint32), what
    assert q.amax.cpu().numpy()[0].view(np.uint32) == np.float32(r.amax).view(np.uint32), what


def _problem(n, k, seed, s=None):
    w = synth.student_t_weights(n, k, 500 + seed)
    x = synth.calibration_activations(s or 2 * k, k, 900 + seed)
    return w, oracle.hessian_factor(x)


# (n, k): one panel and no trailing update; rows that fill no workgroup;
# several panels with ragged row counts (not multiples of 64 or 256)
SHAPES = [(64, 64), (1, 128), (256, 512), (300, 1024), (520, 1024), (160, 2048), (1000, 256)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_gptq_bit_exact(n, k):
    print("gptq case", n, k, flush=True)
    w, u = _problem(n, k, n + k)
    q = _run(w, u)
    r = oracle.gptq_fos(w, u)
    _assert_same(q, r, f"{n}x{k}")
    # GPTQ really moved codes away from round-to-nearest
    if k > 64:
        assert not np.array_equal(r.codes, oracle.quantize_fos(w).codes)


def test_gptq_identity_is_round_to_nearest():
    w, _ = _problem(200, 256, 3)
    q = _run(w, np.eye(256, dtype=np.float32))
    rtn = nv.quantize_fos(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert torch.equal(q.codes, rtn.codes) and torch.equal(q.scales, rtn.scales)
    _assert_same(q, oracle.quantize_fos(w), "identity")


def test_gptq_zero_blocks_outliers_and_amax_in():
    # zero rows and zero blocks (sigma = 0: those elements get code 0 or 8
    # whatever the pushed error), a huge outlier, and a caller amax
    n, k = 130, 512
    w, u = _problem(n, k, 11)
    w[3] = 0.0
    w[7, 64:128] = 0.0
    w[9, 16:32] = 0.0
    w[20, 200] = 3.0
    for amax in (None, 4.0):
        q = _run(w, u, amax)
        _assert_same(q, oracle.gptq_fos(w, u, amax_in=amax), f"edge amax={amax}")


def test_gptq_lowers_calibration_loss():
    n, k = 128, 512
    w, _ = _problem(n, k, 21)
    x = synth.calibration_activations(4 * k, k, 77)
    u = oracle.hessian_factor(x)
    q = _run(w, u)
    rtn = nv.quantize_fos(torch.from_numpy(w).cuda())
    g = nv.dequant(q).cpu().numpy().astype(np.float64)
    r = nv.dequant(rtn).cpu().numpy().astype(np.float64)
    loss = lambda wh: float(np.linalg.norm(x @ (w.astype(np.float64) - wh).T))
    print("calibration loss gptq", loss(g), "rtn", loss(r))
    assert loss(g) < 0.97 * loss(r)


def test_gptq_empty_and_errors():
    u = torch.eye(64, dtype=torch.float32, device="cuda")
    q = nv.quantize_fos_gptq(torch.empty((0, 64), dtype=torch.float32, device="cuda"), u)
    torch.cuda.synchronize()
    assert q.codes.numel() == 0
    with pytest.raises(nv.NVFP4Error, match="UNSUPPORTED_SHAPE"):
        nv.quantize_fos_gptq(torch.zeros((4, 96), dtype=torch.float32, device="cuda"),
                             torch.eye(96, dtype=torch.float32, device="cuda"))
    w = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    small = torch.empty(nv.gptq_workspace_size(4, 64) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(nv.NVFP4Error, match="WORKSPACE_TOO_SMALL"):
        nv.quantize_fos_gptq(w, u, workspace=small)


def test_gptq_full_size_sampled_rows():
    # the measured 4096 x 4096 layer (weights as the benchmark draws them):
    # rows are independent given the tensor amax, so the oracle runs on a
    # sample of rows with amax_in = the whole tensor's amax
    n = k = 4096
    w = synth.student_t_weights(n, k, 2)
    x = synth.calibration_activations(2 * k, k, 4343)
    u = oracle.hessian_factor(x)
    del x
    q = _run(w, u)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 2047, 4095],
                                     np.random.default_rng(5).choice(n, 10, replace=False)]))
    print("full-size rows", rows.tolist(), flush=True)
    amax = float(np.abs(w).max())
    r = oracle.gptq_fos(w[rows], u, amax_in=amax)
    assert np.array_equal(q.codes.cpu().numpy()[rows], r.codes)
    assert np.array_equal(q.scales.cpu().numpy()[rows], r.scales)
    assert np.array_equal(q.m4_mask.cpu().numpy()[rows], r.m4_mask)
    assert q.tensor_scale.cpu().numpy()[0].view(np.uint32) == np.float32(r.tensor_scale).view(np.uint32)


def test_gptq_many_panels_any_triangular_factor():
    # 128 panels, rows that fill no panel workgroup.  Any upper-triangular U
    # with a positive diagonal is a valid factor (U^T U is then SPD); a
    # synthetic one avoids a 8192-channel Hessian inverse on the host.
    n, k = 12, 8192
    rng = np.random.default_rng(31)
    w = synth.student_t_weights(n, k, 32)
    u = np.triu(rng.standard_normal((k, k), dtype=np.float32) * np.float32(0.3 / np.sqrt(k)), 1)
    u[np.diag_indices(k)] = (1.0 + 0.5 * rng.random(k)).astype(np.float32)
    q = _run(w, u)
    r = oracle.gptq_fos(w, u)
    _assert_same(q, r, f"{n}x{k}")
    assert not np.array_equal(r.codes, oracle.quantize_fos(w).codes)


# ---------------------------------------------------------------------------
# nvfp4_gptq_hessian: H = 2 X^T X + damp * mean(diag) * I from bf16 X against
# oracle.hessian (float64) on the same bf16 values.  Products of bf16 values
# are exact in fp32, so the only error is fp32 summation over s samples:
# |dH_ij| <= (s + 4) 2^-24 (2 sum_t |x_ti x_tj|) off the diagonal, plus the
# rounding of the damping on it.
# ---------------------------------------------------------------------------
def _hessian_case(s, k, seed, damp=0.01):
    x = torch.from_numpy(synth.calibration_activations(s, k, seed)).to(torch.bfloat16)
    xv = x.float().numpy().astype(np.float64)
    ref = oracle.hessian(xv, damp)
    h = nv.gptq_hessian(x.cuda(), damp).cpu().numpy().astype(np.float64)
    a = 2.0 * (np.abs(xv).T @ np.abs(xv))
    u = 2.0 ** -24
    bound = (s + 4) * u * a
    bound[np.diag_indices(k)] += (s + 4) * u * damp * float(np.mean(np.diag(a))) + 2 * u * np.abs(np.diag(ref))
    err = np.abs(h - ref)
    assert np.all(err <= bound), (s, k, float(np.max(err / np.maximum(bound, 1e-300))))
    rel = np.linalg.norm(h - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= 1e-5, (s, k, rel)
    assert np.array_equal(h, h.T), "H is symmetric bit for bit"
    return x, h


@pytest.mark.parametrize("s,k", [(1, 16), (37, 48), (300, 130), (512, 256), (1000, 1100), (64, 4096)])
def test_hessian_matches_oracle(s, k):
    print("hessian", s, k, flush=True)
    _hessian_case(s, k, 1700 + s + k)


def test_hessian_full_size_and_deterministic():
    # the benchmark's calibration size for the 4096 x 4096 layer: s = 2k
    print("hessian 8192 x 4096", flush=True)
    x, h = _hessian_case(8192, 4096, 4242)
    h2 = nv.gptq_hessian(x.cuda(), 0.01).cpu().numpy()
    assert np.array_equal(h.astype(np.float32), h2)


def test_hessian_empty_and_errors():
    lib = nv.lib()
    h = torch.full((16, 16), 7.0, dtype=torch.float32, device="cuda")
    out = nv.gptq_hessian(torch.empty((0, 16), dtype=torch.bfloat16, device="cuda"), 0.01, out=h)
    torch.cuda.synchronize()
    assert bool((out == 0).all())  # s = 0: H = 0
    assert lib.nvfp4_gptq_hessian(None, 4, 0, 0.01, None, None, 0, None) == nv.NVFP4_OK  # k = 0: nothing
    x = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    assert lib.nvfp4_gptq_hessian(x.data_ptr(), 4, 16, -1.0, h.data_ptr(), None, 0, None) == 1
    assert "damp" in lib.nvfp4_last_error().decode()
    assert lib.nvfp4_gptq_hessian(x.data_ptr(), 4, 16, 0.01, h.data_ptr(), None, 0, None) == 4  # no workspace
    assert lib.nvfp4_gptq_hessian(x.data_ptr(), 4, 65537, 0.01, h.data_ptr(), None, 0, None) == 2


def test_gptq_from_library_hessian():
    """The library's H feeds GPTQ: U from it (float64 Cholesky route on the
    host, as oracle.hessian_factor does), then the GPU quantizer and the
    oracle on the same U agree bit for bit."""
    from scipy.linalg import lapack

    n, k, s = 96, 256, 512
    w = synth.student_t_weights(n, k, 1800)
    x = torch.from_numpy(synth.calibration_activations(s, k, 1801)).to(torch.bfloat16)
    h = nv.gptq_hessian(x.cuda(), 0.01).cpu().numpy().astype(np.float64)
    c, info = lapack.dpotrf(h, lower=True)
    assert info == 0
    hinv, info = lapack.dpotri(c, lower=True)
    assert info == 0
    hinv = np.tril(hinv) + np.tril(hinv, -1).T
    u = np.ascontiguousarray(np.linalg.cholesky(hinv).T).astype(np.float32)
    _assert_same(_run(w, u), oracle.gptq_fos(w, u), "library Hessian")
