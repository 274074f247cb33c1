"""GPU parity: W4A16 GEMM vs the float64 oracle.

Bar: relative Frobenius error <= 2e-3 for bf16 output (bf16 rounding of the
result alone is about 1.5e-3) and <= 1e-5 for fp32 output (fp32 accumulation
of exactly dequantized bf16 products); on the workload shapes also a bound
on every element (tests/gemm_bounds.py), so that one wrong output cannot
hide under the bf16 rounding floor.  One-hot activations with a
power-of-two tensor scale must reproduce W_hat exactly.
"""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth
from gemm_bounds import assert_gemm_elementwise

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}


def _rel(y, ref):
    y = y.double().cpu().numpy() if isinstance(y, torch.Tensor) else y
    den = np.linalg.norm(ref)
    return np.linalg.norm(y - ref) / (den if den > 0 else 1.0)


def _tol(dt, ref):
    """The Frobenius bar; for bf16 output never below 1.05x the error of the
    exact result rounded once to bf16 (on a small output, such as 6 x 17,
    that rounding alone can exceed 2e-3)."""
    if dt != torch.bfloat16:
        return TOL[dt]
    floor = _rel(torch.from_numpy(ref).float().bfloat16().double().numpy(), ref)
    return max(TOL[dt], 1.05 * floor)


def _quant(w):
    wd = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    q = nv.quantize_fos(wd)
    r = oracle.quantize_fos(w)
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), r.codes) and np.array_equal(q.scales.cpu().numpy(), r.scales)
    return q, r


def test_tiny_config():
    w, x = synth.tiny(0)
    q, r = _quant(w)
    ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
    for dt in (torch.bfloat16, torch.float32):
        y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt)
        assert _rel(y, ref) <= TOL[dt]


SHAPES = [
    # (m, n, k): tails in every dimension, K % 32 == 16, one K step, many splits
    (1, 64, 256), (3, 17, 48), (16, 100, 160), (17, 200, 4096), (33, 129, 528),
    (48, 512, 4096), (64, 130, 272), (5, 300, 14336), (2, 1, 16), (1, 4096, 4096),
    # m <= 2 (VALU dot products): more 16-row workgroups than CUs, K in one
    # round, with and without k % 128 == 0
    (2, 5000, 1040), (1, 4200, 4096),
]


@pytest.mark.parametrize("path", [nv.PATH_SKINNY, nv.PATH_TILED])
@pytest.mark.parametrize("impl", [nv.IMPL_PORTABLE, nv.IMPL_HWCVT])
def test_shapes_both_paths(path, impl):
    for i, (m, n, k) in enumerate(SHAPES):
        print("shape", m, n, k, "path", path, "impl", impl, flush=True)
        w = synth.student_t_weights(n, k, seed=200 + i)
        q, r = _quant(w)
        x = synth.activations(m, k, seed=300 + i)
        ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
        for dt in (torch.bfloat16, torch.float32):
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt, path=path, impl=impl)
            torch.cuda.synchronize()
            e = _rel(y, ref)
            assert e <= TOL[dt], (m, n, k, dt, e)


@pytest.mark.parametrize("split", [1, 2, 3, 7, 64])
def test_forced_split_k(split):
    m, n, k = 8, 256, 4096
    w = synth.student_t_weights(n, k, seed=400)
    q, r = _quant(w)
    x = synth.activations(m, k, seed=401)
    ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
    y = nv.w4a16_gemm(x.cuda(), q, out_dtype=torch.float32, path=nv.PATH_SKINNY, split_k=split)
    assert _rel(y, ref) <= 1e-5


# The pipelined split-K skinny kernel (k % 128 == 0): chunks of 4, 8 or 16
# K steps of 128 (automatic = 4; a forced split count selects it when it
# gives exactly one of those), 1 to 4 token tiles of 16, ragged n and m.
PIPE_CASES = [
    # (m, n, k, split_k): split 0 = automatic
    (17, 200, 2048, 0), (32, 64, 2048, 2), (40, 1000, 2048, 0), (49, 130, 2048, 2), (64, 200, 2048, 0),
    (20, 100, 2048, 1), (1, 300, 2048, 4), (7, 64, 2048, 2), (16, 333, 2048, 1), (64, 64, 512, 0),
    (33, 65, 1536, 3), (45, 190, 2048, 2), (48, 4000, 128, 0),
    # the streaming kernel (16 < m <= 64, k % 1024 == 0): ragged row groups
    # and tiles, one K chunk, several chunks, one to four token tiles (those
    # with at most 256 row tiles and k of 2048 to 4096 take the single-launch
    # full-K kernel instead)
    (33, 1001, 1024, 0), (48, 4000, 2048, 0), (64, 3000, 3072, 0), (40, 17, 1024, 0), (56, 5000, 4096, 0),
    (17, 1001, 1024, 0), (32, 4100, 2048, 0), (24, 300, 3072, 0),
    # 8 < m <= 16 on large matrices (more than 4096 rows): streaming kernel
    # with one token tile, K chunks of 1024 or 512; 4 < m <= 8 with k > 4096
    (9, 4097, 1024, 0), (16, 4200, 2048, 0), (12, 4100, 1536, 0), (8, 4200, 5120, 0),
    # 4 < m < 8 there (token rows >= m repeat row m - 1 in LDS), and the
    # decoder's down projection shape, which takes this route from m = 5
    (5, 4100, 5120, 0), (7, 4096, 14336, 0),
    # K chunks of 512 (k % 1024 == 512), two to four token tiles
    (24, 300, 1536, 0), (48, 1000, 2560, 0), (64, 700, 512, 0),
    # k % 512 != 0: the unpipelined split-K kernel
    (24, 300, 1152, 0), (40, 130, 640, 0),
]


@pytest.mark.parametrize("impl", [nv.IMPL_PORTABLE, nv.IMPL_HWCVT])
def test_pipe_kernel_configs(impl):
    for i, (m, n, k, split) in enumerate(PIPE_CASES):
        print("pipe case", m, n, k, split, "impl", impl, flush=True)
        w = synth.student_t_weights(n, k, seed=800 + i)
        q, r = _quant(w)
        x = synth.activations(m, k, seed=900 + i)
        ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
        for dt in (torch.bfloat16, torch.float32):
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt, path=nv.PATH_SKINNY, split_k=split, impl=impl)
            torch.cuda.synchronize()
            e = _rel(y, ref)
            assert e <= TOL[dt], (m, n, k, split, dt, e)


# The two full-K kernels that need no workspace.  Persistent kernel (4 < m
# <= 16, k % 512 == 0, k <= 4096): a workgroup per CU walks 16-row tiles,
# 8 or 16 token rows in LDS, one to eight 512-wide K slices, fewer tiles
# than CUs, a few tiles per CU, ragged n.  Single-launch kernel (16 < m <=
# 64, at most 256 workgroups of 1 to 4 row tiles): 2 to 4 token tiles, 4
# to 8 waves of 4 or 8 K steps of 128, ragged n and m.
FULL_K_CASES = [
    (5, 4096, 4096), (8, 14336, 4096), (9, 1001, 512), (16, 14336, 4096), (12, 20000, 2048), (7, 300, 1536),
    (6, 17, 3584),
    (17, 4096, 4096), (48, 4000, 4096), (64, 1001, 2048), (33, 4096, 2048), (20, 333, 3584), (40, 100, 2560),
    (32, 4096, 3072), (49, 64, 2048),
    # two to four row tiles per workgroup (more than 256 tiles), ragged n
    (17, 8192, 4096), (48, 12000, 4096), (33, 14336, 2048), (25, 7777, 2048),
    # one or two tokens on more than 1024 row tiles: four waves of two rounds
    # (one token: the row-per-wave kernel with the hardware decode)
    (1, 16400, 4096), (2, 16416, 4096), (1, 20000, 3584),
    # one token, row-per-wave kernel (k = 2048 c): ragged n with one
    # 2048-wide chunk, 3 and 8 chunks, n not a multiple of the 8 rows of a
    # workgroup
    (1, 4100, 2048), (1, 4096, 6144), (1, 2000, 16384), (1, 1003, 4096),
    # from 3 chunks one row per wave with the activations copied by LDS DMA:
    # every chunk count 4 .. 7, n not a multiple of the 4 rows of a
    # workgroup, a single row
    (1, 4097, 8192), (1, 1003, 10240), (1, 1, 12288), (1, 4101, 14336),
    # k % 2048 != 0 (k % 256 == 0): a partial last chunk (lanes past k / 32
    # of it hold no codes); one row per wave, and two rows per wave with two
    # chunks on more than 8192 rows; k from 2816 to 14592 (below 2048 the
    # full-K kernel: 1280, 256, 768)
    (1, 3584, 3584), (1, 4101, 11008), (1, 1003, 2816), (1, 13, 1280), (1, 64, 256), (1, 600, 14592),
    (1, 8200, 3840), (1, 9000, 768),
    # rows of 9 to 16 chunks (k up to 32768), whole and partial
    (1, 77, 18944), (1, 129, 22016), (1, 1030, 28672), (1, 300, 32768),
    # k % 256 != 0 (k % 32 == 0): 14 and 1 lanes with codes in the last chunk
    # (k = 1056 and 32: the full-K kernel)
    (1, 333, 4544), (1, 100, 2080), (1, 8500, 1056), (1, 70, 32), (1, 9000, 2080),
    # one token past the row-per-wave kernel's range (k > 32768, k % 32 != 0): the full-K kernel
    (1, 64, 32800), (1, 64, 48),
    # full-K kernel with its waves trimmed to the rounds (at most 256 row
    # tiles): 7 waves x 4 rounds, 6 x 2, 5 x 2, 7 x 3
    (2, 1000, 13824), (3, 4096, 6144), (4, 300, 5120), (2, 4000, 9728),
]


@pytest.mark.parametrize("impl", [nv.IMPL_PORTABLE, nv.IMPL_HWCVT])
def test_full_k_kernel_configs(impl):
    lib = nv.lib()
    for i, (m, n, k) in enumerate(FULL_K_CASES):
        print("full-K case", m, n, k, "impl", impl, flush=True)
        assert lib.nvfp4_w4a16_gemm_path(m, n, k) == nv.PATH_SKINNY
        assert lib.nvfp4_w4a16_gemm_workspace_size(m, n, k) == 0, (m, n, k)
        w = synth.student_t_weights(n, k, seed=1500 + i)
        q, r = _quant(w)
        x = synth.activations(m, k, seed=1600 + i)
        w_hat = oracle.dequant_f64(r.codes, r.scales, r.tensor_scale)
        ref = np.asarray(x.float().numpy(), dtype=np.float64) @ w_hat.T
        for dt in (torch.bfloat16, torch.float32):
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt, impl=impl)
            torch.cuda.synchronize()
            yd = y.double().cpu().numpy()
            e = _rel(yd, ref)
            assert e <= _tol(dt, ref), (m, n, k, dt, e)
            assert_gemm_elementwise(yd, x, w_hat, ref, dt, f"full-K m={m} n={n} k={k} {dt}")


@pytest.mark.parametrize("path", [nv.PATH_SKINNY, nv.PATH_TILED])
def test_one_hot_exact(path):
    """x = e_k with s_t a power of two: y[:, n] = W_hat[n, k] exactly."""
    n, k = 96, 256
    w = synth.student_t_weights(n, k, seed=500)
    w[0, 0] = np.float32(2688 * 2.0 ** -8)  # tensor amax -> s_t = 2^-8
    q, r = _quant(w)
    assert r.tensor_scale == np.float32(2.0 ** -8)
    wh = oracle.dequant_f64(r.codes, r.scales, r.tensor_scale)
    for k0 in range(0, k, 64):
        x = torch.zeros(min(48, k - k0), k, dtype=torch.bfloat16)
        x[torch.arange(x.shape[0]), k0 + torch.arange(x.shape[0])] = 1.0
        y = nv.w4a16_gemm(x.cuda(), q, out_dtype=torch.float32, path=path).double().cpu().numpy()
        assert np.array_equal(y, wh[:, k0:k0 + x.shape[0]].T)


def test_empty_and_zero_k():
    q = nv.quantize_fos(torch.zeros((32, 64), dtype=torch.float32, device="cuda"))
    y = nv.w4a16_gemm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), q)
    assert y.shape == (0, 32)
    q0 = nv.quantize_fos(torch.zeros((32, 0), dtype=torch.float32, device="cuda"))
    for path in (nv.PATH_SKINNY, nv.PATH_TILED):
        y = nv.w4a16_gemm(torch.zeros((4, 0), dtype=torch.bfloat16, device="cuda"), q0,
                          out_dtype=torch.float32, path=path)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y).item() == 0


def test_deterministic():
    w = synth.student_t_weights(4096, 4096, 2)
    q, r = _quant(w)
    for m in (1, 48, 256):
        x = synth.activations(m, 4096, seed=synth.activation_seed(m)).cuda()
        a = nv.w4a16_gemm(x, q, out_dtype=torch.float32)
        b = nv.w4a16_gemm(x, q, out_dtype=torch.float32)
        assert torch.equal(a, b)


def test_single_layer_config_all_m():
    """4096 x 4096 Student-t layer, M in {1, 8, 16, 32, 48}, default dispatch
    (the launch configuration the bench times)."""
    (name, n, k, seed), = synth.SINGLE_LAYER["layers"]
    w = synth.student_t_weights(n, k, seed)
    q, r = _quant(w)
    for m in synth.SINGLE_LAYER["m"]:
        x = synth.activations(m, k, synth.activation_seed(m))
        ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
        for dt in (torch.bfloat16, torch.float32):
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt)
            e = _rel(y, ref)
            print(f"{name} m={m} {dt}: rel err {e:.3e}")
            assert e <= TOL[dt]


@pytest.mark.parametrize("layer", synth.MLP_SET["layers"], ids=lambda l: l[0])
def test_mlp_config(layer):
    """The MLP set at its seeds and token counts, default dispatch, bf16 and
    fp32 output: Frobenius bars and the per-element bound."""
    name, n, k, seed = layer
    w = synth.student_t_weights(n, k, seed)
    q, r = _quant(w)
    wh = oracle.dequant_f64(r.codes, r.scales, r.tensor_scale)
    for m in synth.MLP_SET["m"]:
        x = synth.activations(m, k, synth.activation_seed(m))
        ref = np.asarray(x.float().numpy(), dtype=np.float64) @ wh.T
        for dt in (torch.bfloat16, torch.float32):
            print("mlp", name, m, dt, flush=True)
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt)
            torch.cuda.synchronize()
            e = _rel(y, ref)
            assert e <= TOL[dt], (name, m, dt, e)
            assert_gemm_elementwise(y, x, wh, ref, dt, f"{name} m={m} {dt}")


@pytest.mark.parametrize("layer", synth.LARGE_M["layers"], ids=lambda l: l[0])
def test_large_m_config_sampled_rows(layer):
    """Large-M prefill shapes: every output row is computed on the GPU; the
    oracle checks a sample of 64 rows (and all columns) per M."""
    name, n, k, seed = layer
    w = synth.student_t_weights(n, k, seed)
    q, r = _quant(w)
    wh = oracle.dequant_f64(r.codes, r.scales, r.tensor_scale)
    rng = np.random.default_rng(7)
    for m in synth.LARGE_M["m"]:
        x = synth.activations(m, k, synth.activation_seed(m))
        rows = np.sort(rng.choice(m, size=min(64, m), replace=False))
        ref = x[rows].double().numpy() @ wh.T
        for dt in (torch.bfloat16, torch.float32):
            print("large m", name, m, dt, flush=True)
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt).double().cpu().numpy()
            assert _rel(y[rows], ref) <= TOL[dt], (name, m, dt)
            assert_gemm_elementwise(y[rows], x[rows], wh, ref, dt, f"{name} m={m} {dt}")
            assert np.isfinite(y).all()


# Tiled kernel configurations for K a multiple of 64: M > 128 the kernel
# with the weights in registers (256 x 128 tiles; an odd number of K steps,
# a single one, K split over workgroups); 64 < M <= 128: 128 x 128 tiles;
# one 64-token tile with 256 (or, for K >= 8192, 128) weight rows for
# M <= 64; ragged M and N, odd N (scalar stores).
LM_SHAPES = [(1000, 8000, 192), (300, 700, 256), (257, 4100, 64), (130, 1001, 128), (5, 333, 128),
             (40, 300, 8192), (33, 520, 1024), (64, 1000, 512), (100, 1001, 192), (128, 600, 4096),
             (200, 260, 4096)]


@pytest.mark.parametrize("impl", [nv.IMPL_PORTABLE, nv.IMPL_HWCVT])
def test_large_m_kernel_configs(impl):
    for i, (m, n, k) in enumerate(LM_SHAPES):
        print("shape", m, n, k, "impl", impl, flush=True)
        w = synth.student_t_weights(n, k, seed=800 + i)
        q, r = _quant(w)
        x = synth.activations(m, k, seed=900 + i)
        ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
        for dt in (torch.bfloat16, torch.float32):
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt, path=nv.PATH_TILED, impl=impl)
            torch.cuda.synchronize()
            e = _rel(y, ref)
            assert e <= TOL[dt], (m, n, k, dt, e)


@pytest.mark.parametrize("split", [0, 1, 2, 3, 7, 16])
@pytest.mark.parametrize("k", [1024, 960])
def test_tiled_split_k(split, k):
    """K split over workgroups on the tiled path (fp32 partials + in-order
    reduction); 0 = the automatic plan.  k = 1024 runs the large-M kernel
    with 128 k per barrier (splits rounded to whole 128-k steps: 3 -> 6 + 6
    + 4 steps of 64, 7 -> 4 splits of 4), k = 960 the one with 64 k."""
    m, n = 200, 520
    w = synth.student_t_weights(n, k, seed=1000)
    q, r = _quant(w)
    x = synth.activations(m, k, seed=1001)
    ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
    for dt in (torch.bfloat16, torch.float32):
        y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt, path=nv.PATH_TILED, split_k=split)
        torch.cuda.synchronize()
        assert _rel(y, ref) <= TOL[dt], (split, k, dt)


def test_workspace_reuse_across_shapes():
    """One workspace, filled with garbage first, shared by a sequence of
    split-K calls of different shapes: its contents on entry never matter."""
    ws = torch.full((8 << 20,), 0xAB, dtype=torch.uint8, device="cuda")
    seq = [(1, 256, 256, 2), (1, 64, 256, 2), (48, 1024, 4096, 0), (3, 64, 4096, 5), (16, 4096, 4096, 3),
           (33, 64, 256, 0), (1, 64, 256, 2)]
    cache = {}
    for i, (m, n, k, split) in enumerate(seq):
        if (n, k) not in cache:
            w = synth.student_t_weights(n, k, seed=600 + len(cache))
            cache[(n, k)] = _quant(w)
        q, r = cache[(n, k)]
        x = synth.activations(m, k, seed=700 + i)
        assert nv.workspace_size(m, n, k, nv.PATH_SKINNY, split) <= ws.numel()
        y = nv.w4a16_gemm(x.cuda(), q, out_dtype=torch.float32, workspace=ws, path=nv.PATH_SKINNY,
                          split_k=split)
        torch.cuda.synchronize()
        ref = oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)
        assert _rel(y, ref) <= 1e-5, (m, n, k, split)


# ---------------------------------------------------------------------------
# nvfp4_w4a16_gemm_grouped: G matrices stacked row-wise, one tensor scale per
# group, one call.  Each group's column block of y against the oracle of that
# matrix alone (its own quantization and tensor scale), through every route
# the stacked shape dispatches to (full-K, persistent, single-launch with
# 1-4 tiles per workgroup, streaming split-K + reduction, tiled).
# ---------------------------------------------------------------------------
GROUPED_CASES = [
    # (group rows, k, token counts)
    ((48, 1024, 16), 512, (1, 5, 17, 40, 100)),
    ((4096, 4096, 4096), 4096, (1, 8, 17, 48)),  # q, k, v of the decoder layer
    ((14336, 14336), 4096, (1, 48)),             # gate, up
    ((256, 512), 1040, (3, 24, 200)),            # k % 512 != 0: split-K skinny and single-stage tiled
]


@pytest.mark.parametrize("rows,k,ms", GROUPED_CASES, ids=lambda v: str(v))
def test_grouped_gemm(rows, k, ms):
    ws = [synth.student_t_weights(n, k, 2000 + 7 * i + n % 97) for i, n in enumerate(rows)]
    gq = nv.quantize_fos_grouped([torch.from_numpy(w).cuda() for w in ws])
    refs = [oracle.quantize_fos(w) for w in ws]
    torch.cuda.synchronize()
    off = 0
    for g, (r, n) in enumerate(zip(refs, rows)):
        q = gq.group(g)
        assert np.array_equal(q.codes.cpu().numpy(), r.codes) and np.array_equal(q.scales.cpu().numpy(), r.scales)
        assert q.tensor_scale.cpu().numpy()[0].view(np.uint32) == np.float32(r.tensor_scale).view(np.uint32)
    w_hats = [oracle.dequant_f64(r.codes, r.scales, r.tensor_scale) for r in refs]
    for m in ms:
        print("grouped", rows, k, "m", m, flush=True)
        x = synth.activations(m, k, 2100 + m)
        xd = x.cuda()
        xv = np.asarray(x.float().numpy(), dtype=np.float64)
        for dt in (torch.bfloat16, torch.float32):
            y = nv.w4a16_gemm_grouped(xd, gq, out_dtype=dt)
            torch.cuda.synchronize()
            yd = y.double().cpu().numpy()
            off = 0
            for g, n in enumerate(rows):
                ref = xv @ w_hats[g].T
                blk = yd[:, off:off + n]
                e = _rel(blk, ref)
                assert e <= _tol(dt, ref), (rows, k, m, g, dt, e)
                assert_gemm_elementwise(blk, x, w_hats[g], ref, dt, f"grouped {rows} g={g} m={m} {dt}")
                off += n


def test_grouped_gemm_errors():
    lib = nv.lib()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((48, 32), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((48, 4), dtype=torch.uint8, device="cuda")
    ts = torch.ones(3, dtype=torch.float32, device="cuda")
    y = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    import ctypes

    def call(rows, groups):
        arr = (ctypes.c_int64 * max(1, len(rows)))(*rows)
        return lib.nvfp4_w4a16_gemm_grouped(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), ts.data_ptr(),
                                            ctypes.cast(arr, ctypes.c_void_p), groups, y.data_ptr(), 4, 64, nv.BF16,
                                            None, 0, None)
    assert call([16, 16, 16], 3) == nv.NVFP4_OK
    assert call([16, 16, 16, 16, 16], 5) == 1
    assert call([16, 24, 8], 3) == 2  # not multiples of 16
    assert call([], 0) == 1
