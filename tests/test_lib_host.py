"""Host-side tests of libnvfp4.so (CPU only: no kernel is launched).

The library must load without a GPU, export every symbol include/nvfp4.h
declares, and reject invalid arguments on the host before any HIP call.
"""

import ctypes
import os
import re

import pytest

import bit_gemm_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        from bit_gemm_amd import build
        build.build()
    return nv.lib()


def _declared():
    text = open(HEADER).read()
    return re.findall(r"NVFP4_API\s+[\w\s\*]+?\b(nvfp4_\w+)\s*\(", text)


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(nv.SIGNATURES)


def test_status_strings_and_version(L):
    for code, name in nv.STATUS_NAMES.items():
        assert L.nvfp4_status_string(code).decode() == name
    assert L.nvfp4_status_string(99).decode() == "NVFP4_ERR_UNKNOWN"
    assert nv.version() == "0.1.0"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first
ODD = 0x10008   # 8-byte aligned only


def test_quantize_rejects_bad_arguments_on_host(L):
    q = L.nvfp4_quantize_fos
    assert q(FAKE, 4, 24, None, FAKE, FAKE, FAKE, FAKE, None, None) == 2  # k % 16
    assert "multiple of 16" in L.nvfp4_last_error().decode()
    assert q(FAKE, -1, 32, None, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert q(FAKE, 4, 32, None, None, FAKE, FAKE, FAKE, None, None) == 1  # amax_out
    assert q(None, 4, 32, None, FAKE, FAKE, FAKE, FAKE, None, None) == 1  # w
    assert q(ODD, 4, 32, None, FAKE, FAKE, FAKE, FAKE, None, None) == 3  # misaligned w
    assert q(FAKE, 4, 32, None, FAKE + 2, FAKE, FAKE, FAKE, None, None) == 3
    assert q(FAKE, 1 << 31, 32, None, FAKE, FAKE, FAKE, FAKE, None, None) == 2
    assert L.nvfp4_quantize_fos_ex(FAKE, 4, 32, None, FAKE, FAKE, FAKE, FAKE, None, 7, None) == 1


def test_gptq_rejects_bad_arguments_on_host(L):
    g = L.nvfp4_quantize_fos_gptq
    ws = L.nvfp4_quantize_fos_gptq_workspace_size(4, 128)
    assert ws == 4 * 128 * 4 + 2 * 4 * 64 * 4  # working copy + two panels of errors
    assert L.nvfp4_quantize_fos_gptq_workspace_size(-1, 128) == 0
    assert L.nvfp4_quantize_fos_gptq_workspace_size(0, 128) == 0
    args = lambda **kw: [kw.get("w", FAKE), kw.get("n", 4), kw.get("k", 128), kw.get("u", FAKE), None,
                         FAKE, FAKE, FAKE, FAKE, None, kw.get("wsp", FAKE), kw.get("wsb", ws), None]
    assert g(*args(k=96)) == 2  # k % 64
    assert "k % 64" in L.nvfp4_last_error().decode()
    assert g(*args(k=24)) == 2  # k % 16 first
    assert g(*args(u=None)) == 1
    assert g(*args(w=None)) == 1
    assert g(*args(u=ODD)) == 3
    assert g(*args(wsb=ws - 1)) == 4
    assert g(*args(wsp=None)) == 1
    assert g(*args(wsp=ODD)) == 3
    assert g(*args(n=1 << 20, k=1 << 16)) == 2  # launch grid beyond 2^32 work-items


def test_w4a4_rejects_bad_arguments_on_host(L):
    qa = L.nvfp4_quantize_act
    assert qa(FAKE, 4, 24, None, FAKE, FAKE, FAKE, FAKE, None, None) == 2  # k % 16
    assert qa(None, 4, 32, None, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert qa(FAKE, 4, 32, None, FAKE, FAKE, FAKE, FAKE, ODD, None) == 3  # x_blockscaled
    e = 8 * 64
    act = 256 + 1024 + 256 + 256  # scalars, bf16 values, codes, scales (256-byte pieces)
    slack = 240  # bytes a 16-byte aligned buffer may skip to its first 256-byte boundary
    assert L.nvfp4_w4a4_gemm_workspace_size(8, 32, 64) == slack + act + L.nvfp4_w4a16_gemm_workspace_size(8, 32, 64)
    assert L.nvfp4_w4a4_gemm_workspace_size(0, 32, 64) == 0
    assert L.nvfp4_w4a4_gemm_workspace_size(8, 32, 24) == 0
    ws = L.nvfp4_w4a4_gemm_workspace_size(8, 32, 64)
    g = L.nvfp4_w4a4_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 32, 64, 0, FAKE, ws - 1, None) == 4
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 32, 64, 0, ODD, ws, None) == 3  # workspace: 16-byte alignment
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 32, 64, 5, FAKE, ws, None) == 1
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 32, 24, 0, FAKE, ws, None) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, 64, 0, None, 0, None) == 0  # empty: no work
    assert e == 512


def test_stream_read_rejects_bad_arguments_on_host(L):
    r = L.nvfp4_stream_read
    assert r(FAKE, 0, 512, 8, 1, FAKE, None) == 0  # nothing to read
    assert r(None, 1024, 512, 8, 1, FAKE, None) == 1
    assert r(FAKE, 1024, 512, 8, 1, None, None) == 1
    assert r(FAKE, 1000, 512, 8, 1, FAKE, None) == 2  # not a multiple of 16
    assert r(FAKE, 1024, 0, 8, 1, FAKE, None) == 1 and r(FAKE, 1024, 65537, 8, 1, FAKE, None) == 1
    assert r(FAKE, 1024, 512, 3, 1, FAKE, None) == 1  # loads in flight: 2, 4, 8 or 16
    assert r(ODD, 1024, 512, 8, 1, FAKE, None) == 3


def test_noalloc_gemm_rejects_on_host(L):
    g = L.nvfp4_w4a16_gemm_noalloc
    assert L.nvfp4_noalloc_scratch_bytes() == 32 << 20
    # a plan whose split-K partials exceed the fixed scratch: rejected before any HIP call
    assert L.nvfp4_w4a16_gemm_workspace_size(64, 14336, 14336) > L.nvfp4_noalloc_scratch_bytes()
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 14336, 14336, 0, None) == 4
    assert "no-allocation" in L.nvfp4_last_error().decode()
    # invalid arguments: the GEMM's own validation
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 32, 24, 0, None) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 32, 64, 7, None) == 1
    assert g(FAKE, FAKE, FAKE, FAKE, ODD, 8, 32, 64, 0, None) == 3
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, 64, 0, None) == 0  # empty: nothing to do


def test_gemm_dx_rejects_bad_arguments_on_host(L):
    g = L.nvfp4_w4a16_gemm_dx
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 24, 0, None, 0, None) == 2  # k % 16
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 32, 0, None, 0, None) == 1
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 32, 3, None, 0, None) == 1  # out dtype
    assert g(None, FAKE, FAKE, FAKE, FAKE, 4, 8, 32, 0, None, 0, None) == 1
    assert g(ODD, FAKE, FAKE, FAKE, FAKE, 4, 8, 32, 0, None, 0, None) == 3
    assert g(FAKE, FAKE, FAKE, FAKE, None, 4, 8, 32, 0, None, 0, None) == 1
    assert g(None, None, None, FAKE, FAKE, 0, 8, 32, 0, None, 0, None) == 0  # m == 0: nothing to do
    # few output tiles: the reduction over n is split (fp32 partial planes)
    ws = L.nvfp4_w4a16_gemm_dx_workspace_size(64, 4096, 4096)
    assert ws == 16 * 64 * 4096 * 4  # 32 tiles, 64 steps: 16 splits of 4 steps
    assert L.nvfp4_w4a16_gemm_dx_workspace_size(4096, 4096, 4096) == 0  # 1024 tiles
    assert L.nvfp4_w4a16_gemm_dx_workspace_size(64, 128, 4096) == 0  # 2 steps: nothing to split
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 4096, 4096, 0, FAKE, ws - 1, None) == 4
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 4096, 4096, 0, None, ws, None) == 1


def test_gemm_rejects_bad_arguments_on_host(L):
    g = L.nvfp4_w4a16_gemm_ex
    args = lambda m, n, k, **kw: dict(dict(x=FAKE, c=FAKE, s=FAKE, t=FAKE, y=FAKE, m=m, n=n, k=k, dt=0,
                                           ws=None, wsb=0, path=0, split=0, impl=0), **kw)

    def call(d):
        return g(d["x"], d["c"], d["s"], d["t"], d["y"], d["m"], d["n"], d["k"], d["dt"], d["ws"], d["wsb"],
                 d["path"], d["split"], d["impl"], None)

    assert call(args(1, 64, 40)) == 2
    assert call(args(-1, 64, 64)) == 1
    assert call(args(1, 64, 64, dt=5)) == 1
    assert call(args(1, 64, 64, path=9)) == 1
    assert call(args(1, 64, 64, impl=9)) == 1
    assert call(args(1, 64, 64, split=-1)) == 1
    assert call(args(65, 64, 64, path=1)) == 2  # skinny takes m <= 64
    assert call(args(1, 64, 64, x=ODD)) == 3
    assert call(args(1, 64, 64, y=None)) == 1
    need = L.nvfp4_w4a16_gemm_workspace_size_ex(1, 4096, 4096, nv.PATH_SKINNY, 4)
    assert need > 0
    assert call(args(1, 4096, 4096, wsb=need - 1, ws=FAKE, path=1, split=4)) == 4
    assert call(args(1, 4096, 4096, wsb=need, ws=None, path=1, split=4)) == 1
    assert call(args(1, 4096, 4096, wsb=need, ws=ODD, path=1, split=4)) == 3


def test_dequant_rejects_bad_arguments_on_host(L):
    d = L.nvfp4_dequant
    assert d(FAKE, FAKE, FAKE, FAKE, 4, 20, 0, None) == 2
    assert d(FAKE, FAKE, FAKE, FAKE, 4, 32, 3, None) == 1
    assert d(None, FAKE, FAKE, FAKE, 4, 32, 0, None) == 1
    assert d(FAKE, FAKE, FAKE, ODD, 4, 32, 0, None) == 3
    assert d(None, None, None, None, 0, 32, 0, None) == 0  # empty: nothing to do


def test_huge_row_counts_take_the_tiled_path(L):
    # the skinny kernels' grid would pass 2^32 work-items from n = 2^27 rows
    assert L.nvfp4_w4a16_gemm_path(1, 1 << 27, 16) == nv.PATH_TILED
    assert L.nvfp4_w4a16_gemm_path(1, (1 << 27) - 1, 16) == nv.PATH_SKINNY
    g = L.nvfp4_w4a16_gemm_ex
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1 << 27, 16, 0, None, 0, nv.PATH_SKINNY, 0, 0, None) == 2
    assert "2^27" in L.nvfp4_last_error().decode()


def test_dispatch_and_workspace_plan(L):
    S, T = nv.PATH_SKINNY, nv.PATH_TILED
    P = L.nvfp4_w4a16_gemm_path
    assert P(1, 4096, 4096) == S and P(16, 14336, 14336) == S
    assert P(48, 4096, 4096) == S and P(64, 4096, 4096) == S and P(65, 4096, 4096) == T
    # the pipelined skinny kernel up to m = 48 (k % 128 == 0), then the
    # tiled kernel on the larger shapes
    assert P(17, 14336, 4096) == S and P(48, 14336, 4096) == S and P(64, 14336, 4096) == S
    assert P(17, 4096, 14336) == S and P(48, 4096, 14336) == S and P(64, 4096, 14336) == S
    assert P(49, 14336, 4608) == S  # k % 512 == 0: the streaming kernel with 512-wide K chunks
    assert P(49, 14336, 4224) == T  # k % 512 != 0 (the streaming kernel needs it): tiled above 16
    assert P(24, 4096, 11008) == T and P(48, 14336, 4224) == T  # large, k % 512 != 0
    assert P(32, 4096, 4224) == S  # k % 512 != 0 but <= 2^25 weights: the split-K skinny kernel
    # 8 < m <= 16, more than 4096 rows, k % 512 != 0: tiled; up to 8 tokens or 4096 rows: full-K skinny
    assert P(12, 14336, 4224) == T and P(16, 5120, 13888) == T
    assert P(8, 14336, 4224) == S and P(16, 4096, 11008) == S and P(16, 14336, 4096) == S
    # 4 < m <= 8 on large matrices with k > 4096: the streaming kernel (a workspace); k <= 4096: full-K (none)
    assert L.nvfp4_w4a16_gemm_workspace_size(8, 13824, 5120) == 5 * 4 * 8 * 13824
    assert L.nvfp4_w4a16_gemm_workspace_size(8, 14336, 4096) == 0 and L.nvfp4_w4a16_gemm_workspace_size(4, 13824, 5120) == 0
    # the decoder's down projection (n = 4096, k = 14336: 2^25.8 weights) takes that route from m = 5
    for m in (5, 6, 7, 8):
        assert P(m, 4096, 14336) == S
        assert L.nvfp4_w4a16_gemm_workspace_size(m, 4096, 14336) == 14 * 4 * m * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size(4, 4096, 14336) == 0
    # one token: the row-per-wave kernel for every k % 32 == 0 from 2048 to 32768
    # (whole or partial chunks of 2048) and the full-K kernel for other k;
    # all skinny, one launch, no workspace
    for n, k in ((4096, 4096), (3584, 3584), (4101, 11008), (70, 32), (333, 4544), (8192, 28672),
                 (300, 32768), (64, 32784), (64, 48), (5, 4112)):
        assert P(1, n, k) == S, (n, k)
        assert L.nvfp4_w4a16_gemm_workspace_size(1, n, k) == 0, (n, k)
    assert P(48, 14336, 4160) == T  # k % 128 != 0, large: tiled
    assert P(48, 14336, 4112) == S and P(64, 4096, 4112) == S  # k % 64 != 0
    assert P(4096, 4096, 4096) == T
    assert L.nvfp4_w4a16_gemm_workspace_size(0, 4096, 4096) == 0
    # tiled path: m <= 64 one 64-token tile, K split to ~450 workgroups;
    # 64 < m <= 128: 128 x 128 tiles split to ~512 workgroups (>= 8 steps
    # per split); m > 128: 256 x 128 tiles split to ~256 workgroups (<= 4);
    # powers of two, >= 4 steps of 64 per split, at most 16 splits; K not a
    # multiple of 64 takes the single-stage kernel, no split
    T = nv.PATH_TILED
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(64, 4096, 4096, T, 0) == 16 * 4 * 64 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(48, 14336, 4096, T, 0) == 8 * 4 * 48 * 14336
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(48, 4096, 14336, T, 0) == 14 * 4 * 48 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size(128, 4096, 4096) == 8 * 4 * 128 * 4096
    # m > 128: 256 x 128 tiles (weights in registers), K split to ~256 workgroups
    # with >= 16 steps of 64 per split
    assert L.nvfp4_w4a16_gemm_workspace_size(256, 4096, 14336) == 8 * 4 * 256 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size(256, 4096, 4096) == 4 * 4 * 256 * 4096  # 32 tiles
    assert L.nvfp4_w4a16_gemm_workspace_size(256, 14336, 4096) == 2 * 4 * 256 * 14336  # 112 tiles
    assert L.nvfp4_w4a16_gemm_workspace_size(512, 14336, 4096) == 0  # 224 tiles
    assert L.nvfp4_w4a16_gemm_workspace_size(1024, 4096, 14336) == 2 * 4 * 1024 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size(2048, 4096, 4096) == 0
    assert L.nvfp4_w4a16_gemm_workspace_size(4096, 4096, 4096) == 0
    assert L.nvfp4_w4a16_gemm_workspace_size(1024, 14336, 4096) == 0
    assert L.nvfp4_w4a16_gemm_workspace_size(1024, 4096, 4096) == 2 * 4 * 1024 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(64, 4096, 4112, T, 0) == 0
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(256, 4096, 4096, T, 3) == 3 * 4 * 256 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(100, 256, 128, T, 5) == 2 * 4 * 100 * 256
    # k % 128 == 0 (128 k per barrier): splits in whole 128-k steps, 16 steps
    # of 64 in 7 -> 4 splits of 4; k % 128 == 64 keeps 64-k steps: 15 in 7 -> 5 of 3
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(200, 520, 1024, T, 7) == 4 * 4 * 200 * 520
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(200, 520, 960, T, 7) == 5 * 4 * 200 * 520
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(100, 256, 128, T, 1) == 0
    for m in (1, 8, 16):  # the full-K skinny kernels need no workspace
        for (n, k) in ((4096, 4096), (14336, 4096), (4096, 14336), (17, 48)):
            if (m > 8 or (m > 4 and k > 4096)) and (n > 4096 or n * k > 1 << 25) and k > 4096:  # streaming split-K
                assert L.nvfp4_w4a16_gemm_workspace_size(m, n, k) == (k // 1024) * 4 * m * n
            else:  # full K: one workgroup per 16 rows, or the persistent kernel (4 < m, k % 512 == 0, k <= 4096)
                assert L.nvfp4_w4a16_gemm_workspace_size(m, n, k) == 0
    # 4 < m <= 16, k % 512 == 0, k <= 4096: the persistent full-K kernel on any n
    for m in (5, 8, 9, 16):
        for (n, k) in ((14336, 4096), (4096, 4096), (1001, 512), (65536, 2048)):
            assert P(m, n, k) == S and L.nvfp4_w4a16_gemm_workspace_size(m, n, k) == 0
    C = 0  # the workspace holds only the fp32 partials [splits, m, n]
    for m in (17, 48):
        for (n, k) in ((4096, 4096), (14336, 4096), (4096, 14336), (17, 48)):
            ws = L.nvfp4_w4a16_gemm_workspace_size(m, n, k)
            assert ws == 0 or ((ws - C) % (4 * m * n) == 0 and ws <= 64 * 4 * m * n + C)
    # 16 < m <= 64 with at most 256 tiles of 16 rows, k <= 4096 a multiple of
    # 128 that 4..8 waves of 4 or 8 steps of 128 cover (m <= 48 unless
    # k <= 2048): the single-launch full-K kernel, no workspace
    for (m, n, k) in ((17, 4096, 4096), (32, 4096, 4096), (48, 4096, 4096), (64, 4096, 2048), (32, 1001, 3072),
                      (48, 4000, 2560), (20, 4096, 3584), (64, 17, 2048)):
        assert P(m, n, k) == S and L.nvfp4_w4a16_gemm_workspace_size(m, n, k) == 0, (m, n, k)
    # more than 256 tiles: 2 to 4 tiles per workgroup when that keeps 192 to
    # 256 workgroups (4 tiles only for k <= 2048)
    for (m, n, k) in ((17, 8192, 4096), (48, 12288, 4096), (48, 14336, 2048), (25, 7777, 2048)):
        assert P(m, n, k) == S and L.nvfp4_w4a16_gemm_workspace_size(m, n, k) == 0, (m, n, k)
    # more than 256 tiles otherwise, k > 4096, m > 48 with k > 2048, or k not
    # so covered: the streaming split-K kernel, K chunks of 1024
    assert L.nvfp4_w4a16_gemm_workspace_size(17, 4097, 4096) == C + 4 * 4 * 17 * 4097  # 129 workgroups of 2 tiles: too few
    assert L.nvfp4_w4a16_gemm_workspace_size(32, 4112, 4096) == C + 4 * 4 * 32 * 4112  # 257 tiles
    assert L.nvfp4_w4a16_gemm_workspace_size(64, 4096, 4096) == C + 4 * 4 * 64 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size(33, 1001, 3072) > 0  # 3 token tiles x 6 waves exceed LDS; 4 waves: 6 steps
    assert L.nvfp4_w4a16_gemm_workspace_size(32, 14336, 4096) == C + 4 * 4 * 32 * 14336
    assert L.nvfp4_w4a16_gemm_workspace_size(17, 4096, 14336) == C + 14 * 4 * 17 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size(48, 14336, 4096) == C + 4 * 4 * 48 * 14336
    assert L.nvfp4_w4a16_gemm_workspace_size(48, 4096, 14336) == C + 14 * 4 * 48 * 4096
    assert L.nvfp4_w4a16_gemm_workspace_size(33, 65, 1536) == C + 3 * 4 * 33 * 65  # k % 1024 != 0: chunks of 512
    assert L.nvfp4_w4a16_gemm_workspace_size(17, 4096, 4608) == C + 9 * 4 * 17 * 4096  # streaming, 9 chunks of 512
    assert L.nvfp4_w4a16_gemm_workspace_size(12, 14336, 4608) == C + 9 * 4 * 12 * 14336  # streaming, one token tile
    assert L.nvfp4_w4a16_gemm_workspace_size(64, 14336, 4608) == C + 9 * 4 * 64 * 14336  # streaming above 48 too
    # explicit split K
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(8, 4096, 2048, nv.PATH_SKINNY, 1) == 0
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(8, 4096, 4096, nv.PATH_SKINNY, 4) == C + 4 * 4 * 8 * 4096
    # a chunk larger than registers / LDS allow is split further (16 steps max)
    assert L.nvfp4_w4a16_gemm_workspace_size_ex(8, 4096, 8192, nv.PATH_SKINNY, 2) == C + 4 * 4 * 8 * 4096


# ---------------------------------------------------------------------------
# The Python binding checks every tensor argument before a pointer reaches
# the C ABI (which cannot see buffer sizes): shapes, dtypes and the packed
# weight's internal consistency, then GPU residence.  These run on CPU
# tensors: the shape and dtype checks come first, so each error below is the
# one named, raised before any GPU call.
# ---------------------------------------------------------------------------
def _cpu_weight(n=32, k=64):
    import torch

    return nv.NVFP4Weight(codes=torch.zeros((n, k // 2), dtype=torch.uint8),
                          scales=torch.zeros((n, k // 16), dtype=torch.uint8),
                          tensor_scale=torch.ones(1, dtype=torch.float32),
                          amax=torch.ones(1, dtype=torch.float32),
                          m4_mask=torch.zeros((n, k // 16), dtype=torch.uint8))


def test_binding_rejects_mismatched_weight_tensors():
    import torch

    q = _cpu_weight()
    q.scales = torch.zeros((32, 3), dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales must have shape"):
        nv.dequant(q)
    q = _cpu_weight()
    q.m4_mask = torch.zeros((31, 4), dtype=torch.uint8)
    with pytest.raises(ValueError, match="m4_mask must have shape"):
        q.check()
    q = _cpu_weight()
    q.tensor_scale = torch.ones(0, dtype=torch.float32)
    with pytest.raises(ValueError, match="tensor_scale must have at least 1"):
        nv.w4a16_gemm(torch.zeros((1, 64), dtype=torch.bfloat16), q)
    q = _cpu_weight()
    q.codes = torch.zeros((32, 12), dtype=torch.uint8)  # k = 24
    with pytest.raises(ValueError, match="not a multiple of 16"):
        q.check()
    q = _cpu_weight()
    q.scales = q.scales.to(torch.int32)
    with pytest.raises(ValueError, match="scales must be torch.uint8"):
        q.check()
    with pytest.raises(ValueError, match="must be a GPU tensor"):  # consistent, but on the host
        _cpu_weight().check()


def test_binding_rejects_wrong_output_shapes():
    import torch

    q = _cpu_weight(32, 64)
    x = torch.zeros((3, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"out must have shape \(3, 32\)"):
        nv.w4a16_gemm(x, q, out=torch.zeros((3, 31), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"x must be \[m, 64\]"):
        nv.w4a16_gemm(torch.zeros((3, 48), dtype=torch.bfloat16), q)
    with pytest.raises(ValueError, match="out_dtype"):
        nv.w4a16_gemm(x, q, out_dtype=torch.float16)
    with pytest.raises(ValueError, match=r"out must have shape \(32, 64\)"):
        nv.dequant(q, torch.float32, out=torch.zeros((32, 63), dtype=torch.float32))
    with pytest.raises(ValueError, match=r"out must have shape \(3, 64\)"):
        nv.w4a16_gemm_dx(torch.zeros((3, 32), dtype=torch.bfloat16), q,
                         out=torch.zeros((3, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dy has n=31"):
        nv.w4a16_gemm_dx(torch.zeros((3, 31), dtype=torch.bfloat16), q)
    with pytest.raises(ValueError, match=r"out must have shape \(3, 32\)"):
        nv.w4a4_gemm(x, q, out=torch.zeros((2, 32), dtype=torch.bfloat16))
    w = torch.zeros((32, 64), dtype=torch.float32)
    bad = _cpu_weight(16, 64)
    with pytest.raises(ValueError, match="out holds a"):
        nv.quantize_fos(w, out=bad)
    with pytest.raises(ValueError, match=r"hinv_u must have shape \(64, 64\)"):
        nv.quantize_fos_gptq(w, torch.zeros((64, 32), dtype=torch.float32))
    act = nv.NVFP4Act(codes=torch.zeros((3, 31), dtype=torch.uint8), scales=torch.zeros((3, 4), dtype=torch.uint8),
                      tensor_scale=torch.ones(1), amax=torch.ones(1), blockscaled=None)
    with pytest.raises(ValueError, match=r"out.codes must have shape \(3, 32\)"):
        nv.quantize_act(x, out=act)
    with pytest.raises(ValueError, match="out must have at least 1"):
        nv.tensor_amax(w, out=torch.zeros(0, dtype=torch.float32))


def test_hessian_host_validation(L):
    """nvfp4_gptq_hessian rejects bad arguments before any GPU call."""
    assert L.nvfp4_gptq_hessian_workspace_size(8192, 4096) == 4096 * 8192 * 2
    assert L.nvfp4_gptq_hessian_workspace_size(37, 48) == 48 * 64 * 2  # samples rounded up to 32
    assert L.nvfp4_gptq_hessian_workspace_size(-1, 48) == 0
    assert L.nvfp4_gptq_hessian(None, 4, 0, 0.01, None, None, 0, None) == nv.NVFP4_OK  # k = 0: nothing
    assert L.nvfp4_gptq_hessian(16, 4, 16, -1.0, 64, None, 0, None) == 1
    assert L.nvfp4_gptq_hessian(16, 4, 16, float("nan"), 64, None, 0, None) == 1
    assert L.nvfp4_gptq_hessian(16, 4, 16, 0.01, 64, None, 0, None) == 4  # workspace too small
    assert L.nvfp4_gptq_hessian(16, 4, 65537, 0.01, 64, None, 0, None) == 2
    assert L.nvfp4_gptq_hessian(17, 4, 16, 0.01, 64, 1024, 1 << 20, None) == 3  # x not 2-byte aligned
    assert L.nvfp4_gptq_hessian(None, 4, 16, 0.01, 64, 1024, 1 << 20, None) == 1  # x required for s > 0


def test_grouped_gemm_host_validation(L):
    import ctypes

    def call(rows, groups):
        arr = (ctypes.c_int64 * max(1, len(rows)))(*rows)
        return L.nvfp4_w4a16_gemm_grouped(16, 16, 16, 16, ctypes.cast(arr, ctypes.c_void_p), groups, 16, 4, 64,
                                          nv.BF16, None, 0, None)
    assert call([16, 16], 0) == 1 and call([16] * 5, 5) == 1
    assert call([16, 24], 2) == 2 and call([0, 16], 2) == 2 and call([-16], 1) == 2
    assert call([1 << 26, 1 << 26], 2) == 2  # 2^27 rows
    assert L.nvfp4_w4a16_gemm_grouped(16, 16, 16, 16, None, 1, 16, 4, 64, nv.BF16, None, 0, None) == 1
