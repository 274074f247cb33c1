"""The pipelined split-K, persistent full-K and one-token row-per-wave skinny kernels and the
large-M kernel with the weights in registers issue their weight loads as inline asm and wait for
them with counted vmcnt waits.  Compile them for gfx950 (device assembly,
the library's own flags) and check that no instruction touches a load's
destination register before the wait that covers it."""

import os
import subprocess

import pytest

from bit_gemm_amd import build
from asm_waits import check_assembly, check_kernel


def test_checker_flags_early_reads():
    # a load, then a read of its destination before any wait
    lines = ["global_load_dwordx4 v[4:7], v[0:1], off", "v_mov_b32_e32 v8, v5", "s_waitcnt vmcnt(0)"]
    assert check_kernel(lines) == ["v_mov_b32_e32 v8, v5"]
    # two loads in order: after vmcnt(1) the first has landed, the second not
    lines = ["global_load_dwordx4 v[4:7], v[0:1], off", "global_load_dword v9, v[0:1], off",
             "s_waitcnt vmcnt(1)", "v_mov_b32_e32 v8, v5", "v_add_u32_e32 v10, v9, v9",
             "s_waitcnt vmcnt(0)", "v_add_u32_e32 v11, v9, v9"]
    assert check_kernel(lines) == ["v_add_u32_e32 v10, v9, v9"]
    # LDS DMA and stores count in the order but have no register result
    lines = ["global_load_dword v9, v[0:1], off", "global_load_lds_dwordx4 v[2:3], off",
             "s_waitcnt vmcnt(1)", "v_mov_b32_e32 v8, v9"]
    assert check_kernel(lines) == []


_HAVE_HIPCC = os.path.exists("/opt/rocm/bin/hipcc") or bool(os.environ.get("HIPCC"))
# (source, extra defines): the GEMM sources are also built with one tensor
# scale per group of stacked matrices (NVFP4_GROUPED), whose epilogues read
# each column's scale; both builds are checked
_BUILDS = [("gemm_skinny.hip", ()), ("gemm_skinny.hip", ("-DNVFP4_GROUPED=1",)),
           ("gemm_tiled.hip", ()), ("gemm_tiled.hip", ("-DNVFP4_GROUPED=1",)), ("gemm_dx.hip", ())]
_ASM = {}


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """Device assembly of every build above, compiled once and in parallel."""
    if not _ASM:
        d = tmp_path_factory.mktemp("asm")
        flags = [f for f in build.COMMON if f != "-fPIC"]
        procs = []
        for i, (source, defs) in enumerate(_BUILDS):
            out = d / f"{i}.s"
            cmd = [build.hipcc(), *flags, *defs, "-x", "hip", "--offload-device-only", "-S",
                   os.path.join(build.CSRC, source), "-o", str(out)]
            procs.append(((source, defs), out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                                 text=True)))
        for key, out, pr in procs:
            _, err = pr.communicate()
            assert pr.returncode == 0, err[-2000:]
            _ASM[key] = out.read_text()
    return _ASM


@pytest.mark.skipif(not _HAVE_HIPCC, reason="hipcc not available")
@pytest.mark.parametrize("grouped", [False, True], ids=["one_scale", "grouped"])
@pytest.mark.parametrize("source,pattern,minimum", [
    ("gemm_skinny.hip", r"k_skinny_pipe", 20),  # MT 1..4 x chunk lengths x 2 conversion implementations
    ("gemm_skinny.hip", r"k_skinny_str", 16),    # streaming kernel: MT 1..4 x chunk lengths x 2 conversion implementations
    ("gemm_skinny.hip", r"k_skinny_pk", 4),      # persistent full-K kernel: 8 or 16 token rows x 2 implementations
    ("gemm_skinny.hip", r"k_skinny_fx", 48),     # single-launch full-K kernel: MT 2..4 x 4 or 8 steps x 1..4 tiles x 2 implementations
    ("gemm_skinny.hip", r"k_skinny_rdot_dma", 16),  # one-token row-per-wave kernel with LDS DMA activations: 2..16 chunks of 2048, two rows per wave at 2
    ("gemm_tiled.hip", r"k_lmr", 4),             # weights-in-registers large-M kernels (64 or 128 k per barrier), 2 implementations each
])
def test_counted_waits_cover_every_use(device_asm, source, pattern, minimum, grouped):
    text = device_asm[(source, ("-DNVFP4_GROUPED=1",) if grouped else ())]
    found, bad = check_assembly(text, pattern)
    assert found >= minimum, found
    assert bad == [], bad[:10]


@pytest.mark.skipif(not _HAVE_HIPCC, reason="hipcc not available")
def test_counted_waits_input_gradient(device_asm):
    """The input-gradient kernel with transposing LDS reads loads the weights
    two steps ahead with inline asm and counted waits, like the kernels above."""
    found, bad = check_assembly(device_asm[("gemm_dx.hip", ())], r"k_gemm_dx_tr")
    assert found >= 1, found
    assert bad == [], bad[:10]
