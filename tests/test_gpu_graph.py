"""GPU: the hot path captured in a HIP graph and replayed.

The entry points only launch kernels on the caller's stream (no memset
nodes, no allocation, no host synchronisation), so a caller may capture
them.  This test captures one whole pass: amax, FourOverSix quantization,
W4A16 GEMMs on every kernel family (one token, full-K MFMA, pipelined and
streaming split-K, tiled), bf16 dequant, the W4A4 product, the input-gradient
GEMM and GPTQ.  It replays the graph several times, with other contents in
the captured input buffers and with eager work and synchronisations between
the replays, and checks every replay bit for bit against eager calls on the
same inputs.  The quantizer's output of each replay is also checked against
the oracle.
"""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth

pytestmark = pytest.mark.gpu

N, K = 1000, 1024
GEMM_M = (1, 8, 17, 48, 130)  # one token, full-K MFMA, pipelined, streaming, tiled
DX_M = (64, 300)
W4A4_M = 80
GN, GK = 256, 512  # GPTQ problem


def _inputs(seed):
    """One set of host inputs (seeded)."""
    return {
        "w": torch.from_numpy(synth.student_t_weights(N, K, seed)),
        "x": {m: synth.activations(m, K, seed * 10 + m) for m in GEMM_M},
        "dy": {m: synth.activations(m, N, seed * 20 + m) for m in DX_M},
        "xa": synth.activations(W4A4_M, K, seed * 30),
        "wg": torch.from_numpy(synth.student_t_weights(GN, GK, seed + 7)),
    }


class _Bufs:
    """Device input buffers, preallocated outputs and workspaces."""

    def __init__(self, inp):
        dev = "cuda"
        self.w = inp["w"].to(dev)
        self.x = {m: v.to(dev) for m, v in inp["x"].items()}
        self.dy = {m: v.to(dev) for m, v in inp["dy"].items()}
        self.xa = inp["xa"].to(dev)
        self.wg = inp["wg"].to(dev)
        self.q = nv.NVFP4Weight(
            codes=torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
            scales=torch.empty((N, K // 16), dtype=torch.uint8, device=dev),
            tensor_scale=torch.empty(1, dtype=torch.float32, device=dev),
            amax=torch.empty(1, dtype=torch.float32, device=dev),
            m4_mask=torch.empty((N, K // 16), dtype=torch.uint8, device=dev),
        )
        self.amax = torch.empty(1, dtype=torch.float32, device=dev)
        self.y = {m: torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in GEMM_M}
        ws = max([nv.workspace_size(m, N, K) for m in GEMM_M] + [nv.gemm_dx_workspace_size(m, N, K) for m in DX_M])
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.deq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        self.dx = {m: torch.empty((m, K), dtype=torch.float32, device=dev) for m in DX_M}
        self.ya = torch.empty((W4A4_M, N), dtype=torch.bfloat16, device=dev)
        self.wsa = torch.empty(nv.w4a4_workspace_size(W4A4_M, N, K) + 256, dtype=torch.uint8, device=dev)
        self.wsg = torch.empty(nv.gptq_workspace_size(GN, GK), dtype=torch.uint8, device=dev)

    def load(self, inp):
        self.w.copy_(inp["w"])
        for m in GEMM_M:
            self.x[m].copy_(inp["x"][m])
        for m in DX_M:
            self.dy[m].copy_(inp["dy"][m])
        self.xa.copy_(inp["xa"])
        self.wg.copy_(inp["wg"])


def _pass(b, u):
    """One pass of every entry point on the buffers of b; returns the outputs."""
    nv.tensor_amax(b.w, out=b.amax)
    nv.quantize_fos(b.w, out=b.q)  # its own amax (fill + reduction + quantizer)
    for m in GEMM_M:
        nv.w4a16_gemm(b.x[m], b.q, out=b.y[m], workspace=b.ws)
    nv.dequant(b.q, dtype=torch.bfloat16, out=b.deq)
    for m in DX_M:
        nv.w4a16_gemm_dx(b.dy[m], b.q, out_dtype=torch.float32, out=b.dx[m], workspace=b.ws)
    nv.w4a4_gemm(b.xa, b.q, out=b.ya, workspace=b.wsa)
    g = nv.quantize_fos_gptq(b.wg, u, workspace=b.wsg)
    outs = {"amax": b.amax, "codes": b.q.codes, "scales": b.q.scales, "ts": b.q.tensor_scale,
            "mask": b.q.m4_mask, "deq": b.deq, "w4a4": b.ya,
            "gptq_codes": g.codes, "gptq_scales": g.scales, "gptq_ts": g.tensor_scale}
    outs.update({f"y{m}": b.y[m] for m in GEMM_M})
    outs.update({f"dx{m}": b.dx[m] for m in DX_M})
    return outs


def _eager(inp, u):
    b = _Bufs(inp)
    outs = _pass(b, u)
    torch.cuda.synchronize()
    return {k: v.clone() for k, v in outs.items()}


def _bits(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def test_graph_replays_match_eager():
    sets = [_inputs(11), _inputs(12)]
    xg = synth.calibration_activations(2 * GK, GK, 913)
    u = torch.from_numpy(np.ascontiguousarray(oracle.hessian_factor(xg), dtype=np.float32)).cuda()
    refs = [_eager(s, u) for s in sets]
    codes_oracle = [oracle.quantize_fos(s["w"].numpy()).codes for s in sets]
    for r, c in zip(refs, codes_oracle):
        assert np.array_equal(r["codes"].cpu().numpy(), c)
    assert not torch.equal(refs[0]["y48"], refs[1]["y48"])  # the two sets give different results

    b = _Bufs(sets[0])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        _pass(b, u)  # warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        outs = _pass(b, u)
    torch.cuda.synchronize()

    for rep, si in enumerate((1, 0, 1, 1)):
        print("graph replay", rep, "input set", si, flush=True)
        b.load(sets[si])
        for t in outs.values():  # eager work between replays: scribble over every output
            if t.dtype == torch.uint8:
                t.fill_(0xA5)
            else:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(_bits(t), _bits(refs[si][name])), f"replay {rep}: {name} differs from eager"
        assert np.array_equal(outs["codes"].cpu().numpy(), codes_oracle[si])
