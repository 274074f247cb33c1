#!/usr/bin/env python
"""Throughput of the W4A16 NVFP4 GEMM (and the FourOverSix quantizer around
it) on one MI355X (gfx950).

Workload (single decode-shaped layer): W fp32 4096 x 4096 drawn from a
Student-t (nu=5) scaled to std 0.02 with 0.1% outliers x20 (seed 2),
quantized with FourOverSix; bf16 activations N(0, 1) of shape M x 4096 for M
in {1, 8, 16, 32, 48} (seed 9000 + M).  Synthetic data stands in for the
pages' real model weights.

The timed step (the metric): the five W4A16 GEMMs, M = 1, 8, 16, 32, 48,
back to back, each reading its own cold copy of the packed weights from HBM
(the copies total ~1 GiB, beyond the 256 MB last-level cache), replayed from
HIP graphs.  value = 5 x packed-weight bytes (0.5625 B/weight) / step time.

Beside it (not in value): the whole hot-path step (tensor amax ->
FourOverSix quantization -> the five GEMMs -> bf16 dequant), per-kernel
durations from HIP events over graph-batched launches, the HBM read ceiling
of this GPU at the layer sizes (a read-only streaming kernel of the
library), the decoder shapes, the 32-layer decoder, GPTQ, and the CPU oracle
timed on this host.

Output: one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 NVFP4 GEMM HBM GB/s (% peak) at M=1..48; quantizer GB/s; bit-exact"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
N, K = 4096, 4096
M_LIST = [1, 8, 16, 32, 48]
W_SEED = 2
ROT_SRC = 8  # fp32 source copies (8 x 64 MiB)
ROT_SLOTS = 16  # rotation slots; each owns 7 packed copies
PASSES_PER_GRAPH = 4  # steps per captured graph
CAL_FLOATS = 64 * 1024 * 1024  # 256 MiB
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "traffic_w4096x4096.txt")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--kernel-reps", type=int, default=20, help="launches per graph when timing one kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg (profiling runs)")
    ap.add_argument("--profile-large-m", action="store_true",
                    help="only run the large-M GEMM configurations a few times, eagerly, for "
                         "rocprofv3 counter collection; prints the run list")
    ap.add_argument("--dispatch-sweep", action="store_true",
                    help="also time both GEMM paths at M = 1 ... 256 on the decoder shapes against the "
                         "automatic dispatch (adds ~1 minute)")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the per-shape GEMM report on the MLP and large-M decoder layers")
    ap.add_argument("--no-gptq", action="store_true", help="skip the GPTQ (FourOverSix scales) report")
    ap.add_argument("--gptq-only", action="store_true",
                    help="only the GPTQ report (for rocprofv3 runs), then exit")
    ap.add_argument("--gptq-shape", default=None,
                    help="restrict the GPTQ report to one shape (w4096x4096, up_gate or down)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time per leg")
    ap.add_argument("--no-cpu-configs", action="store_true",
                    help="skip the oracle on the MLP set and the large-M shapes (per-matrix M=4 share, "
                         "GPU == oracle)")
    ap.add_argument("--no-cpu-full", action="store_true",
                    help="skip the oracle on layers 0 and 31 of the 32-layer decoder in full (about 20 s "
                         "of host work)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the steps directly instead of from HIP graphs (for counter "
                         "collection); prints the step time only")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------
# algorithmic bytes (what the method itself must move per launch)
# ----------------------------------------------------------------------------
def bytes_amax(n, k):
    return 4 * n * k


def bytes_fos(n, k):  # read fp32 W, write codes (1/2), scales (1/16), mask (1/16)
    return n * k * (4 + 0.5 + 1 / 16 + 1 / 16)


def bytes_gemm(m, n, k):  # packed weights + bf16 x + bf16 y
    return n * k * (0.5 + 1 / 16) + 2 * m * k + 2 * m * n


def bytes_gemm_weights(n, k):
    return n * k * (0.5 + 1 / 16)


def bytes_dequant_bf16(n, k):
    return n * k * (0.5 + 1 / 16 + 2)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "bit_gemm_amd", "csrc"))):
        with open(os.path.join(ROOT, "bit_gemm_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic_summary(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 --pmc
    summary (FETCH_SIZE + WRITE_SIZE, calibrated), or None when absent or
    taken on other kernel sources."""
    try:
        kv = {}
        with open(PROFILE_SUMMARY) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    a, b = line.split("=", 1)
                    kv[a.strip()] = b.strip()
        if kv.get("kernel_source_sha") != kernel_source_hash():
            return None
        return float(kv[f"{kernel}.hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        return 2
    import numpy as np
    import torch

    import bit_gemm_amd as nv
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nv.lib()

    # ------- counter calibration: a plain elementwise kernel of known size ----
    # (reads 256 MiB, writes 256 MiB; rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    # of this kernel give the scale of those counters on this GPU)
    cal_a = torch.ones(CAL_FLOATS, dtype=torch.float32, device=dev)
    cal_b = torch.empty_like(cal_a)
    for _ in range(3):
        torch.neg(cal_a, out=cal_b)
    torch.cuda.synchronize()
    del cal_a, cal_b

    # ---------------- inputs -------------------------------------------------
    w_host = synth.student_t_weights(N, K, W_SEED)
    if args.gptq_only:
        print(json.dumps({"metric": "GPTQ within FourOverSix scales", "gptq": gptq_report(
            args, torch.from_numpy(w_host).to(dev))}), flush=True)
        return 0
    if args.profile_large_m:
        runs = profile_large_m(torch.from_numpy(w_host).to(dev))
        print(json.dumps({"metric": "large-M GEMM runs for counter collection", "runs": runs}), flush=True)
        return 0
    src = [torch.from_numpy(w_host).to(dev) for _ in range(ROT_SRC)]
    xs = {m: synth.activations(m, K, synth.activation_seed(m)).to(dev) for m in M_LIST}
    ys = {m: torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in M_LIST}
    ws_bytes = max(nv.workspace_size(m, N, K) for m in M_LIST)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    deq_out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    amax_bufs = torch.empty((ROT_SLOTS, 1), dtype=torch.float32, device=dev)
    n_packed = 7 * ROT_SLOTS

    def packed(i):
        return nv.NVFP4Weight(codes=codes_all[i], scales=scales_all[i], tensor_scale=ts_all[i], amax=am_all[i],
                              m4_mask=mask_all[i])

    codes_all = torch.empty((n_packed, N, K // 2), dtype=torch.uint8, device=dev)
    scales_all = torch.empty((n_packed, N, K // 16), dtype=torch.uint8, device=dev)
    mask_all = torch.empty((n_packed, N, K // 16), dtype=torch.uint8, device=dev)
    ts_all = torch.empty((n_packed, 1), dtype=torch.float32, device=dev)
    am_all = torch.empty((n_packed, 1), dtype=torch.float32, device=dev)
    for i in range(n_packed):
        nv.quantize_fos(src[0], out=packed(i))
    torch.cuda.synchronize()

    # ---------------- one step, per rotation slot ----------------------------
    def op_amax(v):
        nv.tensor_amax(src[v % ROT_SRC], out=amax_bufs[v])

    def op_fos(v):
        nv.quantize_fos(src[v % ROT_SRC], amax=amax_bufs[v], out=packed(7 * v))

    def op_gemm(v, j):
        m = M_LIST[j]
        nv.w4a16_gemm(xs[m], packed(7 * v + 1 + j), out=ys[m], workspace=workspace)

    def op_dequant(v):
        nv.dequant(packed(7 * v + 6), torch.bfloat16, out=deq_out)

    def step(v):
        op_amax(v)
        op_fos(v)
        for j in range(len(M_LIST)):
            op_gemm(v, j)
        op_dequant(v)

    stream = torch.cuda.Stream()
    step_bytes = (bytes_amax(N, K) + bytes_fos(N, K) + sum(bytes_gemm(m, N, K) for m in M_LIST)
                  + bytes_dequant_bf16(N, K))
    gemm_pass_weight_bytes = len(M_LIST) * bytes_gemm_weights(N, K)

    def gemm_pass(v):
        for j in range(len(M_LIST)):
            op_gemm(v, j)

    if args.eager:
        with torch.cuda.stream(stream):
            for s in range(args.warmup):
                step(s % ROT_SLOTS)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s in range(args.steps):
                step((args.warmup + s) % ROT_SLOTS)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / args.steps
        print(json.dumps({"metric": METRIC, "mode": "eager hot-path steps (profiling)",
                          "step_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                          "unit": "GB/s", "ms_per_step": round(ms, 4), "steps": args.steps, "warmup": args.warmup}))
        return 0
    with torch.cuda.stream(stream):
        for v in range(ROT_SLOTS):  # eager warm-up of every path before capture
            step(v)
    torch.cuda.synchronize()
    # Each graph holds PASSES_PER_GRAPH consecutive steps (rotation slots
    # v, v + 1, ...), so the host's graph launches stay ahead of the GPU and
    # the timed region measures the GPU's work, not the launch calls.
    def capture(fn, v, passes):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for p in range(passes):
                fn((v + p) % ROT_SLOTS)
        return g

    gemm_graphs = {p: [capture(gemm_pass, v, p) for v in range(ROT_SLOTS)] for p in (1, PASSES_PER_GRAPH)}
    step_graphs = {p: [capture(step, v, p) for v in range(ROT_SLOTS)] for p in (1, PASSES_PER_GRAPH)}
    torch.cuda.synchronize()

    def timed_replays(graphs):
        """ms per step over exactly args.steps steps (graphs of
        PASSES_PER_GRAPH steps, then single steps for the remainder), each
        step on the next rotation slot."""
        def run(nsteps, first):
            v = first
            for _ in range(nsteps // PASSES_PER_GRAPH):
                graphs[PASSES_PER_GRAPH][v % ROT_SLOTS].replay()
                v += PASSES_PER_GRAPH
            for _ in range(nsteps % PASSES_PER_GRAPH):
                graphs[1][v % ROT_SLOTS].replay()
                v += 1
            return v

        v = run(args.warmup, 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(args.steps, v)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / max(1, args.steps)

    # ---------------- timed region: K steps of the five GEMMs ----------------
    ms_per_step = timed_replays(gemm_graphs)
    value = gemm_pass_weight_bytes / (ms_per_step * 1e-3) / 1e9
    # the whole hot path (beside the metric)
    ms_hot = timed_replays(step_graphs)

    # ---------------- per-kernel durations: HIP events over graph batches ----
    def time_op(fn, L):
        """Average launch duration of fn(r) over a graph of L launches whose
        r-th launch touches rotation copy r (so reads stay cold)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(L):
                fn(r)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = 5
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            ev0.record(stream)
            for _ in range(reps):
                g.replay()
            ev1.record(stream)
        ev1.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / (reps * L)  # microseconds per launch

    def gemm_any(r, j):  # r-th launch reads packed copy r (all copies: ~1 GiB)
        m = M_LIST[j]
        nv.w4a16_gemm(xs[m], packed(r % n_packed), out=ys[m], workspace=workspace)

    def dequant_any(r):
        nv.dequant(packed(r % n_packed), torch.bfloat16, out=deq_out)

    # HBM read ceiling at the sizes the GEMMs stream (read-only kernel of the library)
    ceilings = read_ceilings(stream, time_op)
    ceil_layer = ceilings[str(int(bytes_gemm_weights(N, K)))]

    L = args.kernel_reps
    kernels = {}
    kernels["amax"] = dict(us=time_op(lambda r: op_amax(r % ROT_SLOTS), L), bytes=bytes_amax(N, K), launches=2,
                           note="fill + amax reduction kernels")
    kernels["fos_quantize"] = dict(us=time_op(lambda r: op_fos(r % ROT_SLOTS), L), bytes=bytes_fos(N, K),
                                   launches=1)
    for j, m in enumerate(M_LIST):
        kernels[f"gemm_m{m}"] = dict(us=time_op(lambda r, j=j: gemm_any(r, j), n_packed), bytes=bytes_gemm(m, N, K),
                                     weight_bytes=bytes_gemm_weights(N, K),
                                     path=nv.gemm_path(m, N, K),
                                     launches=2 if nv.workspace_size(m, N, K) > 0 else 1,
                                     flops=2 * m * N * K)
    kernels["dequant_bf16"] = dict(us=time_op(dequant_any, n_packed), bytes=bytes_dequant_bf16(N, K), launches=1)
    for name, kd in kernels.items():
        kd["gbs"] = kd["bytes"] / (kd["us"] * 1e-6) / 1e9
        kd["frac_hbm"] = kd["gbs"] / HBM_PEAK_GBS
        if "weight_bytes" in kd:
            kd["weight_gbs"] = kd["weight_bytes"] / (kd["us"] * 1e-6) / 1e9
            kd["weight_frac_hbm"] = kd["weight_gbs"] / HBM_PEAK_GBS
            kd["weight_frac_read_ceiling"] = kd["weight_gbs"] / ceil_layer["gbs"]
            kd["tflops"] = kd["flops"] / (kd["us"] * 1e-6) / 1e12
    # roofline: the GEMM call of the metric that takes longest (two kernels,
    # main + split-K reduction, when it needs a workspace)
    dominant = max((f"gemm_m{m}" for m in M_LIST), key=lambda k: kernels[k]["us"])
    dk = kernels[dominant]
    traffic = read_traffic_summary(dominant)
    dsts = [torch.empty_like(src[0]) for _ in range(4)]
    copy_bytes = 2 * src[0].numel() * 4
    copy_us = time_op(lambda r: dsts[r % 4].copy_(src[r % ROT_SRC]), L)
    copy_gbs = copy_bytes / (copy_us * 1e-6) / 1e9
    del dsts
    roofline = {"bound": "hbm", "kernel": dominant + (" (main kernel + split-K reduction)" if dk["launches"] == 2
                                                      else ""),
                "achieved": round(dk["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dk["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": dk["bytes"], "avg_launch_us": round(dk["us"], 3),
                "read_ceiling_gbs_same_size": round(ceil_layer["gbs"], 1),
                "frac_of_read_ceiling": round(dk["gbs"] / ceil_layer["gbs"], 4),
                "device_copy_gbs_64MiB": round(copy_gbs, 1)}

    gemm_us = sum(kernels[f"gemm_m{m}"]["us"] for m in M_LIST)
    gemm_summary = {
        "weight_gbs_all_m_events": round(gemm_pass_weight_bytes / (gemm_us * 1e-6) / 1e9, 1),
        "weight_frac_hbm_all_m": round(value / HBM_PEAK_GBS, 4),
        "weight_frac_read_ceiling_all_m": round(value / ceil_layer["gbs"], 4),
        "per_m": {m: {"us": round(kernels[f"gemm_m{m}"]["us"], 3),
                      "weight_gbs": round(kernels[f"gemm_m{m}"]["weight_gbs"], 1),
                      "frac_hbm": round(kernels[f"gemm_m{m}"]["weight_frac_hbm"], 4),
                      "frac_read_ceiling": round(kernels[f"gemm_m{m}"]["weight_frac_read_ceiling"], 4),
                      "tflops": round(kernels[f"gemm_m{m}"]["tflops"], 2)} for m in M_LIST},
    }
    fos = kernels["fos_quantize"]
    quant_us = fos["us"] + kernels["amax"]["us"]
    quant_summary = {
        "fos_kernel_gbs": round(fos["gbs"], 1), "fos_frac_hbm": round(fos["frac_hbm"], 4),
        "with_amax_pass_gbs": round((bytes_fos(N, K) + bytes_amax(N, K)) / (quant_us * 1e-6) / 1e9, 1),
        "weights_per_s": round(N * K / (quant_us * 1e-6), 1),
        "m4_share": round(float(mask_all[0].to(torch.int64).sum().item()) / mask_all[0].numel(), 4),
        "m4_share_pages_context": "40-43% of blocks (GPTQ on real weights, another GPU)",
    }

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "dtype_detail": "FP4 E2M1 weights (E4M3 block scales) x bf16 activations on bf16 MFMA / dot2, fp32 "
                        "accumulate; fp32 quantizer",
        "data": "synthetic",
        "config": {"workload": "W4A16 GEMM on one decode-shaped layer 4096x4096 (Student-t(5) std 0.02 + 0.1% "
                               "outliers x20, FourOverSix NVFP4), bf16 activations M in {1,8,16,32,48}; step = "
                               "the five GEMMs, each on a cold copy of the packed weights; value = packed-weight "
                               "bytes / step time",
                   "n": N, "k": K, "m": M_LIST, "step_weight_bytes": gemm_pass_weight_bytes},
        "roofline": roofline,
        "read_ceiling": ceilings,
        "gemm": gemm_summary,
        "hot_path_step": {"what": "tensor amax + FourOverSix quantize + the five GEMMs + bf16 dequant",
                          "ms": round(ms_hot, 4), "algorithmic_bytes": step_bytes,
                          "gbs": round(step_bytes / (ms_hot * 1e-3) / 1e9, 1)},
        "quantizer": quant_summary,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in kd.items()}
                    for k, kd in kernels.items()},
        "kernel_source_sha": kernel_source_hash(),
    }

    if args.dispatch_sweep:
        result["dispatch_sweep"] = dispatch_sweep(args, stream, time_op, src[0])
    if not args.no_shapes:
        result["decoder_shapes"] = decoder_shapes(args, stream, time_op, src[0], ceilings)
        result["decoder_model_32_layers"] = decoder_model(args, stream, src[0], ceilings)

    if not args.no_gptq:
        result["gptq"] = gptq_report(args, src[0])
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity"] = cpu_baseline(args, w_host, xs, packed(1))
    print(json.dumps(result), flush=True)
    return 0


READ_SIZES = [("layer_4096x4096_packed", 9437184), ("mlp_matrix_packed", 33030144), ("1GiB", 1 << 30)]


def read_ceilings(stream, time_op):
    """The HBM read ceiling at each size: the fastest of a sweep of launch
    shapes (256 .. 2048 workgroups of 256 threads, 4 or 8 16-byte loads per
    thread in flight, plain or non-temporal loads) of the library's
    read-only streaming kernel, each launch reading its own cold region of a
    1.25 GiB buffer (beyond the 256 MB last-level cache)."""
    import torch

    import bit_gemm_amd as nv

    total = 1280 << 20
    buf = torch.empty(total, dtype=torch.uint8, device=stream.device)
    buf.fill_(0x5A)
    sink = torch.empty(64, dtype=torch.int32, device=stream.device)
    out = {}
    for name, size in READ_SIZES:
        copies = total // size
        L = min(100, max(4, copies))
        views = [buf[(i % copies) * size:(i % copies) * size + size] for i in range(L)]
        best = None
        for grid in (256, 512, 1024, 2048):
            for u in (4, 8):
                for nt in (True, False):
                    us = time_op(lambda r: nv.stream_read(views[r % L], grid=grid, loads_in_flight=u,
                                                          nontemporal=nt, sink=sink), L)
                    if best is None or us < best[0]:
                        best = (us, grid, u, nt)
        us, grid, u, nt = best
        out[str(size)] = {"name": name, "bytes": size, "us": round(us, 3), "gbs": round(size / (us * 1e-6) / 1e9, 1),
                          "frac_hbm": round(size / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "launch": {"grid": grid, "loads_in_flight": u, "nontemporal": nt}}
        del views
    del buf
    torch.cuda.empty_cache()
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix rate
# decoder layer shapes (n, k)
MLP_SHAPES = [("up_gate", 14336, 4096, 30), ("down", 4096, 14336, 32)]  # (name, n, k, weight seed)
MLP_M = [1, 4, 16, 48]
LARGE_SHAPES = [("attn", 4096, 4096, 40), ("up_gate", 14336, 4096, 41)]
LARGE_M = [64, 256, 1024, 4096]


def decoder_shapes(args, stream, time_op, w_dev, ceilings):
    """GEMM latency on the other decoder-layer shapes (reported beside the
    step, not part of it): the MLP matrices at decode token counts (weight
    GB/s against HBM) and the large-M prefill shapes (TFLOP/s against the
    bf16 MFMA peak).  Each launch reads its own packed copy (>= 1 GiB of
    copies per shape for the decode counts) so weights come from HBM.  The
    weights are drawn on the GPU from the configs' distribution with their
    seeds (synth.student_t_weights_device: not the host draw's values, which
    would take ~15 s per MLP matrix to make)."""
    import torch

    import bit_gemm_amd as nv
    import synth

    dev = torch.device("cuda:0")
    out = {"mlp": {}, "large_m": {}, "weights": "each shape's own Student-t draw on the GPU (config seeds)"}

    def copies(n, k, count, seed):
        w = synth.student_t_weights_device(n, k, seed, dev)
        q = nv.quantize_fos(w)
        del w
        codes = q.codes.unsqueeze(0).repeat(count, 1, 1)
        scales = q.scales.unsqueeze(0).repeat(count, 1, 1)
        return [nv.NVFP4Weight(codes[i], scales[i], q.tensor_scale, q.amax, None) for i in range(count)]

    for name, n, k, seed in MLP_SHAPES:
        wb = bytes_gemm_weights(n, k)
        count = max(8, int((1 << 30) // wb))
        qs = copies(n, k, count, seed)
        ws = torch.empty(max(16, max(nv.workspace_size(m, n, k) for m in MLP_M)), dtype=torch.uint8, device=dev)
        res = {}
        for m in MLP_M:
            x = synth.activations(m, k, synth.activation_seed(m)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            us = time_op(lambda r: nv.w4a16_gemm(x, qs[r % count], out=y, workspace=ws), count)
            gbs = wb / (us * 1e-6) / 1e9
            ceil = ceilings.get(str(int(wb)))
            res[m] = {"us": round(us, 3), "weight_gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                      "frac_read_ceiling": round(gbs / ceil["gbs"], 4) if ceil else None,
                      "path": "skinny" if nv.gemm_path(m, n, k) == nv.PATH_SKINNY else "tiled"}
        out["mlp"][f"{name}_n{n}_k{k}"] = res
        del qs, ws
        torch.cuda.empty_cache()

    out["w4a4"] = {"note": "activations quantized to NVFP4 (amax pass + quantization kernel writing codes, "
                           "scales and block-scaled bf16 values), then the bf16-MFMA GEMM; tflops over the "
                           "whole call against the bf16 MFMA peak",
                   "shapes": {}}
    out["qat_input_grad"] = {"note": "dx = dy @ W_hat on the packed weights (the backward GEMM of "
                                     "quantization-aware training); tflops against the bf16 MFMA peak",
                             "shapes": {}}
    for name, n, k, seed in LARGE_SHAPES:
        qs = copies(n, k, 4, seed)
        ws = torch.empty(max(16, max(nv.workspace_size(m, n, k) for m in LARGE_M)), dtype=torch.uint8, device=dev)
        ws4 = torch.empty(max(nv.w4a4_workspace_size(m, n, k) for m in LARGE_M), dtype=torch.uint8, device=dev)
        res, res4, resd = {}, {}, {}
        for m in LARGE_M:
            x = synth.activations(m, k, synth.activation_seed(m)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            launches = 16 if m <= 1024 else 4
            us = time_op(lambda r: nv.w4a16_gemm(x, qs[r % 4], out=y, workspace=ws), launches)
            tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
            res[m] = {"us": round(us, 3), "tflops": round(tf, 1), "frac_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                      "path": "skinny" if nv.gemm_path(m, n, k) == nv.PATH_SKINNY else "tiled"}
            us4 = time_op(lambda r: nv.w4a4_gemm(x, qs[r % 4], out=y, workspace=ws4), launches)
            act = nv.quantize_act(x)
            usq = time_op(lambda r: nv.quantize_act(x, out=act), launches)
            tf4 = 2.0 * m * n * k / (us4 * 1e-6) / 1e12
            qbytes = m * k * (2 + 2 + 2 + 0.5 + 1 / 16)  # amax read, read, bf16 + codes + scales written
            res4[m] = {"us": round(us4, 3), "tflops": round(tf4, 1),
                       "frac_mfma_bf16": round(tf4 / MFMA_BF16_PEAK_TFLOPS, 4),
                       "act_quant_us": round(usq, 3),
                       "act_quant_gbs": round(qbytes / (usq * 1e-6) / 1e9, 1)}
            del act
            # quantization-aware training's input gradient on the same
            # weights: dx [m, k] = dy [m, n] @ W_hat
            dy = synth.activations(m, n, synth.activation_seed(m) + 1).to(dev)
            dxo = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
            usd = time_op(lambda r: nv.w4a16_gemm_dx(dy, qs[r % 4], out=dxo), launches)
            tfd = 2.0 * m * n * k / (usd * 1e-6) / 1e12
            resd[m] = {"us": round(usd, 3), "tflops": round(tfd, 1),
                       "frac_mfma_bf16": round(tfd / MFMA_BF16_PEAK_TFLOPS, 4)}
            del dy, dxo
        out["large_m"][f"{name}_n{n}_k{k}"] = res
        out["w4a4"]["shapes"][f"{name}_n{n}_k{k}"] = res4
        out["qat_input_grad"]["shapes"][f"{name}_n{n}_k{k}"] = resd
        del qs, ws, ws4
        torch.cuda.empty_cache()
    return out


SWEEP_SHAPES = [("attn", 4096, 4096), ("up_gate", 14336, 4096), ("down", 4096, 14336)]
SWEEP_M = [1, 2, 4, 8, 12, 16, 24, 32, 40, 48, 56, 64, 96, 128, 192, 256]


PROFILE_M = [256, 1024, 4096]


# fp32 vector ALU rate for separate multiply and subtract (no fused
# multiply-add, no packed fp32): 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
ALU_F32_OPS_PEAK_T = 256 * 4 * 16 * 2.4e9 / 1e12
GPTQ_CALIB_SEED = 4242


GPTQ_SHAPES = [("w4096x4096", 4096, 4096), ("up_gate", 14336, 4096), ("down", 4096, 14336)]


def gptq_report(args, w_dev):
    """GPTQ inside fixed FourOverSix scales on the decoder shapes: the damped
    Hessian H = 2 X^T X + 0.01 mean(diag) I from seeded synthetic calibration
    activations (2k x k, N(0,1) x per-channel U(1,2), as bf16) by the
    library's nvfp4_gptq_hessian (timed: HIP events, TFLOP/s of the full
    2 s k^2 product against the bf16 MFMA peak), then U (upper Cholesky factor
    of H^-1) by torch.linalg in float64 outside the timed region (a standard
    factorization the caller supplies); then the average
    duration of whole calls (amax and quantizer kernels, then one kernel per
    64 columns) with HIP events on the call's stream.  The 4096 x 4096 layer
    is the bench's own matrix; the MLP shapes tile it (the time does not
    depend on the values).

    The trailing updates bound it: each element w[r, l] receives one product
    and one subtraction per earlier column j < l, n k (k - 1) / 2 of each,
    on the fp32 vector ALU (the contract forbids fusing them)."""
    import torch

    import bit_gemm_amd as nv
    import synth

    dev = w_dev.device
    stream = torch.cuda.current_stream(dev)
    factors = {}

    hessians = {}

    def factor(k):
        if k not in factors:
            x = torch.from_numpy(synth.calibration_activations(2 * k, k, GPTQ_CALIB_SEED)).to(torch.bfloat16).to(dev)
            hws = torch.empty(nv.gptq_hessian_workspace_size(2 * k, k), dtype=torch.uint8, device=dev)
            h32 = torch.empty((k, k), dtype=torch.float32, device=dev)
            nv.gptq_hessian(x, 0.01, out=h32, workspace=hws)
            torch.cuda.synchronize()
            reps = 5
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                nv.gptq_hessian(x, 0.01, out=h32, workspace=hws)
            ev1.record(stream)
            ev1.synchronize()
            ms = ev0.elapsed_time(ev1) / reps
            tf = 2.0 * (2 * k) * k * k / (ms * 1e-3) / 1e12
            hessians[k] = {"calibration_samples": 2 * k, "ms": round(ms, 4), "tflops_full_product": round(tf, 1),
                           "frac_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                           "note": "tiles on and above the diagonal only: the executed MFMA work is about half"}
            del x, hws
            h = h32.to(torch.float64)
            del h32
            hinv = torch.cholesky_inverse(torch.linalg.cholesky(h))
            del h
            factors[k] = torch.linalg.cholesky(hinv, upper=True).to(torch.float32).contiguous()
            del hinv
            torch.cuda.empty_cache()
        return factors[k]

    out = {}
    for name, n, k in GPTQ_SHAPES:
        if args.gptq_shape and name != args.gptq_shape:
            continue
        w = w_dev if (n, k) == tuple(w_dev.shape) else \
            w_dev.repeat((n + N - 1) // N, (k + K - 1) // K)[:n, :k].contiguous()
        u = factor(k)
        ws = torch.empty(nv.gptq_workspace_size(n, k), dtype=torch.uint8, device=dev)
        q = None
        for _ in range(2):
            q = nv.quantize_fos_gptq(w, u, workspace=ws)
        torch.cuda.synchronize()
        reps = 5 if k <= 4096 else 3
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            q = nv.quantize_fos_gptq(w, u, workspace=ws)
        ev1.record(stream)
        ev1.synchronize()
        ms = ev0.elapsed_time(ev1) / reps
        rtn = nv.quantize_fos(w)
        torch.cuda.synchronize()
        moved = float((q.codes != rtn.codes).to(torch.float32).mean().item())
        ops = 2 * n * k * (k - 1) // 2
        tops = ops / (ms * 1e-3) / 1e12
        out[f"{name}_n{n}_k{k}"] = {
            "n": n, "k": k, "ms_per_call": round(ms, 4), "launches": 3 + k // 64, "update_ops": ops,
            "achieved_tops": round(tops, 2),
            "roofline": {"bound": "alu", "achieved": round(tops, 2), "peak": round(ALU_F32_OPS_PEAK_T, 2),
                         "unit": "T fp32 ops/s (mul, sub unfused)", "frac": round(tops / ALU_F32_OPS_PEAK_T, 4)},
            "code_bytes_changed_vs_rtn": round(moved, 4)}
        del w, ws, q, rtn
        torch.cuda.empty_cache()
    out["hessian"] = {f"k{k}": v for k, v in hessians.items()}
    return out


def profile_large_m(w_dev):
    """A short, eager run of the large-M configurations for counter
    collection (rocprofv3 --kernel-trace / --pmc): for each shape in
    LARGE_SHAPES and M in PROFILE_M, one warm-up and three launches of the
    automatic-path GEMM on the current stream, then the same for the QAT
    input gradient and for torch's dense bf16 GEMM (for comparison) at the
    largest M, in this fixed order (so dispatches map to configurations by
    their order)."""
    import torch

    import bit_gemm_amd as nv
    import synth

    dev = torch.device("cuda:0")
    runs = []
    for name, n, k, seed in LARGE_SHAPES:
        w = synth.student_t_weights_device(n, k, seed, dev)
        q = nv.quantize_fos(w)
        del w
        for m in PROFILE_M:
            x = synth.activations(m, k, synth.activation_seed(m)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(16, nv.workspace_size(m, n, k)), dtype=torch.uint8, device=dev)
            for _ in range(4):
                nv.w4a16_gemm(x, q, out=y, workspace=ws)
            torch.cuda.synchronize()
            runs.append({"shape": f"{name}_n{n}_k{k}", "m": m, "launches": 4, "flops": 2 * m * n * k,
                         "path": "skinny" if nv.gemm_path(m, n, k) == nv.PATH_SKINNY else "tiled",
                         "workspace_bytes": nv.workspace_size(m, n, k)})
        # the QAT input gradient dx = dy @ W_hat on the same packed weights, M = 4096
        m = PROFILE_M[-1]
        dy = synth.activations(m, n, synth.activation_seed(m) + 1).to(dev)
        dx = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(16, nv.gemm_dx_workspace_size(m, n, k)), dtype=torch.uint8, device=dev)
        for _ in range(4):
            nv.w4a16_gemm_dx(dy, q, out=dx, workspace=ws)
        torch.cuda.synchronize()
        runs.append({"shape": f"{name}_n{n}_k{k}", "m": m, "launches": 4, "flops": 2 * m * n * k, "path": "dx",
                     "workspace_bytes": nv.gemm_dx_workspace_size(m, n, k)})
        # context, not part of the library: torch's dense bf16 GEMM (hipBLASLt)
        # of the same shape, no dequantization - the matrix-core rate a plain
        # bf16 product reaches on this GPU
        a = synth.activations(m, k, synth.activation_seed(m)).to(dev)
        b = torch.randn((k, n), dtype=torch.bfloat16, device=dev)
        for _ in range(4):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        runs.append({"shape": f"{name}_n{n}_k{k}", "m": m, "launches": 4, "flops": 2 * m * n * k, "path": "blas",
                     "workspace_bytes": 0})
    return runs


def dispatch_sweep(args, stream, time_op, w_dev):
    """Both GEMM paths (their own automatic plans) at M = 1 ... 256 on the
    three decoder shapes, beside the path the automatic dispatch picks: the
    pages' rule is that the lower-latency kernel wins, so the dispatch is
    right where it picks the faster one.  Cold rotating copies as in
    decoder_shapes; the skinny path exists for m <= 64."""
    import torch

    import bit_gemm_amd as nv
    import synth

    dev = torch.device("cuda:0")
    out = {}
    for name, n, k in SWEEP_SHAPES:
        wb = bytes_gemm_weights(n, k)
        count = max(8, int((1 << 30) // wb))
        w = w_dev.repeat((n + N - 1) // N, (k + K - 1) // K)[:n, :k].contiguous()
        q = nv.quantize_fos(w)
        del w
        codes = q.codes.unsqueeze(0).repeat(count, 1, 1)
        scales = q.scales.unsqueeze(0).repeat(count, 1, 1)
        qs = [nv.NVFP4Weight(codes[i], scales[i], q.tensor_scale, q.amax, None) for i in range(count)]
        need = max(nv.workspace_size(m, n, k, p) for m in SWEEP_M for p in (nv.PATH_SKINNY, nv.PATH_TILED)
                   if p == nv.PATH_TILED or m <= 64)
        ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
        rows = {}
        for m in SWEEP_M:
            x = synth.activations(m, k, synth.activation_seed(m)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            t = {}
            for pname, p in (("skinny", nv.PATH_SKINNY), ("tiled", nv.PATH_TILED)):
                if p == nv.PATH_SKINNY and m > 64:
                    continue
                launches = count if m <= 64 else 16
                t[pname] = round(time_op(lambda r: nv.w4a16_gemm(x, qs[r % count], out=y, workspace=ws, path=p),
                                         launches), 3)
            auto = "skinny" if nv.gemm_path(m, n, k) == nv.PATH_SKINNY else "tiled"
            best = min(t, key=t.get)
            rows[m] = {"us": t, "auto": auto, "fastest": best,
                       "auto_over_fastest": round(t[auto] / t[best], 3)}
        out[f"{name}_n{n}_k{k}"] = rows
        del qs, codes, scales, ws
        torch.cuda.empty_cache()
    return out


def decoder_model(args, stream, w_dev, ceilings):
    """The full synthetic 32-layer decoder (hidden 4096, MLP width 14336;
    per layer q, k, v, o 4096 x 4096, gate and up n = 14336, k = 4096, down
    n = 4096, k = 14336): one FourOverSix quantization pass over all 224
    fp32 matrices (31.1 GB, amax pass + quantizer per matrix), and one
    sequential pass of the 224 W4A16 GEMMs at M = 1 and at M = 48 over the
    4.38 GB of packed weights, each pass replayed from one HIP graph.  Each
    of the 224 fp32 matrices is its own draw, made on the GPU with a
    generator seeded per layer and matrix (the single layer's distribution;
    drawing 7.8 G values on the host would take minutes); the M=4 share of
    every matrix comes from the GPU quantizer's mask, summarised per matrix
    kind beside the pages' 40-43 %."""
    import torch

    import bit_gemm_amd as nv
    import synth

    dev = torch.device("cuda:0")
    layers = 32
    shapes = [(name, n, k) for name, n, k in synth.decoder_layer_shapes()]
    # fp32 model: one flat buffer, a view per matrix
    sizes = [n * k for _, n, k in shapes] * layers
    total = sum(sizes)
    flat = torch.empty(total, dtype=torch.float32, device=dev)
    views, off = [], 0
    for li in range(layers):
        for j, (_, n, k) in enumerate(shapes):
            v = flat[off:off + n * k].view(n, k)
            v.copy_(synth.student_t_weights_device(n, k, synth.decoder_weight_seed(li, j), dev))
            views.append(v)
            off += n * k
    torch.cuda.synchronize()
    # packed weights stacked per layer as the grouped GEMM reads them: q, k, v
    # in one buffer, gate and up in one, o and down alone; every matrix is
    # also a view of its rows (the per-matrix GEMM pass uses those)
    def stacked(rows, k):
        return nv.NVFP4Grouped(codes=torch.empty((sum(rows), k // 2), dtype=torch.uint8, device=dev),
                               scales=torch.empty((sum(rows), k // 16), dtype=torch.uint8, device=dev),
                               tensor_scales=torch.empty(len(rows), dtype=torch.float32, device=dev),
                               amax=torch.empty(len(rows), dtype=torch.float32, device=dev),
                               m4_mask=torch.empty((sum(rows), k // 16), dtype=torch.uint8, device=dev),
                               group_rows=tuple(rows))

    names = [nm for nm, _, _ in shapes]
    dims = {nm: (n, k) for nm, n, k in shapes}
    groups_of_layer = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    layer_groups, packed = [], []
    for _ in range(layers):
        per = {}
        gl = []
        for grp in groups_of_layer:
            st = stacked([dims[nm][0] for nm in grp], dims[grp[0]][1])
            gl.append(st)
            for i, nm in enumerate(grp):
                per[nm] = st.group(i)
        layer_groups.append(gl)
        packed.extend(per[nm] for nm in names)
    torch.cuda.synchronize()

    def replay_time(fn, reps=3):
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    def quant_pass():
        for v, q in zip(views, packed):
            nv.quantize_fos(v, out=q)

    tq = replay_time(quant_pass)
    # M=4 share per matrix (the last replay's masks: the same weights each time)
    shares = [float(q.m4_mask.float().mean()) for q in packed]
    by_kind = {}
    for i, (name, _, _) in enumerate(shapes * layers):
        by_kind.setdefault(name, []).append(shares[i])
    m4 = {name: {"mean": round(sum(v) / len(v), 4), "min": round(min(v), 4), "max": round(max(v), 4)}
          for name, v in by_kind.items()}
    attn = [x for nm in ("q", "k", "v", "o") for x in by_kind[nm]]
    mlp = [x for nm in ("gate", "up", "down") for x in by_kind[nm]]
    wsum = float(total)
    out = {"layers": layers, "weights": int(total), "fp32_bytes": int(4 * total),
           "packed_bytes": int(sum(bytes_gemm_weights(n, k) for _, n, k in shapes) * layers),
           "quantize_pass_ms": round(tq * 1e3, 3),
           "quantize_weights_per_s": round(wsum / tq, 1),
           "quantize_gbs_with_amax_pass": round(wsum * (4 + 4.625) / tq / 1e9, 1),
           "quantize_gbs_single_read": round(wsum * 4.625 / tq / 1e9, 1),
           "weights_source": "per-layer, per-matrix draws on the GPU (seed 5000 + 8 layer + matrix)",
           "m4_share_per_matrix_kind": m4,
           "m4_share_attention_mean": round(sum(attn) / len(attn), 4),
           "m4_share_mlp_mean": round(sum(mlp) / len(mlp), 4),
           "m4_share_pages_context": "40-43 % of blocks, higher in MLP than in attention QKV (real weights, "
                                     "GPTQ; another GPU): synthetic Student-t layers are not expected to match"}
    del flat, views
    torch.cuda.empty_cache()
    for m in (1, 48):
        xs = {k: synth.activations(m, k, synth.activation_seed(m)).to(dev) for k in {k for _, _, k in shapes}}
        ys = {n: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for n in {n for _, n, _ in shapes}}
        ws = torch.empty(max(16, max(nv.workspace_size(m, n, k) for _, n, k in shapes)), dtype=torch.uint8,
                         device=dev)

        def gemm_pass():
            for q in packed:
                n, k = q.codes.shape[0], q.codes.shape[1] * 2
                nv.w4a16_gemm(xs[k], q, out=ys[n], workspace=ws)

        tg = replay_time(gemm_pass)
        gbs = out["packed_bytes"] / tg / 1e9
        out[f"gemm_pass_m{m}"] = {"us": round(tg * 1e6, 1), "weight_gbs": round(gbs, 1),
                                  "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                  "frac_read_ceiling_1GiB": round(gbs / ceilings[str(1 << 30)]["gbs"], 4),
                                  "us_per_layer": round(tg * 1e6 / layers, 2)}
        # the same pass with the matrices that share an input in one call
        # each (q/k/v, gate/up: nvfp4_w4a16_gemm_grouped): 4 calls per layer
        yg = {sum(st.group_rows): torch.empty((m, sum(st.group_rows)), dtype=torch.bfloat16, device=dev)
              for st in layer_groups[0]}
        wsg = torch.empty(max(16, max(nv.workspace_size(m, sum(st.group_rows), st.codes.shape[1] * 2)
                                      for st in layer_groups[0])), dtype=torch.uint8, device=dev)

        def grouped_pass():
            for gl in layer_groups:
                for st in gl:
                    k = st.codes.shape[1] * 2
                    nv.w4a16_gemm_grouped(xs[k], st, out=yg[sum(st.group_rows)], workspace=wsg)

        tgg = replay_time(grouped_pass)
        gbs = out["packed_bytes"] / tgg / 1e9
        out[f"gemm_pass_grouped_m{m}"] = {"us": round(tgg * 1e6, 1), "weight_gbs": round(gbs, 1),
                                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                          "frac_read_ceiling_1GiB": round(gbs / ceilings[str(1 << 30)]["gbs"], 4),
                                          "us_per_layer": round(tgg * 1e6 / layers, 2), "calls_per_layer": 4}
        del yg, wsg
    del packed, layer_groups
    torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _repeat(fn, seconds):
    """Run fn until at least `seconds` have passed (at least once); returns
    (runs, elapsed seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return reps, dt


def cpu_baseline(args, w_host, xs_dev, q_dev):
    """The CPU oracle (oracle/, as it stands) timed on this host beside the
    GPU run, in the metric's unit: packed-weight GB/s of the W4A16 GEMM at
    M = 1, 8, 16, 32, 48 on the single layer, each GEMM being the oracle's
    float64 reference (exact dequantization, then a float64 product).  One
    leg on one core (the process pinned to it with sched_setaffinity, BLAS /
    torch / numpy on one thread), one on all cores of the affinity mask
    (capped at 16, the GPU machine's CPU share): the dequantizations and the
    quantizer on row chunks in a thread pool (blocks are independent once
    the tensor amax is known; numpy releases the GIL), BLAS on every thread.
    Also the quantizer, the MLP set (whole matrices: quantization time and
    the M=4 share, GPU == oracle bit for bit), the large-M shapes on a row
    sample, and the 32-layer decoder extrapolated from those rates (or run
    on layers 0 and 31 of the decoder in full).  The oracle is a reported baseline,
    not the optimisation target."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import bit_gemm_amd as nv
    import oracle
    import synth

    xs = {m: x.cpu() for m, x in xs_dev.items()}
    mask0 = os.sched_getaffinity(0)
    ncores = max(1, min(16, len(mask0)))
    torch_threads = torch.get_num_threads()
    wbytes = bytes_gemm_weights(N, K)

    def chunks_of(n):
        bounds = np.linspace(0, n, 4 * ncores + 1).astype(int)
        return [(a, b) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]

    # ---- one core: the process pinned to a single CPU ----------------------
    one_cpu = min(mask0)
    os.sched_setaffinity(0, {one_cpu})
    torch.set_num_threads(1)
    try:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            r = oracle.quantize_fos(w_host)  # includes the amax pass
            tq1 = time.perf_counter() - t0

            def gemms_one():
                for x in xs.values():
                    oracle.gemm_ref(x, r.codes, r.scales, r.tensor_scale)

            reps1, dt1 = _repeat(gemms_one, args.cpu_seconds / 2)
    finally:
        os.sched_setaffinity(0, mask0)
    one_core = {"value": round(len(xs) * wbytes * reps1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                "pinned_cpu": one_cpu, "gemm_passes": reps1, "seconds": round(dt1, 2),
                "quantize_s": round(tq1, 2),
                "quantize_weights_per_s": round(N * K / tq1, 1)}

    # ---- all cores ----------------------------------------------------------
    torch.set_num_threads(ncores)
    with threadpool_limits(limits=ncores), ThreadPoolExecutor(ncores) as ex:
        def quant_all(w):
            ch = chunks_of(w.shape[0])
            amax = np.float32(max(ex.map(lambda ab: float(np.abs(w[ab[0]:ab[1]]).max()), ch)))
            parts = list(ex.map(lambda ab: oracle.quantize_fos(w[ab[0]:ab[1]], amax_in=amax), ch))
            return (np.concatenate([q.codes for q in parts]), np.concatenate([q.scales for q in parts]),
                    np.concatenate([q.m4_mask for q in parts]), parts[0].tensor_scale)

        def gemm_all(x, codes, scales, s_t):  # oracle.gemm_ref's two steps, the dequant on row chunks
            w64 = np.concatenate(list(ex.map(
                lambda ab: oracle.dequant_f64(codes[ab[0]:ab[1]], scales[ab[0]:ab[1]], s_t), chunks_of(codes.shape[0]))))
            return np.asarray(x.float().numpy(), dtype=np.float64) @ w64.T

        def gemms_all():
            for x in xs.values():
                gemm_all(x, r.codes, r.scales, r.tensor_scale)

        repsA, dtA = _repeat(gemms_all, args.cpu_seconds / 4)
        qres = {}

        def q_once():
            qres["q"] = quant_all(w_host)

        repsQ, dtQ = _repeat(q_once, args.cpu_seconds / 4)
        all_ok = bool(np.array_equal(qres["q"][0], r.codes) and np.array_equal(qres["q"][1], r.scales))
        quant = {"weights_per_s_all_cores": round(N * K * repsQ / dtQ, 1),
                 "gbs_all_cores": round(N * K * (4 + 4.625) * repsQ / dtQ / 1e9, 3),
                 "weights_per_s_one_core": one_core["quantize_weights_per_s"],
                 "bytes_per_weight": "4 (amax pass) + 4.625 (read fp32, write codes, scales, mask)",
                 "all_cores_matches_one_core": all_ok}

        configs = {}
        rates = {"gemm_gbs": {}, "quant_wps": []}
        if not args.no_cpu_configs:
            configs = cpu_configs(args, ex, quant_all, gemm_all, rates, q_dev.codes.device)
        layers_measured = cpu_decoder_layers(args, quant_all, gemm_all, q_dev.codes.device) if not args.no_cpu_full else None
    torch.set_num_threads(torch_threads)

    gemm_rate_all = len(xs) * wbytes * repsA / dtA / 1e9
    # 32-layer decoder: extrapolated from the measured per-weight rates
    shapes = synth.decoder_layer_shapes()
    weights = 32 * sum(n * k for _, n, k in shapes)
    packed_bytes = 32 * sum(bytes_gemm_weights(n, k) for _, n, k in shapes)
    q_rate = quant["weights_per_s_all_cores"] if not rates["quant_wps"] else \
        sum(rates["quant_wps"]) / len(rates["quant_wps"])
    model = {"weights": weights, "quantize_s_extrapolated": round(weights / q_rate, 1),
             "basis": "all-core oracle rates measured above (quantizer weights/s on the MLP matrices when "
                      "they ran, else the single layer; GEMM packed-weight GB/s per M); every matrix of "
                      "the decoder has the single layer's or an MLP matrix's shape"}
    for m in (1, 48):
        g = rates["gemm_gbs"].get(m)
        if g:
            model[f"gemm_pass_m{m}_s_extrapolated"] = round(packed_bytes / (g * 1e9), 2)
    if layers_measured is not None:
        model["layers_0_31_measured"] = layers_measured

    cpu = {"value": round(gemm_rate_all, 4), "unit": "GB/s", "cores": ncores, "kind": "oracle",
           "sample": f"{repsA} passes of the five float64 reference GEMMs (M = 1, 8, 16, 32, 48) on the "
                     f"4096x4096 layer in {dtA:.1f} s on {ncores} threads, each GEMM dequantizing the packed "
                     f"weights exactly; one-core leg: {reps1} passes in {dt1:.1f} s pinned to CPU {one_cpu}",
           "one_core": one_core, "cpu_model": _cpu_model(), "quantizer": quant, "configs": configs,
           "decoder_model_32_layers": model}

    # parity of what the GPU holds for this workload
    codes_ok = bool(np.array_equal(q_dev.codes.cpu().numpy(), r.codes))
    scales_ok = bool(np.array_equal(q_dev.scales.cpu().numpy(), r.scales))
    mask_ok = bool(np.array_equal(q_dev.m4_mask.cpu().numpy(), r.m4_mask))
    errs = {}
    for m, x in xs_dev.items():
        ref = oracle.gemm_ref(xs[m], r.codes, r.scales, r.tensor_scale)
        y = nv.w4a16_gemm(x, q_dev).double().cpu().numpy()
        errs[m] = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
    parity = {"quantize_bit_exact": codes_ok and scales_ok and mask_ok, "gemm_rel_err_max": max(errs.values()),
              "gemm_rel_err_bound": 2e-3,
              "mlp_set_bit_exact": all(c.get("gpu_equals_oracle", False) for c in configs.get("mlp_set", {}).values())
              if configs.get("mlp_set") else None}
    return cpu, parity


def cpu_configs(args, ex, quant_all, gemm_all, rates, dev):
    """The oracle on the other workloads: the tiny layer in full; the MLP
    set (up, gate, down at their seeds) quantized whole, with the M=4 share
    of each matrix from the oracle and from the GPU (compared bit for bit),
    and the float64 GEMM at M = 1, 4, 16, 48 on a 1024-row sample (rows are
    independent once the matrix is quantized; the rate is per weight); the
    large-M product at M = 64 ... 4096 on a 256-row sample of the 4096 x
    4096 layer (seed 40)."""
    import numpy as np
    import torch

    import bit_gemm_amd as nv
    import oracle
    import synth

    out = {}
    w, x = synth.tiny(0)
    t0 = time.perf_counter()
    q = oracle.quantize_fos(w)
    oracle.gemm_ref(x, q.codes, q.scales, q.tensor_scale)
    out["tiny_256x256_ms"] = round((time.perf_counter() - t0) * 1e3, 2)

    mlp = {}
    for name, n, k, seed in synth.MLP_SET["layers"]:
        w = synth.student_t_weights(n, k, seed)
        t0 = time.perf_counter()
        codes, scales, mask, s_t = quant_all(w)
        tq = time.perf_counter() - t0
        rates["quant_wps"].append(n * k / tq)
        g = nv.quantize_fos(torch.from_numpy(w).to(dev))
        same = bool(np.array_equal(g.codes.cpu().numpy(), codes) and np.array_equal(g.scales.cpu().numpy(), scales)
                    and np.array_equal(g.m4_mask.cpu().numpy(), mask))
        share_gpu = float(g.m4_mask.to(torch.int64).sum().item()) / g.m4_mask.numel()
        rows = 1024
        gem = {}
        for m in synth.MLP_SET["m"]:
            xm = synth.activations(m, k, synth.activation_seed(m))
            t0 = time.perf_counter()
            gemm_all(xm, codes[:rows], scales[:rows], s_t)
            dt = (time.perf_counter() - t0) * n / rows
            gbs = bytes_gemm_weights(n, k) / dt / 1e9
            rates["gemm_gbs"].setdefault(m, gbs)
            gem[m] = {"s_extrapolated": round(dt, 3), "weight_gbs": round(gbs, 4)}
        mlp[f"{name}_n{n}_k{k}_seed{seed}"] = {
            "quantize_s": round(tq, 2), "quantize_weights_per_s": round(n * k / tq, 1),
            "m4_share_oracle": round(float(mask.mean()), 4), "m4_share_gpu": round(share_gpu, 4),
            "gpu_equals_oracle": same, "gemm_row_sample": rows, "gemm": gem}
        del w, g
        torch.cuda.empty_cache()
    out["mlp_set"] = mlp
    out["m4_share_pages_context"] = "40-43% of blocks, higher in MLP layers than in attention QKV (GPTQ on the " \
                                    "real model's weights, another GPU); synthetic Student-t layers are not " \
                                    "expected to match"
    w = synth.student_t_weights(4096, 4096, 40)
    n4, k4 = w.shape
    codes, scales, _, s_t = quant_all(w)
    rows = 256
    lm = {}
    for m in synth.LARGE_M["m"]:
        xm = synth.activations(m, k4, synth.activation_seed(m))
        t0 = time.perf_counter()
        gemm_all(xm, codes[:rows], scales[:rows], s_t)
        dt = (time.perf_counter() - t0) * n4 / rows
        lm[m] = {"s_extrapolated": round(dt, 3), "tflops_fp64": round(2.0 * m * n4 * k4 / dt / 1e12, 4)}
    out[f"large_m_{n4}x{k4}_seed40"] = {"row_sample": rows, "per_m": lm}
    return out


def cpu_decoder_layers(args, quant_all, gemm_all, dev):
    """Layers 0 and 31 of the 32-layer decoder in full: each matrix drawn at
    its seed, quantized by the oracle on all cores and by the GPU, compared
    bit for bit, with its M=4 share; then the oracle's float64 GEMM of the
    whole matrix at M = 1 and 48 (dequantization on row chunks in the thread
    pool, BLAS on all cores).  The 32-layer figures
    are these two layers' times x 16 (every layer has the same shapes and
    draws from the same distribution)."""
    import numpy as np
    import torch

    import bit_gemm_amd as nv
    import synth

    res = {}
    t_q = 0.0
    t_g = {1: 0.0, 48: 0.0}
    xs = {}
    for layer in (0, 31):
        for j, (name, n, k) in enumerate(synth.decoder_layer_shapes()):
            w = synth.student_t_weights(n, k, synth.decoder_weight_seed(layer, j))
            t0 = time.perf_counter()
            codes, scales, mask, s_t = quant_all(w)
            dt = time.perf_counter() - t0
            t_q += dt
            g = nv.quantize_fos(torch.from_numpy(w).to(dev))
            same = bool(np.array_equal(g.codes.cpu().numpy(), codes) and np.array_equal(g.scales.cpu().numpy(), scales)
                        and np.array_equal(g.m4_mask.cpu().numpy(), mask))
            entry = {"quantize_s": round(dt, 2), "m4_share": round(float(mask.mean()), 4), "gpu_equals_oracle": same}
            del w, g
            for m in (1, 48):
                if (m, k) not in xs:
                    xs[(m, k)] = synth.activations(m, k, synth.activation_seed(m))
                t0 = time.perf_counter()
                gemm_all(xs[(m, k)], codes, scales, s_t)
                dg = time.perf_counter() - t0
                t_g[m] += dg
                entry[f"gemm_m{m}_s"] = round(dg, 3)
            res[f"layer{layer}_{name}"] = entry
    res["quantize_s_two_layers"] = round(t_q, 2)
    res["quantize_s_32_layers_extrapolated"] = round(16 * t_q, 1)
    for m in (1, 48):
        res[f"gemm_pass_m{m}_s_two_layers"] = round(t_g[m], 2)
        res[f"gemm_pass_m{m}_s_32_layers_extrapolated"] = round(16 * t_g[m], 1)
    res["extrapolation"] = "32 layers = 16 x (layers 0 and 31): same shapes and weight distribution in every layer"
    return res


if __name__ == "__main__":
    sys.exit(main())
