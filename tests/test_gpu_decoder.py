"""GPU parity on the 32-layer synthetic decoder's own matrices (per-layer
seeds), for layers 0 and 31: the oracle over all 224 matrices would take
tens of minutes on the host, and every layer draws from the same generator
and distribution, so the first and last layer stand for the set.

For each of the 7 matrices of a layer (q, k, v, o: 4096 x 4096; gate, up:
n = 14336, k = 4096; down: n = 4096, k = 14336): the FourOverSix codes,
scales, M=4 mask, amax and tensor scale bit-exact with the oracle over the
whole matrix, and the W4A16 GEMM at the two token counts the decoder passes
run (1 and 48, the launch configuration of those passes: automatic path)
within the relative Frobenius bounds of the float64 oracle (bf16 and fp32
output) and the per-element bound of tests/gemm_bounds.py.
"""

import numpy as np
import pytest
import torch

import bit_gemm_amd as nv
import oracle
import synth
from gemm_bounds import assert_gemm_elementwise

pytestmark = pytest.mark.gpu

CASES = [(layer, j) for layer in (0, 31) for j in range(len(synth.decoder_layer_shapes()))]


@pytest.mark.parametrize("layer,j", CASES, ids=lambda v: str(v))
def test_decoder_layer_matrix(layer, j):
    name, n, k = synth.decoder_layer_shapes()[j]
    seed = synth.decoder_weight_seed(layer, j)
    print("decoder layer", layer, name, n, k, "seed", seed, flush=True)
    w = synth.student_t_weights(n, k, seed)
    q = nv.quantize_fos(torch.from_numpy(w).cuda())
    r = oracle.quantize_fos(w)
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), r.codes), name
    assert np.array_equal(q.scales.cpu().numpy(), r.scales), name
    assert np.array_equal(q.m4_mask.cpu().numpy(), r.m4_mask), name
    assert q.tensor_scale.cpu().numpy()[0].view(np.uint32) == np.float32(r.tensor_scale).view(np.uint32)
    assert q.amax.cpu().numpy()[0].view(np.uint32) == np.float32(r.amax).view(np.uint32)
    w_hat = oracle.dequant_f64(r.codes, r.scales, r.tensor_scale)
    for m in (1, 48):
        x = synth.activations(m, k, synth.activation_seed(m))
        ref = np.asarray(x.float().numpy(), dtype=np.float64) @ w_hat.T
        for dt, tol in ((torch.bfloat16, 2e-3), (torch.float32, 1e-5)):
            y = nv.w4a16_gemm(x.cuda(), q, out_dtype=dt).double().cpu().numpy()
            err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
            assert err <= tol, (name, m, dt, err)
            assert_gemm_elementwise(y, x, w_hat, ref, dt, f"layer {layer} {name} m={m} {dt}")
