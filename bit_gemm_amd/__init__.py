"""Python binding of libnvfp4 (NVFP4 FourOverSix quantizer + W4A16 GEMM for
MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libnvfp4.so`` (built in-tree by ``python -m bit_gemm_amd.build``).  PyTorch
provides device memory and the current stream.  There is no CPU fallback:
if the library is missing, importing the entry points raises.

Entry points mirror the C ABI in ``include/nvfp4.h``:

* ``quantize_fos(w, amax=None)`` -> :class:`NVFP4Weight`
* ``dequant(q, dtype=torch.float32)``
* ``w4a16_gemm(x, q, out_dtype=torch.bfloat16)``
* ``selftest_cvt()``
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK = 0
STATUS_NAMES = {
    0: "NVFP4_OK",
    1: "NVFP4_ERR_INVALID_VALUE",
    2: "NVFP4_ERR_UNSUPPORTED_SHAPE",
    3: "NVFP4_ERR_MISALIGNED",
    4: "NVFP4_ERR_WORKSPACE_TOO_SMALL",
    5: "NVFP4_ERR_HIP",
    6: "NVFP4_ERR_UNSUPPORTED_DEVICE",
}
BF16, F32 = 0, 1
PATH_AUTO, PATH_SKINNY, PATH_TILED = 0, 1, 2
IMPL_DEFAULT, IMPL_PORTABLE, IMPL_HWCVT = 0, 1, 2

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size = ctypes.c_size_t

# name -> (restype, argtypes): every symbol include/nvfp4.h declares
SIGNATURES = {
    "nvfp4_quantize_fos": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "nvfp4_quantize_fos_ex": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_p]),
    "nvfp4_quantize_fos_gptq_workspace_size": (_c_size, [_c_i64, _c_i64]),
    "nvfp4_quantize_fos_gptq": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                         _c_size, _c_p]),
    "nvfp4_gptq_hessian_workspace_size": (_c_size, [_c_i64, _c_i64]),
    "nvfp4_gptq_hessian": (_c_int, [_c_p, _c_i64, _c_i64, ctypes.c_float, _c_p, _c_p, _c_size, _c_p]),
    "nvfp4_w4a16_gemm_grouped": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_p, _c_i64, _c_i64, _c_int, _c_p,
                                          _c_size, _c_p]),
    "nvfp4_tensor_amax": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "nvfp4_dequant": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_int, _c_p]),
    "nvfp4_w4a16_gemm_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "nvfp4_w4a16_gemm": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_p, _c_size, _c_p]),
    "nvfp4_w4a16_gemm_workspace_size_ex": (_c_size, [_c_i64, _c_i64, _c_i64, _c_int, _c_int]),
    "nvfp4_w4a16_gemm_ex": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_p, _c_size,
                                     _c_int, _c_int, _c_int, _c_p]),
    "nvfp4_w4a16_gemm_path": (_c_int, [_c_i64, _c_i64, _c_i64]),
    "nvfp4_w4a16_gemm_dx_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "nvfp4_w4a16_gemm_dx": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_p, _c_size,
                                     _c_p]),
    "nvfp4_quantize_act": (_c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "nvfp4_w4a4_gemm_workspace_size": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "nvfp4_w4a4_gemm": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_p, _c_size, _c_p]),
    "nvfp4_selftest_cvt": (_c_int, [_c_p, _c_p]),
    "nvfp4_stream_read": (_c_int, [_c_p, _c_size, _c_int, _c_int, _c_int, _c_p, _c_p]),
    "nvfp4_w4a16_gemm_noalloc": (_c_int, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_p]),
    "nvfp4_noalloc_scratch_bytes": (_c_size, []),
    "nvfp4_status_string": (ctypes.c_char_p, [_c_int]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
    "nvfp4_version": (_c_int, []),
}

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libnvfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != NVFP4_OK:
        raise NVFP4Error(status, lib().nvfp4_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None, device=None, min_numel: int = 0,
          gpu: bool = True):
    """Check a tensor argument before its pointer reaches the C ABI (which
    cannot see buffer sizes): dtype, contiguity, exact shape or a minimum
    element count, then GPU residence (and the device of the other
    arguments).  Raises ValueError."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} must have at least {min_numel} elements, got {t.numel()}")
    if not gpu:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")


def _on_gpu(dev, *named):
    """GPU residence (on device dev) of (tensor, name) pairs whose dtype and
    shape were checked already; None entries are skipped."""
    for t, name in named:
        if t is not None:
            _need(t, name, t.dtype, None, dev)


@dataclass
class NVFP4Weight:
    """Packed NVFP4 weight of a [n, k] matrix (see include/nvfp4.h)."""

    codes: torch.Tensor  # uint8 [n, k/2]
    scales: torch.Tensor  # uint8 [n, k/16]
    tensor_scale: torch.Tensor  # float32 [1]
    amax: torch.Tensor  # float32 [1]
    m4_mask: Optional[torch.Tensor]  # uint8 [n, k/16] or None

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)

    def check(self, device=None, need_amax: bool = False, gpu: bool = True):
        """Raise ValueError unless codes, scales, mask and the scalars are
        consistent tensors of one [n, k] matrix (k = 2 * codes.shape[1], a
        multiple of 16) and, with gpu, all on the GPU; returns (n, k)."""
        if not isinstance(self.codes, torch.Tensor) or self.codes.dim() != 2:
            raise ValueError("codes must be a 2-D uint8 tensor [n, k/2]")
        n, k = self.shape
        if k % 16 != 0:
            raise ValueError(f"codes imply k={k}, not a multiple of 16")
        dev = self.codes.device if device is None else device
        parts = [(self.codes, "codes", torch.uint8, (n, k // 2), 0),
                 (self.scales, "scales", torch.uint8, (n, k // 16), 0),
                 (self.tensor_scale, "tensor_scale", torch.float32, None, 1)]
        if need_amax:
            parts.append((self.amax, "amax", torch.float32, None, 1))
        if self.m4_mask is not None:
            parts.append((self.m4_mask, "m4_mask", torch.uint8, (n, k // 16), 0))
        for on_gpu in (False, True) if gpu else (False,):  # every shape first, then residence
            for t, name, dtype, shape, least in parts:
                _need(t, name, dtype, shape, dev, min_numel=least, gpu=on_gpu)
        return n, k


def quantize_fos(w: torch.Tensor, amax: Optional[torch.Tensor] = None, with_mask: bool = True,
                 impl: int = IMPL_DEFAULT, out: Optional[NVFP4Weight] = None) -> NVFP4Weight:
    """FourOverSix NVFP4 quantization of a float32 [n, k] GPU matrix."""
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("w must be a 2-D tensor")
    _need(w, "w", torch.float32, gpu=False)
    n, k = w.shape
    dev = w.device
    if out is not None:
        if out.check(dev, need_amax=True, gpu=False) != (n, k):
            raise ValueError(f"out holds a {out.shape} matrix, w is {(n, k)}")
        out.check(dev, need_amax=True)
    _on_gpu(dev, (w, "w"))
    if out is None:
        out = NVFP4Weight(
            codes=torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
            scales=torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
            tensor_scale=torch.empty(1, dtype=torch.float32, device=dev),
            amax=torch.empty(1, dtype=torch.float32, device=dev),
            m4_mask=torch.empty((n, k // 16), dtype=torch.uint8, device=dev) if with_mask else None,
        )
    if amax is not None:
        _need(amax, "amax", torch.float32, None, dev, min_numel=1)
    _check(lib().nvfp4_quantize_fos_ex(
        _ptr(w), n, k, _ptr(amax), _ptr(out.amax), _ptr(out.tensor_scale), _ptr(out.codes),
        _ptr(out.scales), _ptr(out.m4_mask), impl, _stream(dev)))
    return out


def gptq_workspace_size(n: int, k: int) -> int:
    return int(lib().nvfp4_quantize_fos_gptq_workspace_size(n, k))


def quantize_fos_gptq(w: torch.Tensor, hinv_u: torch.Tensor, amax: Optional[torch.Tensor] = None,
                      with_mask: bool = True, workspace: Optional[torch.Tensor] = None) -> NVFP4Weight:
    """FourOverSix scales fixed first, then GPTQ's column updates inside them.

    ``hinv_u``: float32 [k, k] GPU matrix, the upper Cholesky factor of the
    inverse Hessian (only its upper triangle is read)."""
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("w must be a 2-D tensor")
    _need(w, "w", torch.float32, gpu=False)
    n, k = w.shape
    dev = w.device
    _need(hinv_u, "hinv_u", torch.float32, (k, k), gpu=False)
    _on_gpu(dev, (w, "w"), (hinv_u, "hinv_u"))
    out = NVFP4Weight(
        codes=torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
        scales=torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
        tensor_scale=torch.empty(1, dtype=torch.float32, device=dev),
        amax=torch.empty(1, dtype=torch.float32, device=dev),
        m4_mask=torch.empty((n, k // 16), dtype=torch.uint8, device=dev) if with_mask else None,
    )
    if amax is not None:
        _need(amax, "amax", torch.float32, None, dev, min_numel=1)
    ws = gptq_workspace_size(n, k)
    if workspace is None:
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)  # its size: checked by the library
    _check(lib().nvfp4_quantize_fos_gptq(
        _ptr(w), n, k, _ptr(hinv_u), _ptr(amax), _ptr(out.amax), _ptr(out.tensor_scale), _ptr(out.codes),
        _ptr(out.scales), _ptr(out.m4_mask), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def gptq_hessian_workspace_size(s: int, k: int) -> int:
    return int(lib().nvfp4_gptq_hessian_workspace_size(s, k))


def gptq_hessian(x: torch.Tensor, damp: float = 0.01, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H = 2 X^T X + damp * mean(diag(2 X^T X)) * I, float32 [k, k], from
    bf16 calibration activations x [s, k] on the GPU (the Hessian whose
    inverse's upper Cholesky factor quantize_fos_gptq takes)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor")
    _need(x, "x", torch.bfloat16, gpu=False)
    s, k = x.shape
    dev = x.device
    if out is not None:
        _need(out, "out", torch.float32, (k, k), gpu=False)
    _on_gpu(dev, (x, "x"), (out, "out"))
    if out is None:
        out = torch.empty((k, k), dtype=torch.float32, device=dev)
    ws = gptq_hessian_workspace_size(s, k)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)  # its size: checked by the library
    _check(lib().nvfp4_gptq_hessian(_ptr(x), s, k, float(damp), _ptr(out), _ptr(workspace), workspace.numel(),
                                    _stream(dev)))
    return out


def tensor_amax(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """max |w| of a float32 GPU tensor, as a float32 [1] GPU tensor."""
    _need(w, "w", torch.float32, gpu=False)
    n, k = (w.shape[0], w.numel() // max(1, w.shape[0])) if w.dim() else (1, 1)
    if out is not None:
        _need(out, "out", torch.float32, None, min_numel=1, gpu=False)
    _on_gpu(w.device, (w, "w"), (out, "out"))
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=w.device)
    _check(lib().nvfp4_tensor_amax(_ptr(w), n, k, _ptr(out), _stream(w.device)))
    return out


def dequant(q: NVFP4Weight, dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    n, k = q.check(gpu=False)
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    code = {torch.float32: F32, torch.bfloat16: BF16}[dtype]
    dev = q.codes.device
    if out is None:
        out = torch.empty((n, k), dtype=dtype, device=dev)
    _need(out, "out", dtype, (n, k), gpu=False)
    q.check(dev)
    _on_gpu(dev, (out, "out"))
    _check(lib().nvfp4_dequant(_ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), _ptr(out), n, k, code,
                               _stream(q.codes.device)))
    return out


def workspace_size(m: int, n: int, k: int, path: int = PATH_AUTO, split_k: int = 0) -> int:
    return int(lib().nvfp4_w4a16_gemm_workspace_size_ex(m, n, k, path, split_k))


def gemm_path(m: int, n: int, k: int) -> int:
    return int(lib().nvfp4_w4a16_gemm_path(m, n, k))


def w4a16_gemm(x: torch.Tensor, q: NVFP4Weight, out_dtype: torch.dtype = torch.bfloat16,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               path: int = PATH_AUTO, split_k: int = 0, impl: int = IMPL_DEFAULT) -> torch.Tensor:
    """y[m, n] = x[m, k] @ W_hat[n, k]^T for bf16 x and NVFP4 weights."""
    n, k = q.check(gpu=False)
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}], got {tuple(getattr(x, 'shape', ()))}")
    m = x.shape[0]
    dev = q.codes.device
    _need(x, "x", torch.bfloat16, gpu=False)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    code = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (m, n), gpu=False)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, gpu=False)
    q.check(dev)
    _on_gpu(dev, (x, "x"), (out, "out"), (workspace, "workspace"))
    need = workspace_size(m, n, k, path, split_k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(lib().nvfp4_w4a16_gemm_ex(
        _ptr(x), _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), _ptr(out), m, n, k, code,
        _ptr(workspace), ws_bytes, path, split_k, impl, _stream(dev)))
    return out


@dataclass
class NVFP4Grouped:
    """G packed NVFP4 matrices of the same k stacked row-wise (the layout
    nvfp4_w4a16_gemm_grouped reads): group g owns rows
    [sum(group_rows[:g]), sum(group_rows[:g + 1])) of codes, scales and the
    mask, and element g of tensor_scales and amax."""

    codes: torch.Tensor  # uint8 [n_total, k/2]
    scales: torch.Tensor  # uint8 [n_total, k/16]
    tensor_scales: torch.Tensor  # float32 [G]
    amax: torch.Tensor  # float32 [G]
    m4_mask: Optional[torch.Tensor]  # uint8 [n_total, k/16] or None
    group_rows: tuple

    def group(self, g: int) -> NVFP4Weight:
        r0 = sum(self.group_rows[:g])
        r1 = r0 + self.group_rows[g]
        return NVFP4Weight(self.codes[r0:r1], self.scales[r0:r1], self.tensor_scales[g:g + 1], self.amax[g:g + 1],
                           None if self.m4_mask is None else self.m4_mask[r0:r1])


def quantize_fos_grouped(ws, with_mask: bool = True) -> NVFP4Grouped:
    """FourOverSix quantization of G float32 GPU matrices [n_g, k] (each
    n_g a multiple of 16), each with its own tensor scale, straight into
    stacked buffers."""
    ws = list(ws)
    if not ws or len(ws) > 4:
        raise ValueError("1 to 4 matrices")
    for i, w in enumerate(ws):
        if not isinstance(w, torch.Tensor) or w.dim() != 2:
            raise ValueError(f"matrix {i} must be a 2-D tensor")
        if w.shape[1] != ws[0].shape[1] or w.shape[0] % 16 != 0 or w.shape[0] == 0:
            raise ValueError(f"matrix {i}: every matrix needs the same k and a positive multiple of 16 rows")
    k = ws[0].shape[1]
    rows = tuple(int(w.shape[0]) for w in ws)
    n = sum(rows)
    dev = ws[0].device
    out = NVFP4Grouped(codes=torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                       scales=torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
                       tensor_scales=torch.empty(len(ws), dtype=torch.float32, device=dev),
                       amax=torch.empty(len(ws), dtype=torch.float32, device=dev),
                       m4_mask=torch.empty((n, k // 16), dtype=torch.uint8, device=dev) if with_mask else None,
                       group_rows=rows)
    for g, w in enumerate(ws):
        quantize_fos(w, out=out.group(g))
    return out


def w4a16_gemm_grouped(x: torch.Tensor, gq: NVFP4Grouped, out_dtype: torch.dtype = torch.bfloat16,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[m, n_total] = x @ [W_hat_0; W_hat_1; ...]^T, group g's columns with
    its own tensor scale, in one call (nvfp4_w4a16_gemm_grouped)."""
    G = len(gq.group_rows)
    n = sum(gq.group_rows)
    if not isinstance(gq.codes, torch.Tensor) or gq.codes.dim() != 2 or gq.codes.shape[0] != n:
        raise ValueError("codes must be [n_total, k/2]")
    k = gq.codes.shape[1] * 2
    _need(gq.codes, "codes", torch.uint8, (n, k // 2), gpu=False)
    _need(gq.scales, "scales", torch.uint8, (n, k // 16), gpu=False)
    _need(gq.tensor_scales, "tensor_scales", torch.float32, None, min_numel=G, gpu=False)
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}], got {tuple(getattr(x, 'shape', ()))}")
    _need(x, "x", torch.bfloat16, gpu=False)
    m = x.shape[0]
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    dev = gq.codes.device
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (m, n), gpu=False)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, gpu=False)
    _on_gpu(dev, (x, "x"), (gq.codes, "codes"), (gq.scales, "scales"), (gq.tensor_scales, "tensor_scales"),
            (out, "out"), (workspace, "workspace"))
    need = workspace_size(m, n, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    rows = (ctypes.c_int64 * G)(*gq.group_rows)
    _check(lib().nvfp4_w4a16_gemm_grouped(
        _ptr(x), _ptr(gq.codes), _ptr(gq.scales), _ptr(gq.tensor_scales), ctypes.cast(rows, ctypes.c_void_p), G,
        _ptr(out), m, k, {torch.float32: F32, torch.bfloat16: BF16}[out_dtype], _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(dev)))
    return out


def w4a16_gemm_noalloc(x: torch.Tensor, q: NVFP4Weight, out: torch.Tensor) -> torch.Tensor:
    """nvfp4_w4a16_gemm_noalloc: the W4A16 GEMM into a caller-provided
    output (bf16 or fp32 [m, n]) without a workspace and without allocating
    (split-K partials go to the library's fixed per-GPU scratch)."""
    n, k = q.check(gpu=False)
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}], got {tuple(getattr(x, 'shape', ()))}")
    m = x.shape[0]
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out must be a float32 or bfloat16 tensor")
    dev = q.codes.device
    _need(x, "x", torch.bfloat16, gpu=False)
    _need(out, "out", out.dtype, (m, n), gpu=False)
    q.check(dev)
    _on_gpu(dev, (x, "x"), (out, "out"))
    code = F32 if out.dtype == torch.float32 else BF16
    _check(lib().nvfp4_w4a16_gemm_noalloc(_ptr(x), _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), _ptr(out),
                                          m, n, k, code, _stream(dev)))
    return out


def gemm_dx_workspace_size(m: int, n: int, k: int) -> int:
    return int(lib().nvfp4_w4a16_gemm_dx_workspace_size(m, n, k))


def w4a16_gemm_dx(dy: torch.Tensor, q: NVFP4Weight, out_dtype: torch.dtype = torch.bfloat16,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dx = dy @ W_hat for bf16 [m, n] dy: the input gradient of the linear
    layer y = x @ W_hat^T (quantization-aware training's backward pass)."""
    nw, k = q.check(gpu=False)
    if not isinstance(dy, torch.Tensor) or dy.dim() != 2:
        raise ValueError("dy must be a 2-D tensor")
    m, n = dy.shape
    if nw != n:
        raise ValueError(f"dy has n={n}, weights n={nw}")
    dev = q.codes.device
    _need(dy, "dy", torch.bfloat16, gpu=False)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    code = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    if out is None:
        out = torch.empty((m, k), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (m, k), gpu=False)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, gpu=False)
    q.check(dev)
    _on_gpu(dev, (dy, "dy"), (out, "out"), (workspace, "workspace"))
    need = gemm_dx_workspace_size(m, n, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().nvfp4_w4a16_gemm_dx(_ptr(dy), _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), _ptr(out),
                                     m, n, k, code, _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                     _stream(dy.device)))
    return out


@dataclass
class NVFP4Act:
    """NVFP4 activations [m, k] (standard block scale) and, optionally, their
    block-scaled bf16 values val * sigma."""

    codes: torch.Tensor  # uint8 [m, k/2]
    scales: torch.Tensor  # uint8 [m, k/16]
    tensor_scale: torch.Tensor  # float32 [1]
    amax: torch.Tensor  # float32 [1]
    blockscaled: Optional[torch.Tensor]  # bf16 [m, k] or None


def quantize_act(x: torch.Tensor, amax: Optional[torch.Tensor] = None, with_blockscaled: bool = True,
                 out: Optional[NVFP4Act] = None) -> NVFP4Act:
    """NVFP4 quantization of bf16 [m, k] GPU activations (W4A4 input side)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor")
    _need(x, "x", torch.bfloat16, gpu=False)
    m, k = x.shape
    dev = x.device
    if out is not None:
        parts = [(out.codes, "out.codes", torch.uint8, (m, k // 2), 0),
                 (out.scales, "out.scales", torch.uint8, (m, k // 16), 0),
                 (out.tensor_scale, "out.tensor_scale", torch.float32, None, 1),
                 (out.amax, "out.amax", torch.float32, None, 1)]
        if out.blockscaled is not None:
            parts.append((out.blockscaled, "out.blockscaled", torch.bfloat16, (m, k), 0))
        for on_gpu in (False, True):
            for t, name, dtype, shape, least in parts:
                _need(t, name, dtype, shape, dev, min_numel=least, gpu=on_gpu)
    _on_gpu(dev, (x, "x"))
    out = out if out is not None else NVFP4Act(
        codes=torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
        scales=torch.empty((m, k // 16), dtype=torch.uint8, device=dev),
        tensor_scale=torch.empty(1, dtype=torch.float32, device=dev),
        amax=torch.empty(1, dtype=torch.float32, device=dev),
        blockscaled=torch.empty((m, k), dtype=torch.bfloat16, device=dev) if with_blockscaled else None,
    )
    if amax is not None:
        _need(amax, "amax", torch.float32, None, dev, min_numel=1)
    _check(lib().nvfp4_quantize_act(_ptr(x), m, k, _ptr(amax), _ptr(out.amax), _ptr(out.tensor_scale),
                                    _ptr(out.codes), _ptr(out.scales), _ptr(out.blockscaled), _stream(dev)))
    return out


def w4a4_workspace_size(m: int, n: int, k: int) -> int:
    return int(lib().nvfp4_w4a4_gemm_workspace_size(m, n, k))


def w4a4_gemm(x: torch.Tensor, q: NVFP4Weight, out_dtype: torch.dtype = torch.bfloat16,
              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = NVFP4(x) @ W_hat^T for bf16 [m, k] activations (W4A4)."""
    n, kw = q.check(gpu=False)
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor")
    m, k = x.shape
    if kw != k:
        raise ValueError(f"x has k={k}, weights k={kw}")
    dev = q.codes.device
    _need(x, "x", torch.bfloat16, gpu=False)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    code = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (m, n), gpu=False)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, gpu=False)
    q.check(dev)
    _on_gpu(dev, (x, "x"), (out, "out"), (workspace, "workspace"))
    need = w4a4_workspace_size(m, n, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib().nvfp4_w4a4_gemm(_ptr(x), _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), _ptr(out), m, n, k,
                                 code, _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def selftest_cvt(device=None) -> list:
    """Counters of nvfp4_selftest_cvt (see include/nvfp4.h)."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    buf = torch.zeros(8, dtype=torch.int32, device=dev)
    _check(lib().nvfp4_selftest_cvt(_ptr(buf), _stream(dev)))
    return [int(v) & 0xFFFFFFFF for v in buf.cpu().tolist()]


def stream_read(buf: torch.Tensor, nbytes: Optional[int] = None, grid: int = 512, loads_in_flight: int = 8,
                nontemporal: bool = True, sink: Optional[torch.Tensor] = None) -> None:
    """Read the first `nbytes` (default: all) of a contiguous GPU tensor once
    (the read-bandwidth ceiling measurement of nvfp4_stream_read)."""
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous tensor")
    total = buf.numel() * buf.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes < 0 or nbytes > total:
        raise ValueError(f"nbytes={nbytes} outside the buffer ({total} bytes)")
    if sink is None:
        sink = torch.empty(64, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32, None, min_numel=64, gpu=False)
    _on_gpu(buf.device, (buf, "buf"), (sink, "sink"))
    _check(lib().nvfp4_stream_read(_ptr(buf), nbytes, grid, loads_in_flight, 1 if nontemporal else 0, _ptr(sink),
                                   _stream(buf.device)))


def version() -> str:
    v = int(lib().nvfp4_version())
    return f"{v // 10000}.{(v // 100) % 100}.{v % 100}"
