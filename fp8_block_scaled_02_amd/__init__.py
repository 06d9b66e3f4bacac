"""libfp8w: FP8 (e4m3fn) weights for the decode path on MI355X (gfx950).

A thin ctypes binding over the C ABI of ``include/fp8w.h``.  Every function
here only checks and marshals arguments; all arithmetic runs in the HIP
kernels of ``libfp8w.so``.  PyTorch supplies device memory and the stream.
There is no CPU fallback: importing works on any host (so the symbol table
can be checked), but every call needs a ROCm GPU and the built library, and
fails loudly otherwise.

Functions carry the names of the C entry points:

* ``fp8w_quantize_block(w) -> (codes, scales)``   bf16 [n,k] -> u8 [n,k], f32 grid
* ``fp8w_quantize_mx(w) -> (codes, e8m0)``        bf16 [n,k] -> u8 [n,k], u8 [n,ceil(k/32)]
* ``fp8w_gemv_block(x, codes, scales) -> y``      bf16 [m,k] -> bf16 [m,n]
* ``fp8w_gemv_mx(x, codes, e8m0) -> y``
* ``fp8w_grouped_plan_init(xs, codes, scales) -> plan`` and
  ``fp8w_gemv_grouped(plan) -> ys``: many independent GEMVs in one launch
* ``fp8w_dequantize_block(codes, scales) -> w`` / ``fp8w_dequantize_mx``: bf16 [n,k]
* ``fp8w_gemm_block(x, codes, scales) -> y`` / ``fp8w_gemm_mx``: any m, through
  dequantize + a dense bf16 GEMM (the large-M route)
* ``fp8w_quantize_act(x) -> (x_codes, x_scale)`` and
  ``fp8w_gemv_block_w8a8(x_codes, x_scale, codes, scales) -> y`` / ``_mx_w8a8``:
  the W8A8 route (per-tensor fp8 activation, fp8 x fp8 matrix cores)

plus ``Fp8Weight``, a format-tagged weight whose GEMV asserts the format
before dispatch (a scale buffer of the wrong format cannot be detected by a
kernel: "quantize_fp8_bs.rs", Atlas weight_map, module notes).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8w.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_OVERLAP, ERR_HIP, ERR_CAPTURE = range(8)
ROUTE_AUTO, ROUTE_VALU, ROUTE_MFMA = 0, 1, 2
MAX_M = 32
TILE = 128
MX_GROUP = 32

# name -> (restype, argtypes); the exported C ABI, mirrored from include/fp8w.h
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "fp8w_scale_bytes": (_I64, [_I, _I64, _I64]),
    "fp8w_gemv_auto_route": (_I, [_I, _I64, _I64, _I64]),
    "fp8w_quantize": (_I, [_P, _I64, _I64, _I, _P, _P, _P, _I64, _P]),
    "fp8w_dequantize": (_I, [_P, _P, _I, _I64, _I64, _P, _P]),
    "fp8w_gemv": (_I, [_P, _I64, _P, _P, _I, _I64, _I64, _P, _I, _P]),
    "fp8w_gemm": (_I, [_P, _I64, _P, _P, _I, _I64, _I64, _P, _P, _I64, _P]),
    "fp8w_gemv_w8a8": (_I, [_P, _P, _I64, _P, _P, _I, _I64, _I64, _P, _P]),
    "fp8w_quantize_block": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "fp8w_quantize_mx": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "fp8w_gemv_block": (_I, [_P, _I64, _P, _P, _I64, _I64, _P, _P]),
    "fp8w_gemv_mx": (_I, [_P, _I64, _P, _P, _I64, _I64, _P, _P]),
    "fp8w_gemv_block_route": (_I, [_P, _I64, _P, _P, _I64, _I64, _P, _I, _P]),
    "fp8w_gemv_mx_route": (_I, [_P, _I64, _P, _P, _I64, _I64, _P, _I, _P]),
    "fp8w_dequantize_block": (_I, [_P, _P, _I64, _I64, _P, _P]),
    "fp8w_dequantize_mx": (_I, [_P, _P, _I64, _I64, _P, _P]),
    "fp8w_gemm_workspace_bytes": (_I64, [_I64, _I64]),
    "fp8w_gemm_prepare": (_I, []),
    "fp8w_gemm_block": (_I, [_P, _I64, _P, _P, _I64, _I64, _P, _P, _I64, _P]),
    "fp8w_gemm_mx": (_I, [_P, _I64, _P, _P, _I64, _I64, _P, _P, _I64, _P]),
    "fp8w_quantize_act_workspace_bytes": (_I64, []),
    "fp8w_quantize_act": (_I, [_P, _I64, _I64, _P, _P, _P, _I64, _P]),
    "fp8w_quantize_act_noalloc": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "fp8w_gemv_block_w8a8": (_I, [_P, _P, _I64, _P, _P, _I64, _I64, _P, _P]),
    "fp8w_gemv_mx_w8a8": (_I, [_P, _P, _I64, _P, _P, _I64, _I64, _P, _P]),
    "fp8w_read_ceiling": (_I, [_P, _I64, _P, _I64, _P]),
    "fp8w_grouped_table_bytes": (_I64, [_I64]),
    "fp8w_grouped_plan_init": (_I, [_P, _I64, _I64, _I, _I, _P, _P]),
    "fp8w_gemv_grouped": (_I, [_P, _P]),
    "fp8w_quant_table_bytes": (_I64, [_I64]),
    "fp8w_quant_plan_init": (_I, [_P, _I64, _I, _P, _P]),
    "fp8w_quantize_grouped": (_I, [_P, _P]),
    "fp8w_block_scale_count": (_I64, [_I64, _I64]),
    "fp8w_mx_scale_count": (_I64, [_I64, _I64]),
    "fp8w_status_string": (ctypes.c_char_p, [_I]),
    "fp8w_version": (_I, []),
}

FORMAT_BLOCK, FORMAT_MX, FORMAT_BLOCK_BF16, FORMAT_ROW, FORMAT_TENSOR = 0, 1, 2, 3, 4
FORMAT_IDS = {"block": FORMAT_BLOCK, "mx": FORMAT_MX, "block_bf16": FORMAT_BLOCK_BF16,
              "row": FORMAT_ROW, "tensor": FORMAT_TENSOR}


class GemvDesc(ctypes.Structure):
    """fp8w_gemv_desc of include/fp8w.h."""
    _fields_ = [("x", _P), ("codes", _P), ("scales", _P), ("y", _P),
                ("n", _I64), ("k", _I64)]


class GroupedPlanC(ctypes.Structure):
    """fp8w_grouped_plan of include/fp8w.h."""
    _fields_ = [("table", _P), ("count", ctypes.c_int32), ("m", ctypes.c_int32),
                ("format", ctypes.c_int32), ("route", ctypes.c_int32), ("blocks", _I64),
                ("tiles", _I64), ("tiles_per_block", ctypes.c_int32), ("seg_cols", ctypes.c_int32),
                ("mx_packed8", ctypes.c_int32)]


class QuantDesc(ctypes.Structure):
    """fp8w_quant_desc of include/fp8w.h."""
    _fields_ = [("w", _P), ("codes", _P), ("scales", _P), ("n", _I64), ("k", _I64)]


class QuantPlanC(ctypes.Structure):
    """fp8w_quant_plan of include/fp8w.h."""
    _fields_ = [("table", _P), ("count", ctypes.c_int32), ("format", ctypes.c_int32), ("blocks", _I64)]


_lib = None


class Fp8wError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load ``libfp8w.so`` (built by ``__graft_entry__.build()``), or raise."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m fp8_block_scaled_02_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().fp8w_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise Fp8wError(status, what)


def _torch():
    import torch
    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _require(t, dtypes, what: str, dims: int):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a GPU tensor (libfp8w has no CPU path)")
    if t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != dims or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous {dims}-d tensor")
    return t


def _bf16_like(torch):
    return (torch.bfloat16, torch.int16, torch.uint16)


def block_scale_shape(n: int, k: int):
    return ((n + TILE - 1) // TILE, (k + TILE - 1) // TILE)


def mx_scale_shape(n: int, k: int):
    return (n, (k + MX_GROUP - 1) // MX_GROUP)


def scale_shape(fmt: str, n: int, k: int):
    """Shape of the scale buffer of an [n, k] weight in format ``fmt``."""
    return {"block": block_scale_shape(n, k), "mx": mx_scale_shape(n, k),
            "block_bf16": block_scale_shape(n, k), "row": (n,), "tensor": (1,)}[fmt]


def _scale_dtype(torch, fmt: str):
    return {"block": torch.float32, "mx": torch.uint8, "block_bf16": torch.bfloat16,
            "row": torch.float32, "tensor": torch.float32}[fmt]


def _format_id(fmt: str) -> int:
    if fmt not in FORMAT_IDS:
        raise ValueError(f"unknown scale format {fmt!r}")
    return FORMAT_IDS[fmt]


def _check_scales(torch, fmt, scales, n, k, what):
    _require(scales, (_scale_dtype(torch, fmt),), "scales", len(scale_shape(fmt, n, k)))
    if tuple(scales.shape) != scale_shape(fmt, n, k):
        raise ValueError(f"{what}: {fmt} scales must be {scale_shape(fmt, n, k)}, got {tuple(scales.shape)}")


# --------------------------------------------------------------- quantize --

def fp8w_quantize(w, fmt: str = "block", codes=None, scales=None, workspace=None, stream=None):
    """bf16 W [n,k] -> (e4m3 codes u8 [n,k], scales in format ``fmt``)."""
    torch = _torch()
    _require(w, _bf16_like(torch), "w", 2)
    n, k = w.shape
    fid = _format_id(fmt)
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(scale_shape(fmt, n, k), dtype=_scale_dtype(torch, fmt), device=w.device)
    if workspace is None and fmt == "tensor":
        workspace = torch.empty(int(lib().fp8w_quantize_act_workspace_bytes()), dtype=torch.uint8,
                                device=w.device)
    _require(codes, (torch.uint8,), "codes", 2)
    _check_scales(torch, fmt, scales, n, k, "fp8w_quantize")
    ws_ptr, ws_n = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    _check(lib().fp8w_quantize(w.data_ptr(), n, k, fid, codes.data_ptr(), scales.data_ptr(), ws_ptr,
                               ws_n, _stream_handle(stream)), "fp8w_quantize")
    return codes, scales


def fp8w_dequantize(codes, scales, fmt: str = "block", w=None, stream=None):
    torch = _torch()
    _require(codes, (torch.uint8,), "codes", 2)
    n, k = codes.shape
    _check_scales(torch, fmt, scales, n, k, "fp8w_dequantize")
    if w is None:
        w = torch.empty((n, k), dtype=torch.bfloat16, device=codes.device)
    _require(w, _bf16_like(torch), "w", 2)
    _check(lib().fp8w_dequantize(codes.data_ptr(), scales.data_ptr(), _format_id(fmt), n, k,
                                 w.data_ptr(), _stream_handle(stream)), "fp8w_dequantize")
    return w


def fp8w_gemv(x, codes, scales, fmt: str = "block", y=None, route=0, stream=None):
    torch = _torch()
    _require(x, _bf16_like(torch), "x", 2)
    _require(codes, (torch.uint8,), "codes", 2)
    m, k = x.shape
    n = codes.shape[0]
    _check_scales(torch, fmt, scales, n, k, "fp8w_gemv")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _require(y, _bf16_like(torch), "y", 2)
    _check(lib().fp8w_gemv(x.data_ptr(), m, codes.data_ptr(), scales.data_ptr(), _format_id(fmt), n,
                           k, y.data_ptr(), int(route), _stream_handle(stream)), "fp8w_gemv")
    return y


def fp8w_gemv_auto_route(m: int, n: int, k: int, fmt: str = "block") -> int:
    """The kernel family AUTO takes for a single GEMV of m activation rows on an
    [n, k] weight with `fmt` scales: ROUTE_VALU or ROUTE_MFMA (ROUTE_AUTO when
    out of range)."""
    return int(lib().fp8w_gemv_auto_route(_format_id(fmt), int(m), int(n), int(k)))


def fp8w_gemm(x, codes, scales, fmt: str = "block", y=None, workspace=None, stream=None):
    torch = _torch()
    _require(x, _bf16_like(torch), "x", 2)
    _require(codes, (torch.uint8,), "codes", 2)
    m, k = x.shape
    n = codes.shape[0]
    _check_scales(torch, fmt, scales, n, k, "fp8w_gemm")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(int(lib().fp8w_gemm_workspace_bytes(n, k)), dtype=torch.uint8,
                                device=x.device)
    _require(y, _bf16_like(torch), "y", 2)
    _check(lib().fp8w_gemm(x.data_ptr(), m, codes.data_ptr(), scales.data_ptr(), _format_id(fmt), n, k,
                           y.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream_handle(stream)),
           "fp8w_gemm")
    return y


def fp8w_gemv_w8a8(x_codes, x_scale, codes, scales, fmt: str = "block", y=None, stream=None):
    torch = _torch()
    _require(x_codes, (torch.uint8,), "x_codes", 2)
    _require(x_scale, (torch.float32,), "x_scale", 1)
    _require(codes, (torch.uint8,), "codes", 2)
    m, k = x_codes.shape
    n = codes.shape[0]
    _check_scales(torch, fmt, scales, n, k, "fp8w_gemv_w8a8")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=codes.device)
    _require(y, _bf16_like(torch), "y", 2)
    _check(lib().fp8w_gemv_w8a8(x_codes.data_ptr(), x_scale.data_ptr(), m, codes.data_ptr(),
                                scales.data_ptr(), _format_id(fmt), n, k, y.data_ptr(),
                                _stream_handle(stream)), "fp8w_gemv_w8a8")
    return y



def fp8w_quantize_block(w, codes=None, scales=None, stream=None):
    """bf16 W [n,k] -> (e4m3fn codes u8 [n,k], fp32 scales [ceil(n/128), ceil(k/128)])."""
    torch = _torch()
    _require(w, _bf16_like(torch), "w", 2)
    n, k = w.shape
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(block_scale_shape(n, k), dtype=torch.float32, device=w.device)
    _require(codes, (torch.uint8,), "codes", 2)
    _require(scales, (torch.float32,), "scales", 2)
    if tuple(codes.shape) != (n, k) or tuple(scales.shape) != block_scale_shape(n, k):
        raise ValueError("fp8w_quantize_block: output shapes do not match w")
    _check(lib().fp8w_quantize_block(w.data_ptr(), n, k, codes.data_ptr(), scales.data_ptr(),
                                     _stream_handle(stream)), "fp8w_quantize_block")
    return codes, scales


def fp8w_quantize_mx(w, codes=None, e8m0=None, stream=None):
    """bf16 W [n,k] -> (e4m3fn codes u8 [n,k], e8m0 u8 [n, ceil(k/32)])."""
    torch = _torch()
    _require(w, _bf16_like(torch), "w", 2)
    n, k = w.shape
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    if e8m0 is None:
        e8m0 = torch.empty(mx_scale_shape(n, k), dtype=torch.uint8, device=w.device)
    _require(codes, (torch.uint8,), "codes", 2)
    _require(e8m0, (torch.uint8,), "e8m0", 2)
    if tuple(codes.shape) != (n, k) or tuple(e8m0.shape) != mx_scale_shape(n, k):
        raise ValueError("fp8w_quantize_mx: output shapes do not match w")
    _check(lib().fp8w_quantize_mx(w.data_ptr(), n, k, codes.data_ptr(), e8m0.data_ptr(),
                                  _stream_handle(stream)), "fp8w_quantize_mx")
    return codes, e8m0


# ------------------------------------------------------------------- GEMV --

def _gemv(fn_name, x, codes, scale_t, scale_shape, scale_dtype, y, route, stream):
    torch = _torch()
    _require(x, _bf16_like(torch), "x", 2)
    _require(codes, (torch.uint8,), "codes", 2)
    _require(scale_t, (scale_dtype,), "scales", 2)
    m, k = x.shape
    n, k2 = codes.shape
    if k != k2:
        raise ValueError(f"{fn_name}: x has K={k}, codes have K={k2}")
    if tuple(scale_t.shape) != scale_shape(n, k):
        raise ValueError(f"{fn_name}: scale grid {tuple(scale_t.shape)} != {scale_shape(n, k)}")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _require(y, _bf16_like(torch), "y", 2)
    if tuple(y.shape) != (m, n):
        raise ValueError(f"{fn_name}: y must be [{m}, {n}]")
    fn = getattr(lib(), fn_name + "_route")
    _check(fn(x.data_ptr(), m, codes.data_ptr(), scale_t.data_ptr(), n, k, y.data_ptr(),
              int(route), _stream_handle(stream)), fn_name)
    return y


def fp8w_gemv_block(x, codes, scales, y=None, route=ROUTE_AUTO, stream=None):
    """y[m,n] = x[m,k] . deq(W)^T with 128x128 fp32 block scales (bf16 out)."""
    torch = _torch()
    return _gemv("fp8w_gemv_block", x, codes, scales, block_scale_shape, torch.float32, y,
                 route, stream)


def fp8w_gemv_mx(x, codes, e8m0, y=None, route=ROUTE_AUTO, stream=None):
    """y[m,n] = x[m,k] . deq(W)^T with per-32 e8m0 scales (bf16 out)."""
    torch = _torch()
    return _gemv("fp8w_gemv_mx", x, codes, e8m0, mx_scale_shape, torch.uint8, y, route, stream)


# ------------------------------------------------------------- dequantize --

def _dequantize(fn_name, codes, scale_t, scale_shape, scale_dtype, w, stream):
    torch = _torch()
    _require(codes, (torch.uint8,), "codes", 2)
    _require(scale_t, (scale_dtype,), "scales", 2)
    n, k = codes.shape
    if tuple(scale_t.shape) != scale_shape(n, k):
        raise ValueError(f"{fn_name}: scale grid {tuple(scale_t.shape)} != {scale_shape(n, k)}")
    if w is None:
        w = torch.empty((n, k), dtype=torch.bfloat16, device=codes.device)
    _require(w, _bf16_like(torch), "w", 2)
    if tuple(w.shape) != (n, k):
        raise ValueError(f"{fn_name}: w must be [{n}, {k}]")
    _check(getattr(lib(), fn_name)(codes.data_ptr(), scale_t.data_ptr(), n, k, w.data_ptr(),
                                   _stream_handle(stream)), fn_name)
    return w


def fp8w_dequantize_block(codes, scales, w=None, stream=None):
    """bf16 W [n,k] = fl32(dec(codes) * block scale), rounded to bf16."""
    torch = _torch()
    return _dequantize("fp8w_dequantize_block", codes, scales, block_scale_shape, torch.float32, w, stream)


def fp8w_dequantize_mx(codes, e8m0, w=None, stream=None):
    """bf16 W [n,k] = dec(codes) * 2^(e8m0 - 127), rounded to bf16."""
    torch = _torch()
    return _dequantize("fp8w_dequantize_mx", codes, e8m0, mx_scale_shape, torch.uint8, w, stream)


# ------------------------------------------------------------------- GEMM --

def _gemm(fn_name, x, codes, scale_t, scale_shape, scale_dtype, y, workspace, stream):
    torch = _torch()
    _require(x, _bf16_like(torch), "x", 2)
    _require(codes, (torch.uint8,), "codes", 2)
    _require(scale_t, (scale_dtype,), "scales", 2)
    m, k = x.shape
    n, k2 = codes.shape
    if k != k2:
        raise ValueError(f"{fn_name}: x has K={k}, codes have K={k2}")
    if tuple(scale_t.shape) != scale_shape(n, k):
        raise ValueError(f"{fn_name}: scale grid {tuple(scale_t.shape)} != {scale_shape(n, k)}")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _require(y, _bf16_like(torch), "y", 2)
    if tuple(y.shape) != (m, n):
        raise ValueError(f"{fn_name}: y must be [{m}, {n}]")
    nbytes = int(lib().fp8w_gemm_workspace_bytes(n, k))
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _require(workspace, (torch.uint8,), "workspace", 1)
    _check(getattr(lib(), fn_name)(x.data_ptr(), m, codes.data_ptr(), scale_t.data_ptr(), n, k,
                                   y.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream_handle(stream)), fn_name)
    return y


def fp8w_gemm_block(x, codes, scales, y=None, workspace=None, stream=None):
    """y[m,n] = x[m,k] . deq(W)^T for any m: dequantize into ``workspace``
    (u8, fp8w_gemm_workspace_bytes(n, k) bytes; allocated when None), then a
    dense bf16 GEMM."""
    torch = _torch()
    return _gemm("fp8w_gemm_block", x, codes, scales, block_scale_shape, torch.float32, y,
                 workspace, stream)


def fp8w_gemm_mx(x, codes, e8m0, y=None, workspace=None, stream=None):
    torch = _torch()
    return _gemm("fp8w_gemm_mx", x, codes, e8m0, mx_scale_shape, torch.uint8, y, workspace, stream)


def fp8w_gemm_prepare() -> None:
    """Create the current device's rocBLAS handle for the GEMM calls (outside
    stream capture), so that GEMM calls can then be captured in a graph."""
    _check(lib().fp8w_gemm_prepare(), "fp8w_gemm_prepare")


# ------------------------------------------------------------------- W8A8 --

def fp8w_read_ceiling(buf, out=None, stream=None):
    """Read every byte of the contiguous GPU tensor ``buf`` once (measurement
    aid: the practical HBM read ceiling); returns the per-workgroup XOR words
    (2048 int32 by default), whose XOR is the XOR of the buffer's dwords."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("fp8w_read_ceiling: buf must be a contiguous GPU tensor")
    if out is None:
        out = torch.empty(2048, dtype=torch.int32, device=buf.device)
    _require(out, (torch.int32,), "out", 1)
    _check(lib().fp8w_read_ceiling(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                                   out.numel(), _stream_handle(stream)), "fp8w_read_ceiling")
    return out


def fp8w_quantize_act(x, codes=None, scale=None, workspace=None, stream=None):
    """Per-tensor activation quantization: bf16 x [m,k] -> (e4m3 codes u8
    [m,k], fp32 scale [1] on the device)."""
    torch = _torch()
    _require(x, _bf16_like(torch), "x", 2)
    m, k = x.shape
    if codes is None:
        codes = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(int(lib().fp8w_quantize_act_workspace_bytes()), dtype=torch.uint8,
                                device=x.device)
    _require(codes, (torch.uint8,), "codes", 2)
    _require(scale, (torch.float32,), "scale", 1)
    _require(workspace, (torch.uint8,), "workspace", 1)
    if tuple(codes.shape) != (m, k) or scale.numel() != 1:
        raise ValueError("fp8w_quantize_act: codes must be [m, k] and scale one element")
    _check(lib().fp8w_quantize_act(x.data_ptr(), m, k, codes.data_ptr(), scale.data_ptr(),
                                   workspace.data_ptr(), workspace.numel(), _stream_handle(stream)),
           "fp8w_quantize_act")
    return codes, scale


def fp8w_quantize_act_noalloc(x, codes, scale, stream=None):
    """fp8w_quantize_act with its partial maxima in the library's own device
    array: no workspace and no allocation.  The outputs are the caller's
    (codes u8 [m,k], scale fp32 [1])."""
    torch = _torch()
    _require(x, _bf16_like(torch), "x", 2)
    _require(codes, (torch.uint8,), "codes", 2)
    _require(scale, (torch.float32,), "scale", 1)
    m, k = x.shape
    if tuple(codes.shape) != (m, k) or scale.numel() != 1:
        raise ValueError("fp8w_quantize_act_noalloc: codes must be [m, k] and scale one element")
    _check(lib().fp8w_quantize_act_noalloc(x.data_ptr(), m, k, codes.data_ptr(), scale.data_ptr(),
                                           _stream_handle(stream)), "fp8w_quantize_act_noalloc")
    return codes, scale


def _gemv_w8a8(fn_name, x_codes, x_scale, codes, scale_t, scale_shape, scale_dtype, y, stream):
    torch = _torch()
    _require(x_codes, (torch.uint8,), "x_codes", 2)
    _require(x_scale, (torch.float32,), "x_scale", 1)
    _require(codes, (torch.uint8,), "codes", 2)
    _require(scale_t, (scale_dtype,), "scales", 2)
    m, k = x_codes.shape
    n, k2 = codes.shape
    if k != k2:
        raise ValueError(f"{fn_name}: x has K={k}, codes have K={k2}")
    if tuple(scale_t.shape) != scale_shape(n, k):
        raise ValueError(f"{fn_name}: scale grid {tuple(scale_t.shape)} != {scale_shape(n, k)}")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=codes.device)
    _require(y, _bf16_like(torch), "y", 2)
    _check(getattr(lib(), fn_name)(x_codes.data_ptr(), x_scale.data_ptr(), m, codes.data_ptr(),
                                   scale_t.data_ptr(), n, k, y.data_ptr(), _stream_handle(stream)),
           fn_name)
    return y


def fp8w_gemv_block_w8a8(x_codes, x_scale, codes, scales, y=None, stream=None):
    """y = x_scale * dec(x_codes) . deq(W)^T with fp8 x fp8 matrix cores."""
    torch = _torch()
    return _gemv_w8a8("fp8w_gemv_block_w8a8", x_codes, x_scale, codes, scales, block_scale_shape,
                      torch.float32, y, stream)


def fp8w_gemv_mx_w8a8(x_codes, x_scale, codes, e8m0, y=None, stream=None):
    torch = _torch()
    return _gemv_w8a8("fp8w_gemv_mx_w8a8", x_codes, x_scale, codes, e8m0, mx_scale_shape,
                      torch.uint8, y, stream)


# ---------------------------------------------------------------- grouped --

class GroupedPlan:
    """A group of independent GEMVs launched as one kernel.

    Holds the device table and references to every buffer it names, so the
    buffers stay alive as long as the plan.  ``y`` tensors are allocated here
    when not given.
    """

    def __init__(self, xs, codes, scales, ys=None, fmt: str = "block", route=ROUTE_AUTO):
        torch = _torch()
        if not (len(xs) == len(codes) == len(scales)) or not xs:
            raise ValueError("xs, codes and scales must be non-empty lists of equal length")
        fmt_id = _format_id(fmt)
        sdt, sshape = _scale_dtype(torch, fmt), (lambda n, k: scale_shape(fmt, n, k))
        m = int(xs[0].shape[0])
        if ys is None:
            ys = [torch.empty((m, int(c.shape[0])), dtype=torch.bfloat16, device=c.device) for c in codes]
        descs = (GemvDesc * len(xs))()
        for i, (x, c, s, y) in enumerate(zip(xs, codes, scales, ys)):
            _require(x, _bf16_like(torch), "x", 2)
            _require(c, (torch.uint8,), "codes", 2)
            _require(s, (sdt,), "scales", len(sshape(1, 16)))
            _require(y, _bf16_like(torch), "y", 2)
            n, k = c.shape
            if x.shape[0] != m or x.shape[1] != k or tuple(s.shape) != sshape(n, k) \
                    or tuple(y.shape) != (m, n):
                raise ValueError(f"grouped GEMV {i}: inconsistent shapes")
            descs[i] = GemvDesc(x.data_ptr(), c.data_ptr(), s.data_ptr(), y.data_ptr(), n, k)
        nbytes = int(lib().fp8w_grouped_table_bytes(len(xs)))
        self.table = torch.empty(nbytes, dtype=torch.uint8, device=codes[0].device)
        self.plan = GroupedPlanC()
        _check(lib().fp8w_grouped_plan_init(descs, len(xs), m, fmt_id, int(route),
                                            self.table.data_ptr(), ctypes.byref(self.plan)),
               "fp8w_grouped_plan_init")
        self.xs, self.codes, self.scales, self.ys = list(xs), list(codes), list(scales), list(ys)
        self.m, self.fmt = m, fmt

    @property
    def blocks(self) -> int:
        return int(self.plan.blocks)

    @property
    def route(self) -> int:
        return int(self.plan.route)


def fp8w_grouped_plan_init(xs, codes, scales, ys=None, fmt="block", route=ROUTE_AUTO) -> GroupedPlan:
    """Validate a group of GEMVs and write its device table (set-up call)."""
    return GroupedPlan(xs, codes, scales, ys, fmt, route)


def fp8w_gemv_grouped(plan: GroupedPlan, stream=None):
    """Enqueue every GEMV of ``plan`` in one launch; returns the ``y`` list."""
    _check(lib().fp8w_gemv_grouped(ctypes.byref(plan.plan), _stream_handle(stream)),
           "fp8w_gemv_grouped")
    return plan.ys


# ------------------------------------------------------- grouped quantize --

class QuantPlan:
    """Many weights quantized by one kernel launch (load time).

    Holds the device table and references to every buffer it names; codes
    and scales are allocated here when not given."""

    def __init__(self, ws, fmt: str = "block", codes=None, scales=None):
        torch = _torch()
        if not ws:
            raise ValueError("ws must be a non-empty list of bf16 [n, k] weights")
        fid = _format_id(fmt)
        if codes is None:
            codes = [torch.empty(tuple(w.shape), dtype=torch.uint8, device=w.device) for w in ws]
        if scales is None:
            scales = [torch.empty(scale_shape(fmt, *w.shape), dtype=_scale_dtype(torch, fmt), device=w.device)
                      for w in ws]
        if not (len(ws) == len(codes) == len(scales)):
            raise ValueError("ws, codes and scales must have equal lengths")
        descs = (QuantDesc * len(ws))()
        for i, (w, c, sc) in enumerate(zip(ws, codes, scales)):
            _require(w, _bf16_like(torch), "w", 2)
            _require(c, (torch.uint8,), "codes", 2)
            n, k = w.shape
            if tuple(c.shape) != (n, k):
                raise ValueError(f"grouped quantize {i}: codes shape {tuple(c.shape)} != {(n, k)}")
            _check_scales(torch, fmt, sc, n, k, "fp8w_quant_plan_init")
            descs[i] = QuantDesc(w.data_ptr(), c.data_ptr(), sc.data_ptr(), n, k)
        nbytes = int(lib().fp8w_quant_table_bytes(len(ws)))
        self.table = torch.empty(nbytes, dtype=torch.uint8, device=ws[0].device)
        self.plan = QuantPlanC()
        _check(lib().fp8w_quant_plan_init(descs, len(ws), fid, self.table.data_ptr(), ctypes.byref(self.plan)),
               "fp8w_quant_plan_init")
        self.ws, self.codes, self.scales, self.fmt = list(ws), list(codes), list(scales), fmt

    @property
    def blocks(self) -> int:
        return int(self.plan.blocks)


def fp8w_quant_plan_init(ws, fmt="block", codes=None, scales=None) -> QuantPlan:
    """Validate a group of weights to quantize and write its device table
    (set-up call)."""
    return QuantPlan(ws, fmt, codes, scales)


def fp8w_quantize_grouped(plan: QuantPlan, stream=None):
    """Enqueue the quantization of every weight of ``plan`` in one launch;
    returns (codes list, scales list)."""
    _check(lib().fp8w_quantize_grouped(ctypes.byref(plan.plan), _stream_handle(stream)),
           "fp8w_quantize_grouped")
    return plan.codes, plan.scales


# ----------------------------------------------------------- tagged weight --

BLOCK128, MX32, BLOCK128_BF16, ROW, TENSOR = "block128", "mx32", "block128_bf16", "row", "tensor"
_FMT_OF = {BLOCK128: "block", MX32: "mx", BLOCK128_BF16: "block_bf16", ROW: "row", TENSOR: "tensor"}


@dataclass
class Fp8Weight:
    """Quantized weight with its scale format fixed at construction.

    ``fmt`` is one of block128 (fp32 per 128x128 tile), mx32 (e8m0 per 32
    along K), block128_bf16, row (fp32 per row) and tensor (one fp32)."""
    codes: object
    scales: object
    n: int
    k: int
    fmt: str

    @classmethod
    def quantize(cls, w, fmt: str = BLOCK128, stream=None) -> "Fp8Weight":
        if fmt not in _FMT_OF:
            raise ValueError(f"unknown scale format {fmt!r}")
        c, s = fp8w_quantize(w, _FMT_OF[fmt], stream=stream)
        return cls(c, s, int(w.shape[0]), int(w.shape[1]), fmt)

    @property
    def format(self) -> str:
        """The C ABI's name of the scale format."""
        return _FMT_OF[self.fmt]

    def check_format(self) -> None:
        """The single place that decides which scale layout a weight carries."""
        torch = _torch()
        if self.fmt not in _FMT_OF:
            raise ValueError(f"Fp8Weight: unknown format {self.fmt!r}")
        f = _FMT_OF[self.fmt]
        if self.scales.dtype != _scale_dtype(torch, f) or tuple(self.scales.shape) != scale_shape(f, self.n, self.k):
            raise ValueError(f"Fp8Weight: scales do not match format {self.fmt!r}")

    def gemv(self, x, y=None, route=ROUTE_AUTO, stream=None):
        self.check_format()
        return fp8w_gemv(x, self.codes, self.scales, self.format, y, route, stream)

    def dequantize(self, w=None, stream=None):
        self.check_format()
        return fp8w_dequantize(self.codes, self.scales, self.format, w, stream)

    def matmul(self, x, y=None, workspace=None, stream=None):
        """y = x . deq(W)^T for any m: the fused GEMV for m <= 32 (the
        blockwise page's decode routing, Summary), dequantize + dense GEMM
        above."""
        self.check_format()
        if int(x.shape[0]) <= MAX_M:
            return self.gemv(x, y, ROUTE_AUTO, stream)
        return fp8w_gemm(x, self.codes, self.scales, self.format, y, workspace, stream)

    def gemv_w8a8(self, x_codes, x_scale, y=None, stream=None):
        self.check_format()
        return fp8w_gemv_w8a8(x_codes, x_scale, self.codes, self.scales, self.format, y, stream)
