"""CPU oracle for the FP8 weight path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it: the oracle is plain C (``fp8w_oracle.c``, built with
gcc, no HIP headers) driven through ctypes on numpy arrays.

What each function computes, and which passage of the pages it follows, is
stated in ``fp8w_oracle.c``.  In short:

* ``e4m3_decode`` / ``e4m3_encode``: OCP OFP8 E4M3 ("fn") decode, and round to
  nearest with ties to the even code, saturating at +-448, sign kept.
* ``quantize_block``: one fp32 scale per 128x128 tile, ``scale = amax/448``,
  ``code = enc(w/scale)`` with fp32 IEEE divisions.
* ``quantize_mx``: one e8m0 byte per 32 elements along K, exponent
  ``ceil(log2(amax/448))`` clamped to [-127, 127] with bias 127,
  ``code = enc(w * 2^-e)``, processed row-chunked (32 MiB fp32 transient).
* ``dequant_block`` / ``dequant_mx``: the exact fp64 dequantized weight.
* ``gemv_block_f64`` / ``gemv_mx_f64``: ``y = x . deq(W)^T`` and the bound
  ``|x| . |deq(W)|^T``, both in fp64, optionally for a subset of rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8w_oracle.c")
# FP8W_ORACLE_LIB names another build of the oracle to load instead (the
# mutation test loads deliberately broken builds through it, to show that
# the pins catch each planted mistake).
_LIB = os.environ.get("FP8W_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

OK, ERR_ARG, ERR_NONFINITE, ERR_NOMEM = 0, 1, 2, 3
TILE = 128
MX_GROUP = 32


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source into the shared library ``out`` with gcc
    (no fast-math, fp contraction off: every fp32 operation is the IEEE one)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``fp8w_oracle.c`` into ``liboracle.so`` (or the library named
    by FP8W_ORACLE_LIB)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    return compile_source(_SRC, _LIB)


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        sig = {
            "oracle_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
            "oracle_e4m3_encode_array": (None, [P, I64, P]),
            "oracle_e4m3_decode_array": (None, [P, I64, P]),
            "oracle_bf16_to_float": (ctypes.c_float, [ctypes.c_uint16]),
            "oracle_set_threads": (None, [ctypes.c_int]),
            "oracle_max_threads": (ctypes.c_int, []),
            "oracle_block_scale_count": (I64, [I64, I64]),
            "oracle_mx_scale_count": (I64, [I64, I64]),
            "oracle_quantize_block": (ctypes.c_int, [P, I64, I64, P, P]),
            "oracle_e8m0_exponent": (ctypes.c_int, [ctypes.c_float]),
            "oracle_e8m0_exponent_array": (None, [P, I64, P]),
            "oracle_mx_default_chunk_rows": (I64, [I64]),
            "oracle_quantize_mx": (ctypes.c_int, [P, I64, I64, P, P, I64]),
            "oracle_dequant_block": (ctypes.c_int, [P, P, I64, I64, P]),
            "oracle_dequant_mx": (ctypes.c_int, [P, P, I64, I64, P]),
            "oracle_round_bf16": (ctypes.c_uint16, [ctypes.c_double]),
            "oracle_round_bf16_array": (None, [P, I64, P]),
            "oracle_dequant_block_bf16": (ctypes.c_int, [P, P, I64, I64, P]),
            "oracle_dequant_mx_bf16": (ctypes.c_int, [P, P, I64, I64, P]),
            "oracle_quantize_act_tensor": (ctypes.c_int, [P, I64, I64, P, P]),
            "oracle_quantize_block_bf16": (ctypes.c_int, [P, I64, I64, P, P]),
            "oracle_quantize_row": (ctypes.c_int, [P, I64, I64, P, P]),
            "oracle_dequant_format_bf16": (ctypes.c_int, [P, P, ctypes.c_int, I64, I64, P]),
            "oracle_gemv_format_f64": (ctypes.c_int, [P, I64, P, P, ctypes.c_int, I64, I64, P, I64, P, P]),
            "oracle_gemv_w8a8_block_f64": (ctypes.c_int, [P, ctypes.c_float, I64, P, P, I64, I64, P, I64, P, P]),
            "oracle_gemv_w8a8_mx_f64": (ctypes.c_int, [P, ctypes.c_float, I64, P, P, I64, I64, P, I64, P, P]),
            "oracle_gemv_block_f64": (ctypes.c_int, [P, I64, P, P, I64, I64, P, I64, P, P]),
            "oracle_gemv_mx_f64": (ctypes.c_int, [P, I64, P, P, I64, I64, P, I64, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != OK:
        names = {ERR_ARG: "bad argument", ERR_NONFINITE: "non-finite input",
                 ERR_NOMEM: "out of memory"}
        raise OracleError(f"{what}: {names.get(rc, rc)}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def set_threads(threads: int) -> None:
    _load().oracle_set_threads(int(threads))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ codec --

def e4m3_decode(codes) -> np.ndarray:
    c = _as(np.asarray(codes, dtype=np.uint8), np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(q) -> np.ndarray:
    a = _as(np.asarray(q, dtype=np.float32), np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(a), a.size, _ptr(out))
    return out


def e8m0_exponent(amax) -> np.ndarray:
    a = _as(np.asarray(amax, dtype=np.float32), np.float32)
    out = np.empty(a.shape, dtype=np.int32)
    _load().oracle_e8m0_exponent_array(_ptr(a), a.size, _ptr(out))
    return out


def block_scale_shape(n: int, k: int):
    return ((n + TILE - 1) // TILE, (k + TILE - 1) // TILE)


def mx_scale_shape(n: int, k: int):
    return (n, (k + MX_GROUP - 1) // MX_GROUP)


def mx_default_chunk_rows(k: int) -> int:
    return int(_load().oracle_mx_default_chunk_rows(int(k)))


# --------------------------------------------------------------- quantize --

def quantize_block(w_bf16: np.ndarray):
    """bf16 bits [n, k] (uint16) -> (codes uint8 [n, k], scales f32 grid)."""
    w = _as(w_bf16, np.uint16)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty(block_scale_shape(n, k), dtype=np.float32)
    _check(_load().oracle_quantize_block(_ptr(w), n, k, _ptr(codes), _ptr(scales)),
           "quantize_block")
    return codes, scales


def quantize_mx(w_bf16: np.ndarray, chunk_rows: int = 0):
    """bf16 bits [n, k] -> (codes uint8 [n, k], e8m0 uint8 [n, ceil(k/32)])."""
    w = _as(w_bf16, np.uint16)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    e8m0 = np.empty(mx_scale_shape(n, k), dtype=np.uint8)
    _check(_load().oracle_quantize_mx(_ptr(w), n, k, _ptr(codes), _ptr(e8m0),
                                      int(chunk_rows)), "quantize_mx")
    return codes, e8m0


def dequant_block(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = _as(codes, np.uint8)
    s = _as(scales, np.float32)
    n, k = c.shape
    if s.shape != block_scale_shape(n, k):
        raise ValueError("scale grid shape mismatch")
    out = np.empty((n, k), dtype=np.float64)
    _check(_load().oracle_dequant_block(_ptr(c), _ptr(s), n, k, _ptr(out)), "dequant_block")
    return out


def dequant_mx(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    c = _as(codes, np.uint8)
    e = _as(e8m0, np.uint8)
    n, k = c.shape
    if e.shape != mx_scale_shape(n, k):
        raise ValueError("e8m0 shape mismatch")
    out = np.empty((n, k), dtype=np.float64)
    _check(_load().oracle_dequant_mx(_ptr(c), _ptr(e), n, k, _ptr(out)), "dequant_mx")
    return out


def round_bf16(v) -> np.ndarray:
    """bf16 bit patterns nearest to fp64 values (ties to even, IEEE overflow)."""
    a = _as(np.asarray(v, dtype=np.float64), np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_round_bf16_array(_ptr(a), a.size, _ptr(out))
    return out


def dequant_block_bf16(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bf16 bits of fl32(dec(code) * scale), [n, k]."""
    c = _as(codes, np.uint8)
    s = _as(scales, np.float32)
    n, k = c.shape
    if s.shape != block_scale_shape(n, k):
        raise ValueError("scale grid shape mismatch")
    out = np.empty((n, k), dtype=np.uint16)
    _check(_load().oracle_dequant_block_bf16(_ptr(c), _ptr(s), n, k, _ptr(out)),
           "dequant_block_bf16")
    return out


def dequant_mx_bf16(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """bf16 bits of dec(code) * 2^(E - 127), [n, k]."""
    c = _as(codes, np.uint8)
    e = _as(e8m0, np.uint8)
    n, k = c.shape
    if e.shape != mx_scale_shape(n, k):
        raise ValueError("e8m0 shape mismatch")
    out = np.empty((n, k), dtype=np.uint16)
    _check(_load().oracle_dequant_mx_bf16(_ptr(c), _ptr(e), n, k, _ptr(out)),
           "dequant_mx_bf16")
    return out


# ------------------------------------------------------------------- GEMV --

def _gemv(fn, x_bf16, codes, scale_arr, rows):
    x = _as(x_bf16, np.uint16)
    c = _as(codes, np.uint8)
    m, k = x.shape
    n, k2 = c.shape
    if k != k2:
        raise ValueError("x and codes disagree on K")
    if rows is None:
        rows_arr, nrows, rows_ptr = None, n, None
    else:
        rows_arr = _as(np.asarray(rows, dtype=np.int64), np.int64)
        nrows, rows_ptr = rows_arr.size, _ptr(rows_arr)
    y = np.empty((m, nrows), dtype=np.float64)
    bound = np.empty((m, nrows), dtype=np.float64)
    _check(fn(_ptr(x), m, _ptr(c), _ptr(scale_arr), n, k, rows_ptr, nrows,
              _ptr(y), _ptr(bound)), "gemv")
    return y, bound


def gemv_block_f64(x_bf16, codes, scales, rows=None):
    """fp64 ``y = x . deq(W)^T`` and ``|x| . |deq(W)|^T`` ([m, len(rows)])."""
    s = _as(scales, np.float32)
    if s.shape != block_scale_shape(*np.shape(codes)):
        raise ValueError("scale grid shape mismatch")
    return _gemv(_load().oracle_gemv_block_f64, x_bf16, codes, s, rows)


def gemv_mx_f64(x_bf16, codes, e8m0, rows=None):
    e = _as(e8m0, np.uint8)
    if e.shape != mx_scale_shape(*np.shape(codes)):
        raise ValueError("e8m0 shape mismatch")
    return _gemv(_load().oracle_gemv_mx_f64, x_bf16, codes, e, rows)


# ---------------------------------------------------- other scale formats --

FORMATS = {"block": 0, "mx": 1, "block_bf16": 2, "row": 3, "tensor": 4}


def scale_shape(fmt: str, n: int, k: int):
    return {"block": block_scale_shape(n, k), "mx": mx_scale_shape(n, k),
            "block_bf16": block_scale_shape(n, k), "row": (n,), "tensor": (1,)}[fmt]


def scale_dtype(fmt: str):
    return {"block": np.float32, "mx": np.uint8, "block_bf16": np.uint16, "row": np.float32,
            "tensor": np.float32}[fmt]


def quantize_block_bf16(w_bf16: np.ndarray):
    """(codes u8 [n,k], bf16 scale bits u16 [ceil(n/128), ceil(k/128)])."""
    w = _as(w_bf16, np.uint16)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty(block_scale_shape(n, k), dtype=np.uint16)
    _check(_load().oracle_quantize_block_bf16(_ptr(w), n, k, _ptr(codes), _ptr(scales)),
           "quantize_block_bf16")
    return codes, scales


def quantize_row(w_bf16: np.ndarray):
    """(codes u8 [n,k], fp32 scales [n])."""
    w = _as(w_bf16, np.uint16)
    n, k = w.shape
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty((n,), dtype=np.float32)
    _check(_load().oracle_quantize_row(_ptr(w), n, k, _ptr(codes), _ptr(scales)), "quantize_row")
    return codes, scales


def quantize_format(w_bf16: np.ndarray, fmt: str):
    """Quantize in any format: (codes, scales as the format stores them)."""
    if fmt == "block":
        return quantize_block(w_bf16)
    if fmt == "mx":
        return quantize_mx(w_bf16)
    if fmt == "block_bf16":
        return quantize_block_bf16(w_bf16)
    if fmt == "row":
        return quantize_row(w_bf16)
    codes, scale = quantize_act_tensor(w_bf16)
    return codes, np.array([scale], dtype=np.float32)


def _format_scales(fmt, codes, scales):
    s = _as(scales, scale_dtype(fmt))
    if s.shape != scale_shape(fmt, *np.shape(codes)):
        raise ValueError(f"{fmt}: scale shape {s.shape} != {scale_shape(fmt, *np.shape(codes))}")
    return s


def dequant_format_bf16(codes, scales, fmt: str) -> np.ndarray:
    c = _as(codes, np.uint8)
    s = _format_scales(fmt, c, scales)
    n, k = c.shape
    out = np.empty((n, k), dtype=np.uint16)
    _check(_load().oracle_dequant_format_bf16(_ptr(c), _ptr(s), FORMATS[fmt], n, k, _ptr(out)),
           "dequant_format_bf16")
    return out


def gemv_format_f64(x_bf16, codes, scales, fmt: str, rows=None):
    x = _as(x_bf16, np.uint16)
    c = _as(codes, np.uint8)
    s = _format_scales(fmt, c, scales)
    m, k = x.shape
    n, k2 = c.shape
    if k != k2:
        raise ValueError("x and codes disagree on K")
    if rows is None:
        rows_arr, nrows, rows_ptr = None, n, None
    else:
        rows_arr = _as(np.asarray(rows, dtype=np.int64), np.int64)
        nrows, rows_ptr = rows_arr.size, _ptr(rows_arr)
    y = np.empty((m, nrows), dtype=np.float64)
    bound = np.empty((m, nrows), dtype=np.float64)
    _check(_load().oracle_gemv_format_f64(_ptr(x), m, _ptr(c), _ptr(s), FORMATS[fmt], n, k, rows_ptr,
                                          nrows, _ptr(y), _ptr(bound)), "gemv_format")
    return y, bound


# ------------------------------------------------------------- W8A8 path --

def quantize_act_tensor(x_bf16: np.ndarray):
    """Per-tensor activation quantization: (codes u8 [m,k], scale float)."""
    x = _as(x_bf16, np.uint16)
    m, k = x.shape
    codes = np.empty((m, k), dtype=np.uint8)
    scale = np.empty(1, dtype=np.float32)
    _check(_load().oracle_quantize_act_tensor(_ptr(x), m, k, _ptr(codes), _ptr(scale)),
           "quantize_act_tensor")
    return codes, float(scale[0])


def _gemv_w8a8(fn, xc, xs, codes, scale_arr, rows):
    xq = _as(xc, np.uint8)
    c = _as(codes, np.uint8)
    m, k = xq.shape
    n, k2 = c.shape
    if k != k2:
        raise ValueError("x codes and weight codes disagree on K")
    if rows is None:
        rows_arr, nrows, rows_ptr = None, n, None
    else:
        rows_arr = _as(np.asarray(rows, dtype=np.int64), np.int64)
        nrows, rows_ptr = rows_arr.size, _ptr(rows_arr)
    y = np.empty((m, nrows), dtype=np.float64)
    bound = np.empty((m, nrows), dtype=np.float64)
    _check(fn(_ptr(xq), float(xs), m, _ptr(c), _ptr(scale_arr), n, k, rows_ptr, nrows,
              _ptr(y), _ptr(bound)), "gemv_w8a8")
    return y, bound


def gemv_w8a8_block_f64(x_codes, x_scale, codes, scales, rows=None):
    """fp64 y = (dec(x_codes) * x_scale) . deq(W)^T and its magnitude bound."""
    s = _as(scales, np.float32)
    if s.shape != block_scale_shape(*np.shape(codes)):
        raise ValueError("scale grid shape mismatch")
    return _gemv_w8a8(_load().oracle_gemv_w8a8_block_f64, x_codes, x_scale, codes, s, rows)


def gemv_w8a8_mx_f64(x_codes, x_scale, codes, e8m0, rows=None):
    e = _as(e8m0, np.uint8)
    if e.shape != mx_scale_shape(*np.shape(codes)):
        raise ValueError("e8m0 shape mismatch")
    return _gemv_w8a8(_load().oracle_gemv_w8a8_mx_f64, x_codes, x_scale, codes, e, rows)


def gemv_tolerance(bound: np.ndarray) -> np.ndarray:
    """Allowed |y - y_ref|: 2^-7 * (|x| . |deq W|^T) + 1e-6 (elementwise)."""
    return np.ldexp(bound, -7) + 1e-6
