"""CPU oracle for the MX quantize -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its binding) never imports it, and it shares no code with them.

The arithmetic lives in ``mxq_oracle.c`` (plain C, built with gcc); this
module only compiles it on demand and passes numpy arrays across. Type names
used here: input ``"bf16"`` / ``"f16"``; output ``"e4m3fn"`` / ``"e5m2"`` /
``"e2m1"``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmxq_oracle.so")

IN_CODES = {"bf16": 0, "f16": 1}
OUT_CODES = {"e4m3fn": 0, "e5m2": 1, "e2m1": 2}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # MXQ_ORACLE_LIB names another build of mxq_oracle.c to load instead:
        # the mutation test points it at copies with a planted mistake
        path = os.environ.get("MXQ_ORACLE_LIB") or build(force=False)
        lib = ctypes.CDLL(path)
        c = ctypes
        P_u16, P_u8, P_f32, P_f64 = (c.POINTER(c.c_uint16), c.POINTER(c.c_uint8),
                                      c.POINTER(c.c_float), c.POINTER(c.c_double))
        lib.mxq_oracle_quantize.argtypes = [P_u16, c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_int,
                                            P_u8, P_u8]
        lib.mxq_oracle_quantize.restype = c.c_int
        lib.mxq_oracle_dequantize.argtypes = [P_u8, P_u8, c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_int,
                                              c.c_void_p]
        lib.mxq_oracle_dequantize.restype = c.c_int
        lib.mxq_oracle_f32_to_bf16_array.argtypes = [P_f32, c.c_int64, P_u16]
        lib.mxq_oracle_scaled_matmul.argtypes = [P_u8, P_u8, P_u8, P_u8, c.c_int64, c.c_int64, c.c_int64,
                                                 c.c_int, c.c_int, P_f64]
        lib.mxq_oracle_scaled_matmul.restype = c.c_int
        lib.mxq_oracle_scaled_matmul_quantize.argtypes = [P_u8, P_u8, P_u8, P_u8, c.c_int64, c.c_int64, c.c_int64,
                                                          c.c_int, c.c_int, c.c_int, c.c_int, P_u8, P_u8]
        lib.mxq_oracle_scaled_matmul_quantize.restype = c.c_int
        lib.mxq_oracle_quantize_axis.argtypes = [P_u16, c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_int,
                                                 c.c_int, P_u8, P_u8]
        lib.mxq_oracle_quantize_axis.restype = c.c_int
        lib.mxq_oracle_widen_array.argtypes = [P_u16, c.c_int64, c.c_int, P_f32]
        lib.mxq_oracle_narrow_array.argtypes = [P_f32, c.c_int64, c.c_int, P_u8]
        lib.mxq_oracle_prescale_array.argtypes = [P_f32, P_u8, c.c_int64, P_f32]
        lib.mxq_oracle_decode_array.argtypes = [P_u8, c.c_int64, c.c_int, P_f64]
        lib.mxq_oracle_e8m0.argtypes = [c.c_uint8, c.c_int]
        lib.mxq_oracle_e8m0.restype = c.c_uint8
        lib.mxq_oracle_emax.argtypes = [c.c_int]
        lib.mxq_oracle_emax.restype = c.c_int
        lib.mxq_oracle_block_max_exponent.argtypes = [P_f32, c.c_int64, c.c_int64, c.c_int64]
        lib.mxq_oracle_block_max_exponent.restype = c.c_uint8
        lib.mxq_oracle_lane_remap.argtypes = [c.c_int64, c.c_int64]
        lib.mxq_oracle_lane_remap.restype = c.c_int64
        lib.mxq_oracle_scale_slot.argtypes = [c.c_int64]
        lib.mxq_oracle_scale_slot.restype = c.c_int64
        lib.mxq_oracle_encode_e2m1.argtypes = [c.c_float]
        lib.mxq_oracle_encode_e2m1.restype = c.c_uint8
        lib.mxq_oracle_narrow.argtypes = [c.c_float, c.c_int]
        lib.mxq_oracle_narrow.restype = c.c_uint8
        _lib = lib
        return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def data_shape(P: int, F: int, out_dtype: str):
    return (P, F // 2) if out_dtype == "e2m1" else (P, F)


LAYOUTS = {"image": 0, "dense": 1}


def scale_shape(P: int, F: int, layout: str = "image"):
    return (P, F // 4) if layout == "image" else (P // 8, F // 4)


def quantize(x: np.ndarray, in_dtype: str, out_dtype: str, alt_emax: bool = False,
             image: np.ndarray | None = None, layout: str = "image"):
    """Quantize a [P, F] array of bf16/f16 bit patterns (uint16).

    Returns ``(data, image)``: data is uint8 [P, F] (FP8) or [P, F/2] (FP4);
    image is the uint8 [P, F/4] scale image, of which only the rows that the
    scale placement names are written (the others keep the contents of
    ``image``, zeros when it is not given); with ``layout="dense"`` it is the
    fully written [P/8, F/4] scale array.
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    P, F = x.shape
    data = np.zeros(data_shape(P, F, out_dtype), dtype=np.uint8)
    if image is None:
        image = np.zeros(scale_shape(P, F, layout), dtype=np.uint8)
    else:
        image = np.array(image, dtype=np.uint8, copy=True, order="C")
    rc = lib.mxq_oracle_quantize(_ptr(x, ctypes.c_uint16), P, F, IN_CODES[in_dtype], OUT_CODES[out_dtype],
                                 int(bool(alt_emax)), LAYOUTS[layout], _ptr(data, ctypes.c_uint8),
                                 _ptr(image, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("oracle quantize rejected the call (status %d)" % rc)
    return data, image


def quantize_axis(x: np.ndarray, in_dtype: str, out_dtype: str, dim: int, alt_emax: bool = False,
                  layout: str = "image"):
    """Quantize a row-major [R, C] array of bf16/f16 bit patterns with
    32-element blocks along axis ``dim`` (-1: along rows, K = C; -2: down
    columns, K = R). Returns ``(data, scale)`` in the partition-major layout
    :func:`quantize` produces for the [K/4, 4*O] view (O the other extent)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, C = x.shape
    d = dim + 2 if dim < 0 else dim
    K, O = (C, R) if d == 1 else (R, C)
    if d not in (0, 1) or K % 32:
        raise ValueError("dim must be -1 or -2 and the block axis a multiple of 32")
    P, F = K // 4, 4 * O
    data = np.zeros(data_shape(P, F, out_dtype), dtype=np.uint8)
    scale = np.zeros(scale_shape(P, F, layout), dtype=np.uint8)
    rc = lib.mxq_oracle_quantize_axis(_ptr(x, ctypes.c_uint16), R, C, IN_CODES[in_dtype], OUT_CODES[out_dtype], dim,
                                      int(bool(alt_emax)), LAYOUTS[layout], _ptr(data, ctypes.c_uint8),
                                      _ptr(scale, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("oracle quantize_axis rejected the call (status %d)" % rc)
    return data, scale


RES_CODES = {"f32": 0, "bf16": 1}


def dequantize(data: np.ndarray, image: np.ndarray, P: int, F: int, out_dtype: str,
               res_dtype: str = "f32", layout: str = "image") -> np.ndarray:
    """Decode [P, F] values from packed data and the scale image (or dense
    scale array): float32, or bf16 bit patterns (uint16) for
    ``res_dtype="bf16"``."""
    lib = _load()
    data = np.ascontiguousarray(data, dtype=np.uint8)
    image = np.ascontiguousarray(image, dtype=np.uint8)
    out = np.empty((P, F), dtype=np.float32 if res_dtype == "f32" else np.uint16)
    rc = lib.mxq_oracle_dequantize(_ptr(data, ctypes.c_uint8), _ptr(image, ctypes.c_uint8), P, F,
                                   OUT_CODES[out_dtype], RES_CODES[res_dtype], LAYOUTS[layout], out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle dequantize rejected the call (status %d)" % rc)
    return out


def scaled_matmul(lhs: np.ndarray, lhs_scale: np.ndarray, rhs: np.ndarray, rhs_scale: np.ndarray,
                  fmt: str, layout: str = "image") -> np.ndarray:
    """out[m][n] = sum_k L[k][m] * R[k][n] in float64, for operands quantized
    as lhs [P, 4M] and rhs [P, 4N] (x4 containers unpacked along k = 4p + j)."""
    lib = _load()
    lhs = np.ascontiguousarray(lhs, dtype=np.uint8)
    rhs = np.ascontiguousarray(rhs, dtype=np.uint8)
    ls = np.ascontiguousarray(lhs_scale, dtype=np.uint8)
    rs = np.ascontiguousarray(rhs_scale, dtype=np.uint8)
    P = lhs.shape[0]
    M, N = lhs.shape[1] // 4, rhs.shape[1] // 4
    if rhs.shape[0] != P:
        raise ValueError("lhs and rhs must share P")
    out = np.empty((M, N), dtype=np.float64)
    rc = lib.mxq_oracle_scaled_matmul(_ptr(lhs, ctypes.c_uint8), _ptr(ls, ctypes.c_uint8), _ptr(rhs, ctypes.c_uint8),
                                      _ptr(rs, ctypes.c_uint8), P, M, N, OUT_CODES[fmt], LAYOUTS[layout],
                                      _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle scaled_matmul rejected the call (status %d)" % rc)
    return out


def scaled_matmul_quantize(lhs: np.ndarray, lhs_scale: np.ndarray, rhs: np.ndarray, rhs_scale: np.ndarray,
                           fmt: str, out_dtype: str, alt_emax: bool = False, layout: str = "image"):
    """quantize(bf16(scaled_matmul(...))): the M x N matmul result rounded to
    fp32 then bf16 and quantized (8 x 4 blocks over rows m, columns n).
    Returns ``(data, scale)`` shaped as :func:`quantize` would for P = M,
    F = N; operand and result scales share ``layout``."""
    lib = _load()
    lhs = np.ascontiguousarray(lhs, dtype=np.uint8)
    rhs = np.ascontiguousarray(rhs, dtype=np.uint8)
    ls = np.ascontiguousarray(lhs_scale, dtype=np.uint8)
    rs = np.ascontiguousarray(rhs_scale, dtype=np.uint8)
    P = lhs.shape[0]
    M, N = lhs.shape[1] // 4, rhs.shape[1] // 4
    if rhs.shape[0] != P:
        raise ValueError("lhs and rhs must share P")
    data = np.zeros(data_shape(M, N, out_dtype), dtype=np.uint8)
    scale = np.zeros(scale_shape(M, N, layout), dtype=np.uint8)
    rc = lib.mxq_oracle_scaled_matmul_quantize(_ptr(lhs, ctypes.c_uint8), _ptr(ls, ctypes.c_uint8),
                                               _ptr(rhs, ctypes.c_uint8), _ptr(rs, ctypes.c_uint8), P, M, N,
                                               OUT_CODES[fmt], OUT_CODES[out_dtype], int(bool(alt_emax)),
                                               LAYOUTS[layout], _ptr(data, ctypes.c_uint8),
                                               _ptr(scale, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("oracle scaled_matmul_quantize rejected the call (status %d)" % rc)
    return data, scale


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    lib = _load()
    f = np.ascontiguousarray(f, dtype=np.float32).ravel()
    out = np.empty(f.size, dtype=np.uint16)
    lib.mxq_oracle_f32_to_bf16_array(_ptr(f, ctypes.c_float), f.size, _ptr(out, ctypes.c_uint16))
    return out


def widen(h: np.ndarray, in_dtype: str) -> np.ndarray:
    lib = _load()
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    out = np.empty(h.size, dtype=np.float32)
    lib.mxq_oracle_widen_array(_ptr(h, ctypes.c_uint16), h.size, IN_CODES[in_dtype], _ptr(out, ctypes.c_float))
    return out


def narrow(y: np.ndarray, out_dtype: str) -> np.ndarray:
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    out = np.empty(y.size, dtype=np.uint8)
    lib.mxq_oracle_narrow_array(_ptr(y, ctypes.c_float), y.size, OUT_CODES[out_dtype], _ptr(out, ctypes.c_uint8))
    return out


def prescale(x: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    e = np.ascontiguousarray(np.broadcast_to(e8m0, x.shape), dtype=np.uint8).ravel()
    out = np.empty(x.size, dtype=np.float32)
    lib.mxq_oracle_prescale_array(_ptr(x, ctypes.c_float), _ptr(e, ctypes.c_uint8), x.size, _ptr(out, ctypes.c_float))
    return out


def decode(codes: np.ndarray, out_dtype: str) -> np.ndarray:
    lib = _load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    out = np.empty(codes.size, dtype=np.float64)
    lib.mxq_oracle_decode_array(_ptr(codes, ctypes.c_uint8), codes.size, OUT_CODES[out_dtype],
                                _ptr(out, ctypes.c_double))
    return out


def e8m0(max_exponent: int, emax_bias: int) -> int:
    return int(_load().mxq_oracle_e8m0(max_exponent, emax_bias))


def emax(out_dtype: str) -> int:
    return int(_load().mxq_oracle_emax(OUT_CODES[out_dtype]))


def block_max_exponent(xf32: np.ndarray, row_group: int, col_block: int) -> int:
    xf32 = np.ascontiguousarray(xf32, dtype=np.float32)
    return int(_load().mxq_oracle_block_max_exponent(_ptr(xf32, ctypes.c_float), xf32.shape[1], row_group,
                                                     col_block))


def lane_remap(index: int, stride: int) -> int:
    return int(_load().mxq_oracle_lane_remap(index, stride))


def scale_slot(i: int) -> int:
    return int(_load().mxq_oracle_scale_slot(i))


def encode_e2m1(y: float) -> int:
    return int(_load().mxq_oracle_encode_e2m1(y))
