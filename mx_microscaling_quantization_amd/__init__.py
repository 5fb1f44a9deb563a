"""MX (microscaling) quantize on AMD MI355X -- Python binding of ``libmxq.so``.

A thin ctypes layer over the C ABI declared in ``include/mxq.h``: it maps
torch dtypes to the ABI's codes, allocates outputs with torch when the caller
gives none, and passes raw device pointers and the current HIP stream. Every
step of the quantize runs in the library's HIP kernels; there is no fallback.
If ``libmxq.so`` is missing or cannot be loaded, importing the functions below
raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
import threading

import torch  # loaded first so that the library binds to torch's HIP runtime

__all__ = [
    "IN_DTYPES", "OUT_DTYPES", "RES_DTYPES", "MXQError", "quantize", "dequantize", "quantize_axis", "scaled_matmul",
    "scaled_matmul_quantize", "data_bytes", "scale_image_bytes", "result_bytes", "data_shape", "scale_image_shape",
    "axis_view_shape", "logical_scale_view", "status_string", "library_path", "load",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmxq.so"

IN_DTYPES = {torch.bfloat16: 0, torch.float16: 1}
OUT_DTYPES = {"e4m3fn": 0, "e5m2": 1, "e2m1": 2}
RES_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
FLAG_ALT_EMAX = 1
FLAG_DENSE_SCALE = 2
ABI_VERSION = 1

_lock = threading.Lock()
_lib = None


class MXQError(RuntimeError):
    """A non-zero status from the library (``status`` holds the code)."""

    def __init__(self, status: int, message: str):
        super().__init__("mxq status %d: %s" % (status, message))
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load():
    """Load ``libmxq.so`` (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise ImportError("%s is not built; run `python -m mx_microscaling_quantization_amd._build` (hipcc, gfx950) first" % path)
        lib = ctypes.CDLL(path)
        c = ctypes
        lib.mxq_quantize.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_void_p,
                                     c.c_void_p, c.c_void_p]
        lib.mxq_quantize.restype = c.c_int
        lib.mxq_quantize_ex.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_uint,
                                        c.c_void_p, c.c_void_p, c.c_void_p]
        lib.mxq_quantize_ex.restype = c.c_int
        lib.mxq_dequantize_ex.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int, c.c_int,
                                          c.c_uint, c.c_void_p, c.c_void_p]
        lib.mxq_dequantize_ex.restype = c.c_int
        lib.mxq_scaled_matmul.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64, c.c_int64,
                                          c.c_int64, c.c_int, c.c_int, c.c_uint, c.c_void_p, c.c_void_p]
        lib.mxq_scaled_matmul.restype = c.c_int
        lib.mxq_scaled_matmul_quantize.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_void_p, c.c_int64,
                                                   c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_uint, c.c_void_p,
                                                   c.c_void_p, c.c_void_p]
        lib.mxq_scaled_matmul_quantize.restype = c.c_int
        lib.mxq_quantize_axis.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_int, c.c_int, c.c_int, c.c_uint,
                                          c.c_void_p, c.c_void_p, c.c_void_p]
        lib.mxq_quantize_axis.restype = c.c_int
        lib.mxq_scale_bytes.argtypes = [c.c_int64, c.c_int64, c.c_uint]
        lib.mxq_scale_bytes.restype = c.c_size_t
        lib.mxq_data_bytes.argtypes = [c.c_int64, c.c_int64, c.c_int]
        lib.mxq_data_bytes.restype = c.c_size_t
        lib.mxq_scale_image_bytes.argtypes = [c.c_int64, c.c_int64]
        lib.mxq_scale_image_bytes.restype = c.c_size_t
        lib.mxq_dequantize.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int, c.c_int,
                                       c.c_void_p, c.c_void_p]
        lib.mxq_dequantize.restype = c.c_int
        lib.mxq_result_bytes.argtypes = [c.c_int64, c.c_int64, c.c_int]
        lib.mxq_result_bytes.restype = c.c_size_t
        lib.mxq_status_string.argtypes = [c.c_int]
        lib.mxq_status_string.restype = c.c_char_p
        lib.mxq_abi_version.argtypes = []
        lib.mxq_abi_version.restype = c.c_int
        if lib.mxq_abi_version() != ABI_VERSION:
            raise ImportError("libmxq.so ABI %d, binding expects %d" % (lib.mxq_abi_version(), ABI_VERSION))
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().mxq_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise MXQError(status, status_string(status))


def _out_code(out_dtype: str) -> int:
    try:
        return OUT_DTYPES[out_dtype]
    except KeyError:
        raise MXQError(2, "output element type must be one of %s" % sorted(OUT_DTYPES)) from None


# torch's accessor for the raw handle of a device's current stream (what its
# own kernels launch on), when it has one; the public route costs more per
# call
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, device: torch.device) -> int:
    """The raw HIP stream handle to enqueue on: ``stream``'s, else the current
    stream of ``device``."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_current_stream is not None:
        return _raw_current_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _call_on(device: torch.device, fn, *args) -> int:
    """Call ``fn(*args)`` with ``device`` current (the library launches on
    the current device), entering a device context only when it is not."""
    if torch.cuda.current_device() == device.index:
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


@functools.lru_cache(maxsize=256)
def _data_nbytes(P: int, F: int, code: int) -> int:
    return int(load().mxq_data_bytes(P, F, code))


@functools.lru_cache(maxsize=256)
def _scale_nbytes(P: int, F: int, flags: int) -> int:
    return int(load().mxq_scale_bytes(P, F, flags))


def _check_out_buffer(name: str, t: torch.Tensor, nbytes: int, device: torch.device) -> None:
    """An output the library writes through a raw pointer: contiguous, on
    ``device``, and at least ``nbytes`` long (its element type is not read)."""
    if t.device != device or not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ValueError("%s must be a contiguous buffer of >= %d bytes on %s" % (name, nbytes, device))


def data_bytes(P: int, F: int, out_dtype: str) -> int:
    return int(load().mxq_data_bytes(P, F, _out_code(out_dtype)))


def scale_image_bytes(P: int, F: int) -> int:
    return int(load().mxq_scale_image_bytes(P, F))


def result_bytes(P: int, F: int, res_dtype: torch.dtype) -> int:
    return int(load().mxq_result_bytes(P, F, RES_DTYPES[res_dtype]))


def data_shape(P: int, F: int, out_dtype: str):
    """uint8 shape of the data output: [P, F] (FP8) or [P, F/2] (FP4)."""
    return (P, F // 2) if out_dtype == "e2m1" else (P, F)


def scale_image_shape(P: int, F: int, dense_scale: bool = False):
    """uint8 shape of the scale output: the [P, F/4] image, or [P/8, F/4]
    with ``dense_scale``."""
    return (P // 8, F // 4) if dense_scale else (P, F // 4)


def logical_scale_view(image: torch.Tensor) -> torch.Tensor:
    """View [P/32, 4, F/4] of the written rows of a scale image (P % 32 == 0):
    element [q, j, c] is the E8M0 of row group 4q + j, column block c."""
    P, C = image.shape
    if P % 32:
        raise ValueError("logical_scale_view needs P % 32 == 0")
    return image.view(P // 32, 32, C)[:, :4, :]


def quantize(x: torch.Tensor, out_dtype: str = "e4m3fn", data_out: torch.Tensor | None = None,
             scale_out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None,
             alt_emax: bool = False, dense_scale: bool = False):
    """MX-quantize a contiguous [P, F] bf16/f16 CUDA (HIP) tensor.

    Returns ``(data, scale)`` as uint8 tensors: data [P, F] (FP8) or
    [P, F/2] (FP4); the scale image [P, F/4], of which rows
    (i mod 4) + 32 * floor(i / 4) hold row group i's E8M0 bytes and the other
    rows keep whatever ``scale_out`` held -- or, with ``dense_scale``, the
    dense [P/8, F/4] scale array. ``alt_emax`` selects the EMAX - 1 bias.
    The kernel is enqueued on ``stream`` (default: the current stream of x's
    device).
    """
    lib = load()
    if x.dtype not in IN_DTYPES:
        raise MXQError(1, "input element type must be bfloat16 or float16, got %s" % x.dtype)
    code = _out_code(out_dtype)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [P, F]")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (row pitch F)")
    P, F = x.shape
    if data_out is None:
        data_out = torch.empty(data_shape(P, F, out_dtype), dtype=torch.uint8, device=x.device)
    flags = (FLAG_ALT_EMAX if alt_emax else 0) | (FLAG_DENSE_SCALE if dense_scale else 0)
    if scale_out is None:
        scale_out = torch.empty(scale_image_shape(P, F, dense_scale), dtype=torch.uint8, device=x.device)
    _check_out_buffer("data_out", data_out, _data_nbytes(P, F, code), x.device)
    _check_out_buffer("scale_out", scale_out, _scale_nbytes(P, F, flags), x.device)
    sh = _stream_handle(stream, x.device)
    if flags == 0:    # the contract's own entry point
        _check(_call_on(x.device, lib.mxq_quantize, x.data_ptr(), P, F, IN_DTYPES[x.dtype], code,
                        data_out.data_ptr(), scale_out.data_ptr(), sh))
    else:
        _check(_call_on(x.device, lib.mxq_quantize_ex, x.data_ptr(), P, F, IN_DTYPES[x.dtype], code, flags,
                        data_out.data_ptr(), scale_out.data_ptr(), sh))
    return data_out, scale_out


def dequantize(data: torch.Tensor, scale_image: torch.Tensor, out_dtype: str = "e4m3fn",
               res_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
               stream: torch.cuda.Stream | None = None, dense_scale: bool = False) -> torch.Tensor:
    """Decode MX data back to [P, F] float32 or bfloat16.

    ``data`` is the uint8 data output of :func:`quantize` for format
    ``out_dtype`` ([P, F] FP8 or [P, F/2] FP4) and ``scale_image`` its
    [P, F/4] scale image (or, with ``dense_scale``, its [P/8, F/4] scale
    array). Each result is decode(code) * 2^(E8M0 - 127), rounded once to
    float32 (then nearest-even to bfloat16).
    """
    lib = load()
    code = _out_code(out_dtype)
    if res_dtype not in RES_DTYPES:
        raise MXQError(10, "result type must be float32 or bfloat16, got %s" % res_dtype)
    if data.dim() != 2 or scale_image.dim() != 2:
        raise ValueError("data and scale_image must be 2-D")
    if not data.is_cuda or scale_image.device != data.device:
        raise ValueError("data and scale_image must be device tensors on one device")
    if not (data.is_contiguous() and scale_image.is_contiguous()):
        raise ValueError("data and scale_image must be contiguous")
    if data.dtype != torch.uint8 or scale_image.dtype != torch.uint8:
        raise ValueError("data and scale_image must be uint8 (the bytes quantize wrote)")
    P = data.shape[0]
    F = scale_image.shape[1] * 4
    if tuple(data.shape) != data_shape(P, F, out_dtype) or \
            tuple(scale_image.shape) != scale_image_shape(P, F, dense_scale):
        raise ValueError("data %s / scale_image %s do not describe one [P, F] tensor in format %s"
                         % (tuple(data.shape), tuple(scale_image.shape), out_dtype))
    if out is None:
        out = torch.empty((P, F), dtype=res_dtype, device=data.device)
    elif out.dtype != res_dtype or tuple(out.shape) != (P, F) or not out.is_contiguous() or out.device != data.device:
        raise ValueError("out must be a contiguous [%d, %d] %s tensor on %s" % (P, F, res_dtype, data.device))
    sh = _stream_handle(stream, data.device)
    _check(_call_on(data.device, lib.mxq_dequantize_ex, data.data_ptr(), scale_image.data_ptr(), P, F, code,
                    RES_DTYPES[res_dtype], FLAG_DENSE_SCALE if dense_scale else 0, out.data_ptr(), sh))
    return out


def _check_operands(lhs, lhs_scale, rhs, rhs_scale, dense_scale):
    for t in (lhs, lhs_scale, rhs, rhs_scale):
        if t.dim() != 2 or t.dtype != torch.uint8 or not t.is_contiguous() or t.device != lhs.device or not t.is_cuda:
            raise ValueError("operands must be contiguous 2-D uint8 device tensors on one device")
    P = lhs.shape[0]
    M, N = lhs.shape[1] // 4, rhs.shape[1] // 4
    if rhs.shape[0] != P or lhs.shape[1] % 4 or rhs.shape[1] % 4:
        raise ValueError("lhs [P, 4M] and rhs [P, 4N] must share P")
    if tuple(lhs_scale.shape) != scale_image_shape(P, 4 * M, dense_scale) or \
            tuple(rhs_scale.shape) != scale_image_shape(P, 4 * N, dense_scale):
        raise ValueError("scale shapes do not match the operands")
    return P, M, N


def scaled_matmul(lhs: torch.Tensor, lhs_scale: torch.Tensor, rhs: torch.Tensor, rhs_scale: torch.Tensor,
                  fmt: str = "e4m3fn", res_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None,
                  stream: torch.cuda.Stream | None = None, dense_scale: bool = False) -> torch.Tensor:
    """Block-scaled matmul of two quantized operands.

    ``lhs`` [P, 4M] and ``rhs`` [P, 4N] are FP8 data outputs of
    :func:`quantize` (format ``fmt``) with their scale images ``lhs_scale``
    [P, M] and ``rhs_scale`` [P, N] (or dense [P/8, M], [P/8, N] with
    ``dense_scale``). Each operand is read as the [K = 4P, C] matrix whose
    row k = 4p + j holds element (p, 4c + j). Returns
    out[m][n] = sum_k L[k][m] * R[k][n] as [M, N] float32 or bfloat16.
    """
    lib = load()
    code = _out_code(fmt)
    if res_dtype not in RES_DTYPES:
        raise MXQError(10, "result type must be float32 or bfloat16, got %s" % res_dtype)
    P, M, N = _check_operands(lhs, lhs_scale, rhs, rhs_scale, dense_scale)
    if out is None:
        out = torch.empty((M, N), dtype=res_dtype, device=lhs.device)
    elif out.dtype != res_dtype or tuple(out.shape) != (M, N) or not out.is_contiguous() or out.device != lhs.device:
        raise ValueError("out must be a contiguous [%d, %d] %s tensor on %s" % (M, N, res_dtype, lhs.device))
    sh = _stream_handle(stream, lhs.device)
    _check(_call_on(lhs.device, lib.mxq_scaled_matmul, lhs.data_ptr(), lhs_scale.data_ptr(), rhs.data_ptr(),
                    rhs_scale.data_ptr(), P, M, N, code, RES_DTYPES[res_dtype],
                    FLAG_DENSE_SCALE if dense_scale else 0, out.data_ptr(), sh))
    return out


def scaled_matmul_quantize(lhs: torch.Tensor, lhs_scale: torch.Tensor, rhs: torch.Tensor, rhs_scale: torch.Tensor,
                           fmt: str = "e4m3fn", out_dtype: str = "e4m3fn", data_out: torch.Tensor | None = None,
                           scale_out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None,
                           alt_emax: bool = False, dense_scale: bool = False):
    """The scaled matmul with its [M, N] result quantized in the same kernel.

    Operands as for :func:`scaled_matmul`. Returns ``(data, scale)`` -- the
    bytes :func:`quantize` would write for the bfloat16 result of
    :func:`scaled_matmul` (P = M rows, F = N columns, format ``out_dtype``),
    without that result ever being stored. ``dense_scale`` applies to the
    operand scales and the result scale; ``alt_emax`` to the result.
    """
    lib = load()
    code = _out_code(fmt)
    out_code = _out_code(out_dtype)
    P, M, N = _check_operands(lhs, lhs_scale, rhs, rhs_scale, dense_scale)
    flags = (FLAG_ALT_EMAX if alt_emax else 0) | (FLAG_DENSE_SCALE if dense_scale else 0)
    if M % 8:
        raise MXQError(3, "the result's rows M = %d must be a multiple of 8" % M)
    if data_out is None:
        data_out = torch.empty(data_shape(M, N, out_dtype), dtype=torch.uint8, device=lhs.device)
    if scale_out is None:
        scale_out = torch.empty(scale_image_shape(M, N, dense_scale), dtype=torch.uint8, device=lhs.device)
    _check_out_buffer("data_out", data_out, _data_nbytes(M, N, out_code), lhs.device)
    _check_out_buffer("scale_out", scale_out, _scale_nbytes(M, N, flags), lhs.device)
    sh = _stream_handle(stream, lhs.device)
    _check(_call_on(lhs.device, lib.mxq_scaled_matmul_quantize, lhs.data_ptr(), lhs_scale.data_ptr(),
                    rhs.data_ptr(), rhs_scale.data_ptr(), P, M, N, code, out_code, flags,
                    data_out.data_ptr(), scale_out.data_ptr(), sh))
    return data_out, scale_out


def axis_view_shape(R: int, C: int, dim: int):
    """(P, F) of the partition-major view that :func:`quantize_axis` writes
    for an R x C tensor: (K/4, 4*O) with K the block axis' extent."""
    d = dim + 2 if dim < 0 else dim
    if d not in (0, 1):
        raise MXQError(11, "quantize axis must be -1 or -2 (or 1, 0), got %r" % dim)
    K, O = (C, R) if d == 1 else (R, C)
    return K // 4, 4 * O


def quantize_axis(x: torch.Tensor, out_dtype: str = "e4m3fn", dim: int = -1, data_out: torch.Tensor | None = None,
                  scale_out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None,
                  alt_emax: bool = False, dense_scale: bool = False):
    """Quantize a row-major [R, C] bf16/f16 device tensor with its 32-element
    blocks along ``dim`` (-1: along each row, -2: down each column).

    Returns ``(data, scale)`` in the layout :func:`quantize` produces for the
    partition-major [K/4, 4*O] view (K the block axis' extent, O the other):
    the operand layout of :func:`scaled_matmul`. Activations X [M, K] with
    ``dim=-1`` and weights W [K, N] with ``dim=-2`` make it compute X @ W.
    """
    lib = load()
    code = _out_code(out_dtype)
    if x.dtype not in IN_DTYPES:
        raise MXQError(1, "input must be bfloat16 or float16, got %s" % x.dtype)
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D device tensor [R, C]")
    R, C = x.shape
    P, F = axis_view_shape(R, C, dim)
    flags = (FLAG_ALT_EMAX if alt_emax else 0) | (FLAG_DENSE_SCALE if dense_scale else 0)
    if data_out is None:
        data_out = torch.empty(data_shape(P, F, out_dtype), dtype=torch.uint8, device=x.device)
    if scale_out is None:
        scale_out = torch.empty(scale_image_shape(P, F, dense_scale), dtype=torch.uint8, device=x.device)
    _check_out_buffer("data_out", data_out, _data_nbytes(P, F, code), x.device)
    _check_out_buffer("scale_out", scale_out, _scale_nbytes(P, F, flags), x.device)
    sh = _stream_handle(stream, x.device)
    _check(_call_on(x.device, lib.mxq_quantize_axis, x.data_ptr(), R, C, IN_DTYPES[x.dtype], code, dim, flags,
                    data_out.data_ptr(), scale_out.data_ptr(), sh))
    return data_out, scale_out
