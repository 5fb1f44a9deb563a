"""Definition-level checker used to pin the oracle (tiny and exhaustive cases).

Independent of ``oracle/``: it shares no code with it and computes each step
from a different definition --

* widening through numpy's own float16 / bit-level bfloat16 conversion;
* the block scale from the closed form
  E8M0 = max(1, floor(log2 max|x|) + 127 - EMAX) (frexp in double), which the
  bit trick of "MX Microscaling: Quantize, Block-Scaling and E8M0"
  (Block-Scale Computation) must equal;
* the prescaled value exactly in float64 (x * 2^(127 - E8M0));
* the narrow by brute force: the nearest of all finite codes of the format,
  ties to the even code, values beyond the largest code saturating;
* FP4 container positions from the hand-worked table in
  ``tests/golden/fp4_container_order.txt``;
* scale rows from the hand-worked ``tests/golden/scale_slots.txt`` pattern.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Format definitions (OCP FP8 e4m3fn / e5m2, OCP FP4 e2m1).
FORMATS = {
    "e4m3fn": dict(ebits=4, mbits=3, bias=7, maxcode=0x7E, signbit=0x80),
    "e5m2": dict(ebits=5, mbits=2, bias=15, maxcode=0x7B, signbit=0x80),
    "e2m1": dict(ebits=2, mbits=1, bias=1, maxcode=0x7, signbit=0x8),
}
EMAX = {"e2m1": 2, "e4m3fn": 8, "e5m2": 15}


def read_table(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def code_values(fmt: str) -> np.ndarray:
    """Value of every non-negative finite code 0..maxcode, from the format's
    sign/exponent/mantissa definition (float64, exact)."""
    f = FORMATS[fmt]
    codes = np.arange(f["maxcode"] + 1)
    m = codes & ((1 << f["mbits"]) - 1)
    e = codes >> f["mbits"]
    sub = np.ldexp(m.astype(np.float64), 1 - f["bias"] - f["mbits"])
    nor = np.ldexp(((1 << f["mbits"]) + m).astype(np.float64), e - f["bias"] - f["mbits"])
    return np.where(e == 0, sub, nor)


def narrow_bruteforce(y: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest finite code, ties to the even code, saturating; NaN -> signed
    zero (the reading used for the FP8 formats, and the FP4 page rule)."""
    f = FORMATS[fmt]
    vals = code_values(fmt)
    with np.errstate(invalid="ignore"):
        y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    hi = np.searchsorted(vals, a, side="left")          # vals[hi-1] < a <= vals[hi]
    hi_c = np.minimum(hi, vals.size - 1)
    lo_c = np.maximum(hi - 1, 0)
    d_hi = np.abs(vals[hi_c] - a)
    d_lo = np.abs(a - vals[lo_c])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(pick_hi, hi_c, lo_c)
    code = np.where(a >= vals[-1], vals.size - 1, code)  # saturate (and +-inf)
    sign = np.signbit(y)                               # NaN keeps its sign bit too
    return (code | np.where(sign, f["signbit"], 0)).astype(np.uint8)


def widen(h: np.ndarray, in_dtype: str) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    with np.errstate(invalid="ignore"):   # NaN patterns stay NaN
        if in_dtype == "f16":
            return h.view(np.float16).astype(np.float64)
        return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e8m0_closed_form(block_absmax: np.ndarray, fmt: str, alt: bool = False) -> np.ndarray:
    """max(1, floor(log2 a) + 127 - bias) for finite a > 0; 1 for a == 0;
    255 - bias for a non-finite block (its exponent field is all ones)."""
    bias = EMAX[fmt] - (1 if alt else 0)
    a = np.asarray(block_absmax, dtype=np.float64)
    finite = np.isfinite(a)
    safe = np.where(finite & (a > 0), a, 1.0)
    _, ex = np.frexp(safe)                 # a = f * 2^ex, f in [0.5, 1)
    e = (ex - 1) + 127 - bias
    e = np.where(finite & (a > 0), e, np.where(finite, 0, 255 - bias))
    return np.maximum(e, 1).astype(np.uint8)


def container_table():
    """element-in-container -> (byte-in-container, high nibble?)"""
    tab = {}
    for k, _r, byte, hi in read_table("fp4_container_order.txt"):
        tab[int(k)] = (int(byte), int(hi))
    return tab


def scale_slot(i: np.ndarray) -> np.ndarray:
    """Runs of four rows, each run 32 rows after the last (the hand-worked
    table in tests/golden/scale_slots.txt is checked against this)."""
    i = np.asarray(i)
    return (i % 4) + 32 * (i // 4)


def quantize(x: np.ndarray, in_dtype: str, fmt: str, alt: bool = False, image: np.ndarray | None = None,
             layout: str = "image"):
    """Whole quantize by the definitions above; returns (data, image).
    layout "dense" returns the [P/8, F/4] scale array instead of the image."""
    x = np.asarray(x, dtype=np.uint16)
    P, F = x.shape
    v = widen(x, in_dtype)
    blocks = np.abs(v).reshape(P // 8, 8, F // 4, 4)
    absmax = blocks.max(axis=(1, 3))                   # NaN propagates
    e = e8m0_closed_form(absmax, fmt, alt)             # [P/8, F/4]
    e_full = np.repeat(np.repeat(e, 8, axis=0), 4, axis=1).astype(np.int64)
    y = v * np.ldexp(1.0, 127 - e_full)                # exact in float64
    # reading: E8M0 254 (alternative bias, FP4, non-finite block) has a zero
    # multiplier, so every element of such a block is a zero of its own sign
    y = np.where(e_full == 254, np.copysign(0.0, v), y)
    codes = narrow_bruteforce(y, fmt).reshape(P, F)
    if fmt == "e2m1":
        tab = container_table()
        data = np.zeros((P, F // 2), dtype=np.uint8)
        c4 = codes.reshape(P, F // 4, 4)
        out = data.reshape(P, F // 4, 2)
        for k in range(4):
            byte, hi = tab[k]
            out[:, :, byte] |= (c4[:, :, k] << (4 if hi else 0)).astype(np.uint8)
    else:
        data = codes.astype(np.uint8)
    if layout == "dense":
        return data, e.astype(np.uint8)
    if image is None:
        image = np.zeros((P, F // 4), dtype=np.uint8)
    else:
        image = image.copy()
    image[scale_slot(np.arange(P // 8))] = e
    return data, image


def unpack_codes(data: np.ndarray, P: int, F: int, fmt: str) -> np.ndarray:
    """[P, F] element codes from packed data (FP4 via the golden container table)."""
    if fmt != "e2m1":
        return np.asarray(data, dtype=np.uint8).reshape(P, F)
    tab = container_table()
    d = np.asarray(data, dtype=np.uint8).reshape(P, F // 4, 2)
    codes = np.zeros((P, F // 4, 4), dtype=np.uint8)
    for k in range(4):
        byte, hi = tab[k]
        codes[:, :, k] = (d[:, :, byte] >> 4) if hi else (d[:, :, byte] & 0xF)
    return codes.reshape(P, F)


def decode_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Values of codes (float64): the finite-code table with the sign bit;
    e4m3fn 0x7F/0xFF and e5m2 0x7D-0x7F are NaN, e5m2 0x7C is Inf."""
    f = FORMATS[fmt]
    codes = np.asarray(codes, dtype=np.int64)
    mag = codes & (f["signbit"] - 1)
    sign = np.where(codes & f["signbit"], -1.0, 1.0)
    vals = code_values(fmt)
    table = np.full(f["signbit"], np.nan)
    table[: vals.size] = vals
    if fmt == "e5m2":
        table[0x7C] = np.inf
    return sign * table[mag]


def dequantize(data: np.ndarray, image: np.ndarray, P: int, F: int, fmt: str) -> np.ndarray:
    """float32 [P, F]: decode(q) * 2^(E8M0 - 127), exact in float64, rounded
    once to float32 (numpy's own conversion)."""
    codes = unpack_codes(data, P, F, fmt)
    e = np.asarray(image, dtype=np.int64)[scale_slot(np.arange(P // 8))]      # [P/8, F/4]
    e_full = np.repeat(np.repeat(e, 8, axis=0), 4, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        return (decode_codes(codes, fmt) * np.ldexp(1.0, e_full - 127)).astype(np.float32)
