"""Seeded synthetic inputs for the MX quantize workloads.

This module draws random numbers and rounds them to bf16 / f16 bit patterns.
It holds none of the quantize arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it.

Workloads (P x F, input type, output types, seed, value recipe):

* ``bf16-128x512-handplaced``  -- N(0,1), plus four hand-placed blocks:
  all zero (with one -0.0), exact round-to-nearest-even ties, one 2^20
  outlier among N(0,1), and bf16 subnormals. Output e4m3fn.
* ``bf16-4096x4096-rowscaled`` -- z * r_p, z ~ N(0,1), per-row r_p =
  exp(N(0, 2^2)); 0.1 % of the elements set to +-1000. Outputs e4m3fn and e5m2.
* ``f16-8192x14336-student-t`` -- Student-t (nu = 3) clipped to +-65504;
  1 % of the 8x4 blocks all zero, a disjoint 1 % filled with f16 subnormals.
  Output e5m2.
* ``bf16-16384x8192-blockexp`` -- per 8x4 block an integer k ~ U{-60..60},
  x = U(-1, 1) * 2^k. Output e2m1.
* ``bf16-131072x8192-colscaled`` -- z * c_f, z ~ N(0,1) drawn on the device,
  per-column c_f = exp(N(0, 1)). Output e4m3fn. 1.07 G elements, 2 GiB in.
* ``bf16-131072x8200-colscaled``, ``bf16-131072x8188-colscaled`` -- the same
  recipe on row pitches that are not a multiple of 128 bytes (F % 8 == 0 and
  F % 8 == 4). Outputs e4m3fn and e2m1. Measurement cases for those pitches.

The pages measure on no dataset, so these seeded recipes stand alone.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "bf16-128x512-handplaced": dict(P=128, F=512, in_dtype="bf16", outs=("e4m3fn",), seed=1),
    "bf16-4096x4096-rowscaled": dict(P=4096, F=4096, in_dtype="bf16", outs=("e4m3fn", "e5m2"), seed=2),
    "f16-8192x14336-student-t": dict(P=8192, F=14336, in_dtype="f16", outs=("e5m2",), seed=3),
    "bf16-16384x8192-blockexp": dict(P=16384, F=8192, in_dtype="bf16", outs=("e2m1",), seed=4),
    "bf16-131072x8192-colscaled": dict(P=131072, F=8192, in_dtype="bf16", outs=("e4m3fn",), seed=5),
    "bf16-131072x8200-colscaled": dict(P=131072, F=8200, in_dtype="bf16", outs=("e4m3fn", "e2m1"), seed=6),
    "bf16-131072x8188-colscaled": dict(P=131072, F=8188, in_dtype="bf16", outs=("e4m3fn", "e2m1"), seed=7),
}
# Workloads drawn on the device (too large to draw on the host).
DEVICE_DRAWN = ("bf16-131072x8192-colscaled", "bf16-131072x8200-colscaled", "bf16-131072x8188-colscaled")

# Hand-placed blocks of the 128x512 workload: (row group, column block).
HANDPLACED = {"zero": (0, 0), "ties": (3, 17), "outlier": (7, 64), "subnormal": (15, 127)}
# Values of the "ties" block after its 256.0 pilot, repeated to fill the block.
TIE_VALUES = (1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 464.0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns, nearest-even (inputs finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _block_view(a: np.ndarray) -> np.ndarray:
    P, F = a.shape
    return a.reshape(P // 8, 8, F // 4, 4)


def handplaced_bf16_128x512(seed: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    P, F = 128, 512
    x = f32_to_bf16_bits(rng.standard_normal((P, F), dtype=np.float32))
    b = _block_view(x)
    # all zero, one of them negative zero
    g, c = HANDPLACED["zero"]
    b[g, :, c, :] = 0
    b[g, 5, c, 2] = 0x8000
    # ties: pilot 256, then the tie values cycling, the rest zero
    g, c = HANDPLACED["ties"]
    vals = [256.0] + [TIE_VALUES[k % len(TIE_VALUES)] for k in range(28)] + [0.0] * 3
    b[g, :, c, :] = f32_to_bf16_bits(np.array(vals, dtype=np.float32)).reshape(8, 4)
    # one 2^20 outlier among N(0,1)
    g, c = HANDPLACED["outlier"]
    b[g, 2, c, 1] = f32_to_bf16_bits(np.array([2.0 ** 20], dtype=np.float32))[0]
    # bf16 subnormals: exponent field 0, fraction 1..127, random sign
    g, c = HANDPLACED["subnormal"]
    frac = rng.integers(1, 128, size=(8, 4)).astype(np.uint16)
    sign = rng.integers(0, 2, size=(8, 4)).astype(np.uint16) << 15
    b[g, :, c, :] = frac | sign
    return x


def rowscaled_bf16(P: int = 4096, F: int = 4096, seed: int = 2) -> np.ndarray:
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((P, F), dtype=np.float32)
    r = np.exp(rng.normal(0.0, 2.0, size=(P, 1))).astype(np.float32)
    x = f32_to_bf16_bits(z * r).ravel()
    n_out = (P * F) // 1000
    pos = rng.permutation(P * F)[:n_out]
    sign = rng.integers(0, 2, size=n_out).astype(np.uint16) << 15
    x[pos] = f32_to_bf16_bits(np.full(n_out, 1000.0, dtype=np.float32)) | sign
    return x.reshape(P, F)


def student_t_f16(P: int = 8192, F: int = 14336, seed: int = 3) -> np.ndarray:
    rng = np.random.default_rng(seed)
    t = rng.standard_t(3, size=(P, F)).astype(np.float32)
    np.clip(t, -65504.0, 65504.0, out=t)
    x = f32_to_f16_bits(t)
    nblocks = (P // 8) * (F // 4)
    k = nblocks // 100
    ids = rng.permutation(nblocks)[: 2 * k]
    b = _block_view(x)
    gz, cz = np.divmod(ids[:k], F // 4)
    b[gz, :, cz, :] = 0
    gs, cs = np.divmod(ids[k:], F // 4)
    frac = rng.integers(1, 1024, size=(k, 8, 4)).astype(np.uint16)
    sign = rng.integers(0, 2, size=(k, 8, 4)).astype(np.uint16) << 15
    b[gs, :, cs, :] = frac | sign
    return x


def blockexp_bf16(P: int = 16384, F: int = 8192, seed: int = 4) -> np.ndarray:
    rng = np.random.default_rng(seed)
    k = rng.integers(-60, 61, size=(P // 8, 1, F // 4, 1)).astype(np.int32)
    u = rng.uniform(-1.0, 1.0, size=(P // 8, 8, F // 4, 4)).astype(np.float32)
    x = np.ldexp(u, k).astype(np.float32)
    return f32_to_bf16_bits(x.reshape(P, F))


def colscale_factors(F: int = 8192, seed: int = 5) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.exp(rng.normal(0.0, 1.0, size=F)).astype(np.float32)


def colscaled_bf16_device(P: int = 131072, F: int = 8192, seed: int = 5, device: str = "cuda"):
    """The large workload, drawn on the device with torch's seeded generator.

    Returns a contiguous torch.bfloat16 tensor [P, F] on ``device``. Rows are
    drawn in slabs to bound the fp32 temporary.
    """
    import torch

    c = torch.from_numpy(colscale_factors(F, seed)).to(device)
    out = torch.empty((P, F), dtype=torch.bfloat16, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    slab = 8192
    for r0 in range(0, P, slab):
        r1 = min(P, r0 + slab)
        z = torch.randn((r1 - r0, F), generator=g, device=device, dtype=torch.float32)
        out[r0:r1] = (z * c).to(torch.bfloat16)
    return out


def colscaled_bf16_host(P: int, F: int, seed: int = 5) -> np.ndarray:
    """Host version of the column-scaled recipe, for sizes small enough to draw
    on the CPU (same distribution, different stream from the device one)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((P, F), dtype=np.float32)
    return f32_to_bf16_bits(z * colscale_factors(F, seed)[None, :])


def make_host(name: str) -> np.ndarray:
    """uint16 [P, F] bit patterns of a host-drawn workload."""
    if name == "bf16-128x512-handplaced":
        return handplaced_bf16_128x512()
    if name == "bf16-4096x4096-rowscaled":
        return rowscaled_bf16()
    if name == "f16-8192x14336-student-t":
        return student_t_f16()
    if name == "bf16-16384x8192-blockexp":
        return blockexp_bf16()
    raise KeyError(name)


def random_bits(P: int, F: int, in_dtype: str, seed: int, specials: bool = False) -> np.ndarray:
    """Generic seeded test tensor: N(0,1) times a per-block power of two in
    [2^-40, 2^40], optionally salted with zeros, subnormals, +-Inf and NaN."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((P, F)).astype(np.float32)
    if P % 8 == 0 and F % 4 == 0 and P and F:
        k = rng.integers(-40, 41, size=(P // 8, 1, F // 4, 1))
        scale = np.broadcast_to(np.ldexp(1.0, k), (P // 8, 8, F // 4, 4)).reshape(P, F)
        z = (z * scale).astype(np.float32)
    if in_dtype == "f16":
        z = np.clip(z, -65504.0, 65504.0)
        x = f32_to_f16_bits(z)
        sub_mask, inf_bits, nan_bits, frac_hi = 0x03FF, 0x7C00, 0x7E00, 1024
    else:
        x = f32_to_bf16_bits(z)
        sub_mask, inf_bits, nan_bits, frac_hi = 0x007F, 0x7F80, 0x7FC0, 128
    if specials and x.size:
        flat = x.ravel()
        n = flat.size
        picks = rng.integers(0, n, size=max(1, n // 50))
        kinds = rng.integers(0, 5, size=picks.size)
        sign = (rng.integers(0, 2, size=picks.size).astype(np.uint16) << 15)
        sub = rng.integers(1, frac_hi, size=picks.size).astype(np.uint16) & sub_mask
        vals = np.where(kinds == 0, 0, np.where(kinds == 1, sub, np.where(kinds == 2, inf_bits,
                        np.where(kinds == 3, nan_bits, flat[picks] & 0x7FFF)))).astype(np.uint16)
        flat[picks] = vals | sign
    return x
