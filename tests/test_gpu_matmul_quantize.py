"""GPU parity of quantize-on-produce (the scaled matmul with its result
quantized in the epilogue).

The kernel's bytes are defined as quantize(bf16(matmul)), so two checks:

* consistency: they equal, bit for bit, the unfused pair on the GPU -- the
  bf16 result of scaled_matmul quantized by quantize (both of which are
  checked against the oracle elsewhere);
* oracle parity: the oracle composes the exact sum, fp32 and bf16 rounding
  and its quantize. The matrix cores do not sum exactly (the bound is the
  one the scaled-matmul tests derive), so where the GPU byte differs from the
  oracle's it must be one that a sum inside the bound produces: the block's
  E8M0 lies between the E8M0 of the smallest and of the largest block
  maximum any admissible sum gives, and each code lies between the codes of
  the interval's two ends under the GPU's own E8M0 (quantize is monotone in
  the value for a fixed scale). Most bytes must match exactly.
"""
import numpy as np
import pytest
import torch

import defcheck
import mx_microscaling_quantization_amd as mxq
import oracle
from conftest import progress
from test_gpu_matmul import _patch_255, bound, make_operand, values64

pytestmark = pytest.mark.gpu


def _emax_bias(out_dtype, alt):
    return oracle.emax(out_dtype) - (1 if alt else 0)


def _bf16_values(x64: np.ndarray) -> np.ndarray:
    """float64 -> fp32 (nearest-even) -> bf16 (oracle rounding), as float64."""
    with np.errstate(over="ignore", invalid="ignore"):
        b = oracle.f32_to_bf16(x64.astype(np.float32)).reshape(x64.shape)
    return oracle.widen(b, "bf16").reshape(x64.shape).astype(np.float64)


def _e8m0_of(mag: np.ndarray, bias: int) -> np.ndarray:
    """E8M0 of blocks whose maximum magnitude is `mag` (a bf16 value, NaN
    counts as exponent field 255): max(1, field - bias)."""
    field = (mag.astype(np.float32).view(np.uint32) >> 23) & 0xFF
    field = np.where(np.isnan(mag), 255, field).astype(np.int64)
    return np.maximum(1, field - bias)


def check_admissible(exact, tol, data, scale, M, N, out_dtype, alt, layout):
    """Check the GPU's (data, scale) for an M x N result against the exact
    sums and their bound; returns the fraction of codes equal to the
    oracle composition's bytes' codes."""
    bias = _emax_bias(out_dtype, alt)
    nan = np.isnan(exact)
    lo = _bf16_values(np.where(nan, 0.0, exact - tol))
    hi = _bf16_values(np.where(nan, 0.0, exact + tol))
    lmag = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    umag = np.maximum(np.abs(lo), np.abs(hi))
    lmag = np.where(nan, np.nan, lmag)
    umag = np.where(nan, np.nan, umag)
    blk = lambda a: a.reshape(M // 8, 8, N // 4, 4)
    with np.errstate(invalid="ignore"):
        has_nan = blk(nan).any(axis=(1, 3))
        bmin = np.where(has_nan, np.nan, np.nanmax(np.where(np.isnan(blk(lmag)), -1, blk(lmag)), axis=(1, 3)))
        bmax = np.where(has_nan, np.nan, np.nanmax(np.where(np.isnan(blk(umag)), -1, blk(umag)), axis=(1, 3)))
    e_lo, e_hi = _e8m0_of(bmin, bias), _e8m0_of(bmax, bias)
    placed = np.arange(M // 8) if layout == "dense" else defcheck.scale_slot(np.arange(M // 8))
    e_got = scale[placed].astype(np.int64)                                  # [M/8, N/4]
    bad = (e_got < e_lo) | (e_got > e_hi)
    assert not bad.any(), "E8M0 outside the admissible range at block %s: got %d, range [%d, %d]" % (
        tuple(np.argwhere(bad)[0]), e_got[bad][0], e_lo[bad][0], e_hi[bad][0])

    codes = defcheck.unpack_codes(data, M, N, out_dtype)
    got = defcheck.decode_codes(codes, out_dtype)
    e_full = np.repeat(np.repeat(e_got, 8, axis=0), 4, axis=1).astype(np.uint8).ravel()
    q_lo = oracle.narrow(oracle.prescale(lo.astype(np.float32), e_full), out_dtype).reshape(M, N)
    q_hi = oracle.narrow(oracle.prescale(hi.astype(np.float32), e_full), out_dtype).reshape(M, N)
    v_lo = oracle.decode(q_lo, out_dtype).reshape(M, N)
    v_hi = oracle.decode(q_hi, out_dtype).reshape(M, N)
    ok = np.where(nan, got == 0, (got >= v_lo) & (got <= v_hi))
    assert ok.all(), "code outside the admissible interval at %s: got %r, interval [%r, %r]" % (
        tuple(np.argwhere(~ok)[0]), got[~ok][0], v_lo[~ok][0], v_hi[~ok][0])


def _unfused(dl, sl, dr, sr, fmt, out_dtype, alt, dense, M, N):
    res = mxq.scaled_matmul(dl, sl, dr, sr, fmt, torch.bfloat16, dense_scale=dense)
    scale = torch.zeros(mxq.scale_image_shape(M, N, dense), dtype=torch.uint8, device="cuda")
    return mxq.quantize(res, out_dtype, scale_out=scale, alt_emax=alt, dense_scale=dense)


def run_case(P, M, N, fmt, out_dtype, alt=False, dense=False, seed=0, oracle_check=True):
    layout = "dense" if dense else "image"
    dl, sl, hl, hsl = make_operand(P, M, fmt, seed * 2 + 1, dense)
    dr, sr, hr, hsr = make_operand(P, N, fmt, seed * 2 + 2, dense)
    scale = torch.zeros(mxq.scale_image_shape(M, N, dense), dtype=torch.uint8, device="cuda")
    data, scale = mxq.scaled_matmul_quantize(dl, sl, dr, sr, fmt, out_dtype, scale_out=scale, alt_emax=alt,
                                             dense_scale=dense)
    ud, us = _unfused(dl, sl, dr, sr, fmt, out_dtype, alt, dense, M, N)
    torch.cuda.synchronize()
    assert torch.equal(data, ud), "fused data differs from quantize(scaled_matmul bf16)"
    assert torch.equal(scale, us), "fused scale differs from quantize(scaled_matmul bf16)"
    if not oracle_check:
        return
    got_d, got_s = data.cpu().numpy(), scale.cpu().numpy()
    ref_d, ref_s = oracle.scaled_matmul_quantize(hl, hsl, hr, hsr, fmt, out_dtype, alt_emax=alt, layout=layout)
    exact = oracle.scaled_matmul(hl, hsl, hr, hsr, fmt, layout=layout)
    L = values64(hl, hsl, P, M, fmt, layout)
    R = values64(hr, hsr, P, N, fmt, layout)
    tol = bound(L, R, torch.float32, exact)
    check_admissible(exact, tol, got_d, got_s, M, N, out_dtype, alt, layout)
    same_codes = np.mean(defcheck.unpack_codes(got_d, M, N, out_dtype) == defcheck.unpack_codes(ref_d, M, N, out_dtype))
    progress("codes equal to the oracle composition: %.5f" % same_codes)
    assert same_codes > 0.99


SHAPES = [(8, 8, 4), (32, 128, 128), (64, 256, 256), (40, 136, 260), (256, 200, 68), (96, 512, 384),
          (520, 64, 132)]


@pytest.mark.parametrize("out_dtype", ["e4m3fn", "e5m2", "e2m1"])
@pytest.mark.parametrize("fmt", ["e4m3fn", "e5m2"])
@pytest.mark.parametrize("P,M,N", SHAPES)
def test_matmul_quantize_against_oracle(P, M, N, fmt, out_dtype):
    progress("matmul_quantize %s -> %s P=%d M=%d N=%d" % (fmt, out_dtype, P, M, N))
    run_case(P, M, N, fmt, out_dtype, seed=P + M + N)


@pytest.mark.parametrize("out_dtype", ["e4m3fn", "e5m2", "e2m1"])
def test_matmul_quantize_many_tiles(out_dtype):
    """5 x 5 output tiles, both edges ragged, a K tail, and 138 row groups (scale
    image rows up to 1089): fused bytes equal the unfused pair's, whose two
    kernels the oracle checks separately."""
    progress("matmul_quantize e4m3fn -> %s P=24 M=1104 N=1160" % out_dtype)
    run_case(24, 1104, 1160, "e4m3fn", out_dtype, seed=23, oracle_check=False)


@pytest.mark.parametrize("out_dtype", ["e4m3fn", "e2m1"])
@pytest.mark.parametrize("alt,dense", [(True, False), (False, True), (True, True)])
def test_matmul_quantize_modes(out_dtype, alt, dense):
    progress("matmul_quantize modes %s alt=%s dense=%s" % (out_dtype, alt, dense))
    run_case(64, 264, 132, "e4m3fn", out_dtype, alt=alt, dense=dense, seed=11)


def test_matmul_quantize_empty_k():
    """K = 0: every result is +0, so the data is all zero codes and every
    block's E8M0 is 1."""
    d = torch.zeros((0, 32), dtype=torch.uint8, device="cuda")
    s = torch.zeros((0, 8), dtype=torch.uint8, device="cuda")
    r = torch.zeros((0, 64), dtype=torch.uint8, device="cuda")
    rs = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    data = torch.full((8, 16), 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.zeros((8, 4), dtype=torch.uint8, device="cuda")
    mxq.scaled_matmul_quantize(d, s, r, rs, "e4m3fn", "e4m3fn", data_out=data, scale_out=scale)
    torch.cuda.synchronize()
    assert not bool(data.any())
    assert scale[0].tolist() == [1, 1, 1, 1] and not bool(scale[1:].any())


def test_matmul_quantize_nan_block():
    """A NaN code in lhs column 3 makes result row 3 NaN; its blocks take
    E8M0 255 - EMAX and their codes are zeros, as the quantize does for a
    NaN."""
    P, M, N = 32, 16, 8
    dl, sl, hl, hsl = make_operand(P, M, "e4m3fn", 31)
    dr, sr, hr, hsr = make_operand(P, N, "e4m3fn", 32)
    dl[0, 12] = 0x7F                   # k = 0 of container 3: the e4m3fn NaN
    hl[0, 12] = 0x7F
    scale = torch.zeros((M, N // 4), dtype=torch.uint8, device="cuda")
    data, scale = mxq.scaled_matmul_quantize(dl, sl, dr, sr, "e4m3fn", "e5m2", scale_out=scale)
    ud, us = _unfused(dl, sl, dr, sr, "e4m3fn", "e5m2", False, False, M, N)
    torch.cuda.synchronize()
    assert torch.equal(data, ud) and torch.equal(scale, us)
    exact = oracle.scaled_matmul(hl, hsl, hr, hsr, "e4m3fn")
    assert np.isnan(exact[3]).all()
    d, s = data.cpu().numpy(), scale.cpu().numpy()
    assert (s[defcheck.scale_slot(0)] == 255 - 15).all()                 # row group 0 holds row 3
    assert not (d[3] & 0x7F).any()
    L = values64(hl, hsl, P, M, "e4m3fn")
    R = values64(hr, hsr, P, N, "e4m3fn")
    check_admissible(exact, bound(L, R, torch.float32, exact), d, s, M, N, "e5m2", False, "image")


@pytest.mark.parametrize("out_dtype", ["e4m3fn", "e2m1"])
def test_matmul_quantize_e8m0_255_blocks(out_dtype):
    """Operand blocks under E8M0 255 (the scale 2^128): the fused bytes
    equal the unfused pair's, and the oracle's within the bound."""
    P, M, N = 32, 72, 136
    dl, sl, hl, hsl = make_operand(P, M, "e4m3fn", 41)
    dr, sr, hr, hsr = make_operand(P, N, "e4m3fn", 42)
    _patch_255(lhs_blocks=[(1, 2)], rhs_blocks=[(2, 9)])(sl, hsl, sr, hsr)
    scale = torch.zeros((M, N // 4), dtype=torch.uint8, device="cuda")
    data, scale = mxq.scaled_matmul_quantize(dl, sl, dr, sr, "e4m3fn", out_dtype, scale_out=scale)
    ud, us = _unfused(dl, sl, dr, sr, "e4m3fn", out_dtype, False, False, M, N)
    torch.cuda.synchronize()
    assert torch.equal(data, ud) and torch.equal(scale, us)
    exact = oracle.scaled_matmul(hl, hsl, hr, hsr, "e4m3fn")
    assert np.isfinite(exact).all() and np.abs(exact[2]).max() > 2.0 ** 60
    tol = bound(values64(hl, hsl, P, M, "e4m3fn"), values64(hr, hsr, P, N, "e4m3fn"), torch.float32, exact,
                adds_per_block=4)
    check_admissible(exact, tol, data.cpu().numpy(), scale.cpu().numpy(), M, N, out_dtype, False, "image")


def test_matmul_quantize_full_size_sampled():
    """The bench's 8192 x 8192 x 8192 e4m3fn -> e4m3fn case: all bytes
    against the unfused pair, and 512 sampled blocks (8 rows x 4 columns)
    against the oracle's exact sums, on the host's threads."""
    P, M, N = 2048, 8192, 8192
    progress("matmul_quantize full size: operands")
    g = torch.Generator(device="cuda")
    g.manual_seed(23)
    xl = torch.randn((P, 4 * M), generator=g, device="cuda").to(torch.bfloat16)
    xr = torch.randn((P, 4 * N), generator=g, device="cuda").to(torch.bfloat16)
    dl, sl = mxq.quantize(xl, "e4m3fn")
    dr, sr = mxq.quantize(xr, "e4m3fn")
    del xl, xr
    progress("matmul_quantize full size: fused and unfused")
    scale = torch.zeros((M, N // 4), dtype=torch.uint8, device="cuda")
    data, scale = mxq.scaled_matmul_quantize(dl, sl, dr, sr, "e4m3fn", "e4m3fn", scale_out=scale)
    ud, us = _unfused(dl, sl, dr, sr, "e4m3fn", "e4m3fn", False, False, M, N)
    torch.cuda.synchronize()
    assert torch.equal(data, ud) and torch.equal(scale, us)
    del ud, us
    progress("matmul_quantize full size: 512 sampled oracle blocks")
    import concurrent.futures
    import os

    rng = np.random.default_rng(9)
    picks = [(int(rng.integers(M // 8)), int(rng.integers(N // 4))) for _ in range(512)]
    cols = lambda idx: np.concatenate([np.arange(4 * c, 4 * c + 4) for c in idx])
    hdata, hscale = data.cpu().numpy(), scale.cpu().numpy()
    blocks = []
    for gi, cb in picks:
        ms, ns = np.arange(8 * gi, 8 * gi + 8), np.arange(4 * cb, 4 * cb + 4)
        blocks.append((gi, cb, np.ascontiguousarray(dl[:, torch.from_numpy(cols(ms)).cuda()].cpu().numpy()),
                       np.ascontiguousarray(sl[:, torch.from_numpy(ms).cuda()].cpu().numpy()),
                       np.ascontiguousarray(dr[:, torch.from_numpy(cols(ns)).cuda()].cpu().numpy()),
                       np.ascontiguousarray(sr[:, torch.from_numpy(ns).cuda()].cpu().numpy())))

    def check_block(b):
        gi, cb, hl, hsl, hr, hsr = b
        exact = oracle.scaled_matmul(hl, hsl, hr, hsr, "e4m3fn")
        tol = bound(values64(hl, hsl, P, 8, "e4m3fn"), values64(hr, hsr, P, 4, "e4m3fn"), torch.float32, exact)
        blk_data = hdata[8 * gi:8 * gi + 8, 4 * cb:4 * cb + 4]
        blk_scale = np.zeros((8, 1), np.uint8)
        blk_scale[defcheck.scale_slot(0)] = hscale[int(defcheck.scale_slot(gi)), cb]
        check_admissible(exact, tol, blk_data, blk_scale, 8, 4, "e4m3fn", False, "image")

    check_block(blocks[0])   # loads the oracle before the threads
    with concurrent.futures.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(check_block, blocks[1:]))
