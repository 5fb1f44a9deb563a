"""Seeded random shapes, flags and output offsets for every streaming entry
point, bit-exact against the CPU oracle.

Each case draws a shape (row pitches aligned or not to 128 bytes, so both
the shared-line and the line-owning launches run, with run counts that hit
exact multiples of a workgroup's strips and one strip past them), the
formats, the scale layout and EMAX mode, and a byte offset of the output
buffers inside a larger, sentinel-filled allocation; the bytes before and
after each output must keep their sentinel.
"""
import numpy as np
import pytest
import torch

import mx_microscaling_quantization_amd as mxq
import oracle
import workloads
from conftest import progress

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}
FMTS = ("e4m3fn", "e5m2", "e2m1")
SENT = 0x5A
GUARD = 256
# strips per workgroup that the launches use (64, 56, 48): row lengths
# around their multiples
EDGES = (48, 56, 64)


def _cols(rng):
    """A column count: either random, or placed at/next to a multiple of a
    workgroup's strip count for 1-, 2- and 4-column strips."""
    if rng.random() < 0.5:
        return int(rng.integers(1, 1200)) * 4
    strip_cols = int(rng.choice([4, 8, 16]))
    k = int(rng.integers(1, 5)) * int(rng.choice(EDGES))
    return max(4, strip_cols * k + int(rng.choice([-strip_cols, 0, strip_cols])))


def _buf(nbytes, offset):
    buf = torch.full((offset + nbytes + GUARD,), SENT, dtype=torch.uint8, device="cuda")
    return buf, buf[offset:offset + nbytes]


def _guards(buf, offset, nbytes, what):
    h = buf.cpu().numpy()
    assert (h[:offset] == SENT).all() and (h[offset + nbytes:] == SENT).all(), "write outside the %s buffer" % what
    return h[offset:offset + nbytes]


@pytest.mark.parametrize("seed", range(24))
def test_random_quantize(seed):
    rng = np.random.default_rng(1000 + seed)
    P, F = 8 * int(rng.integers(1, 40)), _cols(rng)
    in_dtype, out = str(rng.choice(["bf16", "f16"])), str(rng.choice(FMTS))
    alt, dense = bool(rng.integers(2)), bool(rng.integers(2))
    off = int(rng.choice([0, 16, 48, 112]))
    progress("random quantize seed=%d %dx%d %s->%s alt=%d dense=%d off=%d" % (seed, P, F, in_dtype, out, alt, dense, off))
    x = workloads.random_bits(P, F, in_dtype, seed=seed, specials=True)
    xt = torch.from_numpy(x.view(np.int16)).view(TDT[in_dtype]).cuda()
    nd = mxq.data_bytes(P, F, out)
    sshape = mxq.scale_image_shape(P, F, dense)
    ns = sshape[0] * sshape[1]
    dbuf, d = _buf(nd, off)
    sbuf, s = _buf(ns, off)
    mxq.quantize(xt, out, data_out=d.view(mxq.data_shape(P, F, out)), scale_out=s.view(sshape), alt_emax=alt,
                 dense_scale=dense)
    torch.cuda.synchronize()
    got_d = _guards(dbuf, off, nd, "data")
    got_s = _guards(sbuf, off, ns, "scale").reshape(sshape)
    layout = "dense" if dense else "image"
    fill = np.full(oracle.scale_shape(P, F, layout), SENT, np.uint8)
    ref_d, ref_s = oracle.quantize(x, in_dtype, out, image=fill, alt_emax=alt, layout=layout)
    assert np.array_equal(got_d, ref_d.reshape(-1)), "data differs"
    assert np.array_equal(got_s, ref_s), "scales differ"


@pytest.mark.parametrize("seed", range(24))
def test_random_dequantize(seed):
    rng = np.random.default_rng(2000 + seed)
    P, F = 8 * int(rng.integers(1, 40)), _cols(rng)
    fmt, res = str(rng.choice(FMTS)), str(rng.choice(["bf16", "f32"]))
    dense = bool(rng.integers(2))
    off = int(rng.choice([0, 16, 48, 112]))
    progress("random dequantize seed=%d %dx%d %s->%s dense=%d off=%d" % (seed, P, F, fmt, res, dense, off))
    nd = P * F // 2 if fmt == "e2m1" else P * F
    data = rng.integers(0, 256, size=nd, dtype=np.uint8)
    sshape = (P // 8, F // 4) if dense else (P, F // 4)
    image = rng.integers(0, 256, size=sshape, dtype=np.uint8)
    d = torch.from_numpy(data.reshape(mxq.data_shape(P, F, fmt))).cuda()
    im = torch.from_numpy(image).cuda()
    esz = 4 if res == "f32" else 2
    rbuf, r = _buf(P * F * esz, off)
    rt = r.view(torch.float32 if res == "f32" else torch.bfloat16).view(P, F)
    mxq.dequantize(d, im, fmt, rt.dtype, out=rt, dense_scale=dense)
    torch.cuda.synchronize()
    got = _guards(rbuf, off, P * F * esz, "result")
    ref = oracle.dequantize(data, image, P, F, fmt, res, layout="dense" if dense else "image")
    got = got.view(np.uint32 if res == "f32" else np.uint16).reshape(P, F)
    refb = ref.view(np.uint32) if res == "f32" else ref
    if res == "f32":
        nan_g, nan_r = (got & 0x7FFFFFFF) > 0x7F800000, (refb & 0x7FFFFFFF) > 0x7F800000
    else:
        nan_g, nan_r = (got & 0x7FFF) > 0x7F80, (refb & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_g, nan_r), "NaN positions differ"
    assert np.array_equal(got[~nan_g], refb[~nan_r]), "results differ"


@pytest.mark.parametrize("seed", range(16))
def test_random_quantize_axis(seed):
    rng = np.random.default_rng(3000 + seed)
    dim = int(rng.choice([-1, -2]))
    if dim == -2:
        R, C = 32 * int(rng.integers(1, 12)), _cols(rng) // 4 * int(rng.choice([1, 2, 4])) + int(rng.integers(0, 4))
        C = max(1, C)
    else:
        R, C = int(rng.integers(1, 600)), 32 * int(rng.integers(1, 24))
    in_dtype, out = str(rng.choice(["bf16", "f16"])), str(rng.choice(FMTS))
    off = int(rng.choice([0, 16, 48, 112]))
    progress("random quantize_axis seed=%d dim=%d %dx%d %s->%s off=%d" % (seed, dim, R, C, in_dtype, out, off))
    x = workloads.random_bits(R, C, in_dtype, seed=seed, specials=True)
    xt = torch.from_numpy(x.view(np.int16)).view(TDT[in_dtype]).cuda()
    VP, VF = mxq.axis_view_shape(R, C, dim)
    nd = int(np.prod(mxq.data_shape(VP, VF, out)))
    sshape = mxq.scale_image_shape(VP, VF)
    dbuf, d = _buf(nd, off)
    sbuf = torch.full(sshape, SENT, dtype=torch.uint8, device="cuda")
    mxq.quantize_axis(xt, out, dim, data_out=d, scale_out=sbuf)
    torch.cuda.synchronize()
    got_d = _guards(dbuf, off, nd, "data")
    got_s = sbuf.cpu().numpy()
    ref_d, ref_s = oracle.quantize_axis(x, in_dtype, out, dim)
    assert np.array_equal(got_d, ref_d.reshape(-1)), "data differs"
    placed = np.zeros(VP, bool)
    placed[(np.arange(VP // 8) % 4) + 32 * (np.arange(VP // 8) // 4)] = True
    assert (got_s[~placed] == SENT).all(), "an unplaced scale row was written"
    assert np.array_equal(got_s[placed], ref_s[placed]), "scales differ"
