"""GPU parity of the quantize along either axis of a row-major tensor
(mxq_quantize_axis) against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import mx_microscaling_quantization_amd as mxq
import oracle
import workloads
from conftest import progress

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5
GUARD = 64

IN_T = {"bf16": torch.bfloat16, "f16": torch.float16}


def _device(bits: np.ndarray, in_dtype: str) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(IN_T[in_dtype]).cuda()


def _view_on_device(x: torch.Tensor, dim: int) -> torch.Tensor:
    """torch re-layout into the [K/4, 4*O] view (an independent route)."""
    if dim in (-1, 1):
        O, K = x.shape
        return x.reshape(O, K // 4, 4).permute(1, 0, 2).reshape(K // 4, 4 * O).contiguous()
    K, O = x.shape
    return x.reshape(K // 4, 4, O).permute(0, 2, 1).reshape(K // 4, 4 * O).contiguous()


def run(bits, in_dtype, fmt, dim, alt=False, dense=False):
    R, C = bits.shape
    P, F = mxq.axis_view_shape(R, C, dim)
    layout = "dense" if dense else "image"
    nd = int(np.prod(mxq.data_shape(P, F, fmt)))
    data = torch.full((nd + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
    scale = torch.full(mxq.scale_image_shape(P, F, dense), SENTINEL, dtype=torch.uint8, device="cuda")
    x = _device(bits, in_dtype)
    mxq.quantize_axis(x, fmt, dim, data_out=data, scale_out=scale, alt_emax=alt, dense_scale=dense)
    torch.cuda.synchronize()
    got = data.cpu().numpy()
    assert (got[nd:] == SENTINEL).all(), "write past the data buffer"
    got_d = got[:nd].reshape(mxq.data_shape(P, F, fmt))
    got_s = scale.cpu().numpy()
    ref_d, ref_s = oracle.quantize_axis(bits, in_dtype, fmt, dim, alt_emax=alt, layout=layout)
    if not dense:
        placed = np.zeros(P, bool)
        placed[(np.arange(P // 8) % 4) + 32 * (np.arange(P // 8) // 4)] = True
        assert (got_s[~placed] == SENTINEL).all(), "an unplaced scale row was written"
        got_s = np.where(placed[:, None], got_s, 0)
    assert np.array_equal(got_d, ref_d), "data differs at %s" % (np.argwhere(got_d != ref_d)[:3].tolist(),)
    assert np.array_equal(got_s, ref_s), "scales differ at %s" % (np.argwhere(got_s != ref_s)[:3].tolist(),)
    return x


# dim -1 rows (R) cover both store widths (R % 4 == 0: 16/8-byte stores; else
# one row per lane), partial 256-row tiles and odd block counts (C/32 odd:
# the last tile holds one block); the last three have grids of 272, 90 and
# 102 workgroups with R % 256 != 0, so whole 32-workgroup windows are
# renumbered and a tail is not
SHAPES = [(-2, 32, 4), (-2, 64, 36), (-2, 96, 64), (-2, 128, 130), (-2, 256, 257), (-2, 1024, 1000),
          (-1, 13, 96), (-1, 64, 64), (-1, 100, 256), (-1, 1000, 512), (-1, 7, 32), (1, 70, 160), (0, 160, 70),
          (-1, 4, 32), (-1, 260, 96), (-1, 516, 1056), (-1, 1001, 160), (-1, 256, 64),
          (-1, 4100, 1024), (-1, 2050, 640), (-1, 4104, 352)]


@pytest.mark.parametrize("in_dtype,fmt", [("bf16", "e4m3fn"), ("bf16", "e5m2"), ("bf16", "e2m1"),
                                          ("f16", "e4m3fn"), ("f16", "e5m2"), ("f16", "e2m1")])
@pytest.mark.parametrize("dim,R,C", SHAPES)
def test_axis_against_oracle(dim, R, C, in_dtype, fmt):
    progress("quantize_axis dim=%d %dx%d %s->%s" % (dim, R, C, in_dtype, fmt))
    bits = workloads.random_bits(R, C, in_dtype, seed=R * 3 + C + dim, specials=True)
    run(bits, in_dtype, fmt, dim)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e2m1"])
@pytest.mark.parametrize("dim", [-1, -2])
@pytest.mark.parametrize("alt,dense", [(True, False), (False, True), (True, True)])
def test_axis_modes(dim, fmt, alt, dense):
    bits = workloads.random_bits(256, 192, "bf16", seed=5 + dim, specials=True)
    run(bits, "bf16", fmt, dim, alt=alt, dense=dense)


@pytest.mark.parametrize("dim", [-1, -2])
def test_axis_equals_plain_quantize_of_the_view(dim):
    bits = workloads.random_bits(512, 384, "bf16", seed=17, specials=True)
    x = _device(bits, "bf16")
    P, F = mxq.axis_view_shape(512, 384, dim)
    d, s = mxq.quantize_axis(x, "e5m2", dim, scale_out=torch.zeros((P, F // 4), dtype=torch.uint8, device="cuda"))
    d_ref, s_ref = mxq.quantize(_view_on_device(x, dim), "e5m2",
                                scale_out=torch.zeros((P, F // 4), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(d, d_ref) and torch.equal(s, s_ref)


def test_axis_quantize_feeds_the_matmul_as_x_times_w():
    """Small integers are exact in e4m3fn and in the matrix cores' sums:
    X [M, K] along its rows and W [K, N] down its columns multiply to X @ W
    exactly."""
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    M, K, N = 264, 512, 136
    X = torch.randint(-4, 5, (M, K), generator=g, device="cuda").to(torch.bfloat16)
    W = torch.randint(-4, 5, (K, N), generator=g, device="cuda").to(torch.bfloat16)
    dl, sl = mxq.quantize_axis(X, "e4m3fn", -1)
    dr, sr = mxq.quantize_axis(W, "e4m3fn", -2)
    out = mxq.scaled_matmul(dl, sl, dr, sr, "e4m3fn", torch.float32)
    ref = X.double().cpu() @ W.double().cpu()
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().double(), ref)


def test_axis_empty_is_noop():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    d, s = mxq.quantize_axis(x, "e4m3fn", -1)
    assert d.numel() == 0 and s.numel() == 0


@pytest.mark.parametrize("dim", [-2, -1])
def test_axis_full_size(dim):
    """The 1.07 G-element bench input quantized along each axis: all bytes
    against the plain GPU quantize of the torch-built view, and all bytes
    (data and placed scale rows) against the oracle's quantize_axis, run
    over slabs of whole 128-element stretches of the block axis (32 view
    rows, so each slab's scale rows are the global ones shifted) on the
    host's threads."""
    from bands import run_bands

    progress("quantize_axis full size dim=%d: input" % dim)
    x = workloads.colscaled_bf16_device(device="cuda")
    R, C = x.shape
    d, s = mxq.quantize_axis(x, "e4m3fn", dim)
    progress("quantize_axis full size dim=%d: view + plain quantize" % dim)
    v = _view_on_device(x, dim)
    d_ref, s_ref = mxq.quantize(v, "e4m3fn")
    torch.cuda.synchronize()
    del v
    assert torch.equal(d, d_ref)
    P = s.shape[0]
    placed = (np.arange(P // 8) % 4) + 32 * (np.arange(P // 8) // 4)
    assert torch.equal(s[torch.from_numpy(placed).cuda()], s_ref[torch.from_numpy(placed).cuda()])
    del d_ref, s_ref
    progress("quantize_axis full size dim=%d: copy to host" % dim)
    bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    del x
    hd, hs = d.cpu().numpy(), s.cpu().numpy()
    del d, s
    oracle.quantize_axis(bits[:32, :32].copy(), "bf16", "e4m3fn", dim)   # load the library before the threads
    progress("quantize_axis full size dim=%d: whole-tensor oracle compare" % dim)
    K = R if dim == -2 else C

    def check(v0, v1):
        # view rows [v0, v1) = block-axis elements [4 v0, 4 v1)
        k0, k1 = 4 * v0, 4 * v1
        part = bits[k0:k1] if dim == -2 else np.ascontiguousarray(bits[:, k0:k1])
        ref_d, ref_s = oracle.quantize_axis(part, "bf16", "e4m3fn", dim)
        if not np.array_equal(hd[v0:v1], ref_d):
            r, c = np.argwhere(hd[v0:v1] != ref_d)[0]
            return "data differs at view (%d, %d)" % (v0 + r, c)
        rows = placed[(placed >= 0) & (placed < v1 - v0)]
        if not np.array_equal(hs[v0 + rows], ref_s[rows]):
            return "scale rows differ in view rows [%d, %d)" % (v0, v1)
        return None

    bad = run_bands(K // 4, check)
    assert not bad, "%d slabs differ; first: %s" % (len(bad), bad[0])


# ---------------------------------------------- dim -2 on misaligned view rows

# Four-column strips on view rows of 4*C (FP8) or 2*C (FP4) bytes that are not
# a multiple of 128: each workgroup owns 56 (FP8) or 48 (FP4) strips, also
# quantizes the next 128 bytes' worth, and writes the lines that start inside
# its own strips. These put run boundaries at many offsets within a line,
# one or two strips past a run, and several runs per view row.
OWN_SHAPES = [(32, 232), (64, 196), (32, 452), (96, 900), (64, 8200), (32, 1000)]


@pytest.mark.parametrize("in_dtype,fmt", [("bf16", "e4m3fn"), ("bf16", "e5m2"), ("bf16", "e2m1"),
                                          ("f16", "e4m3fn"), ("f16", "e2m1")])
@pytest.mark.parametrize("R,C", OWN_SHAPES)
def test_axis_down_line_ownership(R, C, in_dtype, fmt):
    progress("quantize_axis own-lines dim=-2 %dx%d %s->%s" % (R, C, in_dtype, fmt))
    bits = workloads.random_bits(R, C, in_dtype, seed=R * 5 + C, specials=True)
    run(bits, in_dtype, fmt, -2)


@pytest.mark.parametrize("offset", (16, 48, 112))
@pytest.mark.parametrize("fmt", ("e4m3fn", "e2m1"))
def test_axis_down_pointer_off_a_line(fmt, offset):
    """A data buffer starting `offset` bytes into a 128-byte line: the line
    ownership follows the absolute addresses; nothing is written before or
    after the buffer."""
    R, C = 64, 1000
    bits = workloads.random_bits(R, C, "bf16", seed=offset, specials=True)
    P, F = mxq.axis_view_shape(R, C, -2)
    nd = int(np.prod(mxq.data_shape(P, F, fmt)))
    buf = torch.full((offset + nd + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
    scale = torch.full(mxq.scale_image_shape(P, F), SENTINEL, dtype=torch.uint8, device="cuda")
    progress("quantize_axis dim=-2 pointer offset %d %dx%d -> %s" % (offset, R, C, fmt))
    mxq.quantize_axis(_device(bits, "bf16"), fmt, -2, data_out=buf[offset:offset + nd], scale_out=scale)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert (got[:offset] == SENTINEL).all() and (got[offset + nd:] == SENTINEL).all(), "write outside the buffer"
    ref_d, _ = oracle.quantize_axis(bits, "bf16", fmt, -2)
    assert np.array_equal(got[offset:offset + nd].reshape(ref_d.shape), ref_d)


@pytest.mark.parametrize("fmt", ["e4m3fn", "e2m1"])
def test_axis_down_16384x8200_whole(fmt):
    """W [16384, 8200] down its columns (misaligned view rows, the owning
    path): every data byte and placed scale row against the oracle's
    quantize_axis over slabs of whole 128-row stretches on the host's
    threads."""
    from bands import run_bands

    R, C = 16384, 8200
    progress("quantize_axis dim=-2 %dx%d -> %s: input" % (R, C, fmt))
    x = workloads.colscaled_bf16_device(R, C, seed=13)
    d, s = mxq.quantize_axis(x, fmt, -2)
    torch.cuda.synchronize()
    bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
    del x
    hd, hs = d.cpu().numpy(), s.cpu().numpy()
    del d, s
    P = hs.shape[0]
    placed = (np.arange(P // 8) % 4) + 32 * (np.arange(P // 8) // 4)
    oracle.quantize_axis(bits[:32, :32].copy(), "bf16", fmt, -2)   # load the library before the threads
    progress("quantize_axis dim=-2 %dx%d -> %s: whole-tensor oracle compare" % (R, C, fmt))

    def check(v0, v1):
        ref_d, ref_s = oracle.quantize_axis(bits[4 * v0:4 * v1], "bf16", fmt, -2)
        if not np.array_equal(hd[v0:v1], ref_d):
            r, c = np.argwhere(hd[v0:v1] != ref_d)[0]
            return "data differs at view (%d, %d)" % (v0 + r, c)
        rows = placed[placed < v1 - v0]
        if not np.array_equal(hs[v0 + rows], ref_s[rows]):
            return "scale rows differ in view rows [%d, %d)" % (v0, v1)
        return None

    bad = run_bands(R // 4, check)
    assert not bad, "%d slabs differ; first: %s" % (len(bad), bad[0])
