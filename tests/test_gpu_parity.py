"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact on both outputs (quantized codes are integer results). Every case
also checks that the scale image rows the placement does not name keep their
sentinel and that nothing is written past the end of the data buffer.
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
EMAX = {"e2m1": 2, "e4m3fn": 8, "e5m2": 15}
COMBOS = [(i, o) for i in ("bf16", "f16") for o in ("e4m3fn", "e5m2", "e2m1")]
SENTINEL = 0xA5
GUARD = 256


def to_device(x: np.ndarray, in_dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(TDT[in_dtype]).to("cuda")


def gpu_quantize(xt: torch.Tensor, out: str, stream=None, alt: bool = False, dense: bool = False):
    """Quantize through the binding into guarded, sentinel-filled buffers.
    Returns numpy (data, scale) after checking the guard bands."""
    P, F = xt.shape
    nbytes = mxq.data_bytes(P, F, out)
    buf = torch.full((nbytes + GUARD,), 0xEE, dtype=torch.uint8, device=xt.device)
    data = buf[:nbytes].view(mxq.data_shape(P, F, out))
    sshape = mxq.scale_image_shape(P, F, dense)
    sbytes = sshape[0] * sshape[1]
    sbuf = torch.full((sbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=xt.device)
    image = sbuf[:sbytes].view(sshape)
    mxq.quantize(xt, out, data_out=data, scale_out=image, stream=stream, alt_emax=alt, dense_scale=dense)
    torch.cuda.synchronize()
    assert np.all(buf[nbytes:].cpu().numpy() == 0xEE), "write past the end of the data buffer"
    assert np.all(sbuf[sbytes:].cpu().numpy() == SENTINEL), "write past the end of the scale buffer"
    return data.cpu().numpy(), image.cpu().numpy()


def check_against_oracle(x: np.ndarray, in_dtype: str, out: str, tag: str, alt: bool = False,
                         dense: bool = False):
    progress("%s %s->%s shape=%s alt=%d dense=%d" % (tag, in_dtype, out, x.shape, alt, dense))
    d_gpu, im_gpu = gpu_quantize(to_device(x, in_dtype), out, alt=alt, dense=dense)
    layout = "dense" if dense else "image"
    fill = np.full(oracle.scale_shape(x.shape[0], x.shape[1], layout), SENTINEL, np.uint8)
    d_ref, im_ref = oracle.quantize(x, in_dtype, out, image=fill, alt_emax=alt, layout=layout)
    if not np.array_equal(d_gpu, d_ref):
        bad = np.argwhere(d_gpu != d_ref)
        r, c = bad[0]
        raise AssertionError("%s: %d data bytes differ, first at %s: gpu %#x oracle %#x"
                             % (tag, len(bad), (r, c), d_gpu[r, c], d_ref[r, c]))
    if not np.array_equal(im_gpu, im_ref):
        bad = np.argwhere(im_gpu != im_ref)
        r, c = bad[0]
        raise AssertionError("%s: %d scale bytes differ, first at %s: gpu %#x oracle %#x"
                             % (tag, len(bad), (r, c), im_gpu[r, c], im_ref[r, c]))


# ---------------------------------------------------------------- small shapes

SHAPES = [(8, 4), (8, 8), (16, 12), (40, 8), (40, 12), (64, 96), (8, 2056), (264, 1032),
          (136, 2052), (256, 4100), (32, 8192), (1032, 520)]


@pytest.mark.parametrize("in_dtype,out", COMBOS)
@pytest.mark.parametrize("P,F", SHAPES)
def test_shapes_with_specials(in_dtype, out, P, F):
    x = workloads.random_bits(P, F, in_dtype, seed=P * 7919 + F, specials=True)
    check_against_oracle(x, in_dtype, out, "shape")


@pytest.mark.parametrize("in_dtype,out", COMBOS)
def test_nonfinite_blocks(in_dtype, out):
    P, F = 32, 64
    x = workloads.random_bits(P, F, in_dtype, seed=5)
    inf = 0x7F80 if in_dtype == "bf16" else 0x7C00
    nan = 0x7FC0 if in_dtype == "bf16" else 0x7E00
    b = x.reshape(P // 8, 8, F // 4, 4)
    b[0, 0, 0, 0] = inf                  # +Inf with finite neighbours
    b[0, 1, 1, 2] = inf | 0x8000         # -Inf
    b[1, 3, 2, 1] = nan                  # NaN
    b[1, 4, 3, 0] = nan | 0x8000         # -NaN
    b[2, :, 4, :] = nan                  # all NaN
    b[2, :, 5, :] = inf | 0x8000         # all -Inf
    b[3, 0, 6, 0] = nan
    b[3, 0, 6, 1] = inf                  # NaN and Inf together
    check_against_oracle(x, in_dtype, out, "nonfinite")


def _pilot_sweep(in_dtype: str) -> np.ndarray:
    """Blocks that put every input pattern under every scale it can meet:
    for each reachable block maximum exponent m, one pilot element with
    exponent m and every pattern whose exponent is at most m, 31 per block."""
    h = np.arange(65536, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        f32 = workloads.bf16_bits_to_f32(h) if in_dtype == "bf16" else h.view(np.float16).astype(np.float32)
    ex = (f32.view(np.uint32) >> 23) & 0xFF
    blocks = []
    for m in np.unique(ex):
        pilot = h[(ex == m) & (h < 0x8000)][0]
        cand = h[ex <= m]
        pad = (-cand.size) % 31
        cand = np.concatenate([cand, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((cand.shape[0], 1), pilot, np.uint16), cand], axis=1))
    blocks = np.concatenate(blocks)
    ncb = 256
    nrg = -(-blocks.shape[0] // ncb)
    blocks = np.concatenate([blocks, np.zeros((nrg * ncb - blocks.shape[0], 32), np.uint16)])
    # block b -> row group b // ncb, column block b % ncb; element k -> (k // 4, k % 4)
    return blocks.reshape(nrg, ncb, 8, 4).transpose(0, 2, 1, 3).reshape(nrg * 8, ncb * 4)


@pytest.mark.parametrize("alt", (False, True))
@pytest.mark.parametrize("in_dtype,out", COMBOS)
def test_exhaustive_pattern_scale_sweep(in_dtype, out, alt):
    x = _pilot_sweep(in_dtype)
    check_against_oracle(x, in_dtype, out, "sweep", alt=alt)


MODES = [(True, False), (False, True), (True, True)]


@pytest.mark.parametrize("alt,dense", MODES)
@pytest.mark.parametrize("in_dtype,out", COMBOS)
@pytest.mark.parametrize("P,F", [(8, 4), (40, 12), (264, 1032), (136, 2052)])
def test_modes_with_specials(in_dtype, out, P, F, alt, dense):
    x = workloads.random_bits(P, F, in_dtype, seed=P * 31 + F, specials=True)
    check_against_oracle(x, in_dtype, out, "mode", alt=alt, dense=dense)


@pytest.mark.parametrize("dense", (False, True))
def test_alt_emax_fp4_nonfinite_blocks(dense):
    """E8M0 254: every element of a block holding Inf/NaN is a zero of its sign."""
    P, F = 16, 16
    x = workloads.random_bits(P, F, "bf16", seed=12)
    b = x.reshape(P // 8, 8, F // 4, 4)
    b[0, 0, 0, 0] = 0x7F80
    b[0, 3, 1, 1] = 0xFF80
    b[1, 2, 2, 3] = 0xFFC0
    b[1, 7, 3, 0] = 0x7FC0
    check_against_oracle(x, "bf16", "e2m1", "alt-nonfinite", alt=True, dense=dense)


# ------------------------------------------------------------------ workloads

def test_workload_bf16_128x512_handplaced():
    check_against_oracle(workloads.handplaced_bf16_128x512(), "bf16", "e4m3fn", "bf16-128x512-handplaced")


@pytest.mark.parametrize("out", ["e4m3fn", "e5m2"])
def test_workload_bf16_4096x4096_rowscaled(out):
    check_against_oracle(workloads.rowscaled_bf16(), "bf16", out, "bf16-4096x4096-rowscaled")


def test_workload_f16_8192x14336_student_t():
    check_against_oracle(workloads.student_t_f16(), "f16", "e5m2", "f16-8192x14336-student-t")


def test_workload_bf16_16384x8192_blockexp():
    check_against_oracle(workloads.blockexp_bf16(), "bf16", "e2m1", "bf16-16384x8192-blockexp")


def _whole_tensor_check(xt: torch.Tensor, out: str, tag: str) -> np.ndarray:
    """Quantize a large bf16 device tensor in one call and compare every data
    byte and every scale image row (placed rows against the oracle, unplaced
    rows against their sentinel) with the oracle, run over whole 32-row bands
    on the host's threads. Returns the GPU's scale image."""
    from bands import run_bands

    P, F = xt.shape
    progress("%s: quantize" % tag)
    data = torch.empty(mxq.data_shape(P, F, out), dtype=torch.uint8, device="cuda")
    image = torch.full((P, F // 4), SENTINEL, dtype=torch.uint8, device="cuda")
    mxq.quantize(xt, out, data_out=data, scale_out=image)
    torch.cuda.synchronize()
    progress("%s: copy to host" % tag)
    x = xt.view(torch.int16).cpu().numpy().view(np.uint16)
    d_gpu, im_gpu = data.cpu().numpy(), image.cpu().numpy()
    del data, image
    oracle.quantize(np.zeros((8, 4), np.uint16), "bf16", out)     # load the library before the threads
    progress("%s: whole-tensor oracle compare" % tag)

    def check(r0, r1):
        fill = np.full((r1 - r0, F // 4), SENTINEL, np.uint8)
        d_ref, im_ref = oracle.quantize(x[r0:r1], "bf16", out, image=fill)
        if not np.array_equal(d_gpu[r0:r1], d_ref):
            r, c = np.argwhere(d_gpu[r0:r1] != d_ref)[0]
            return "data differs at (%d, %d): gpu %#x oracle %#x" % (r0 + r, c, d_gpu[r0 + r, c], d_ref[r, c])
        if not np.array_equal(im_gpu[r0:r1], im_ref):
            r, c = np.argwhere(im_gpu[r0:r1] != im_ref)[0]
            return "scale image differs at (%d, %d): gpu %#x oracle %#x" % (r0 + r, c, im_gpu[r0 + r, c], im_ref[r, c])
        return None

    bad = run_bands(P, check)
    assert not bad, "%s: %d slabs differ; first: %s" % (tag, len(bad), bad[0])
    return im_gpu


def test_workload_bf16_131072x8192_colscaled():
    """Full size, same call as the bench, every output byte compared."""
    P, F = 131072, 8192
    progress("bf16-131072x8192-colscaled: generate on device")
    xt = workloads.colscaled_bf16_device(P, F, seed=5)
    im_gpu = _whole_tensor_check(xt, "e4m3fn", "bf16-131072x8192-colscaled")
    # the input is finite: every placed scale is in range
    placed = im_gpu.reshape(P // 32, 32, F // 4)[:, :4, :]
    assert int(placed.min()) >= 1 and int(placed.max()) <= 254 - 8


# ------------------------------------------------------ misaligned row pitches

# FP8 codes on a pitch of F % 8 == 0, F % 128 != 0 bytes: each workgroup owns
# 48 two-block strips (384 bytes a row), also quantizes the next 16, and
# writes the 128-byte lines that start inside its own strips. These pitches
# put the run boundaries at many offsets within a line, and include one strip
# past a run (49 strips), a run ending at the row's end, several runs per
# row, and a single short run.
OWN_SHAPES = [(72, 392), (24, 776), (16, 8200), (8, 8208), (40, 3080), (32, 1160), (8, 120), (264, 1544)]


@pytest.mark.parametrize("in_dtype,out", COMBOS)
@pytest.mark.parametrize("P,F", OWN_SHAPES)
def test_misaligned_pitch_line_ownership(in_dtype, out, P, F):
    x = workloads.random_bits(P, F, in_dtype, seed=P * 131 + F, specials=True)
    check_against_oracle(x, in_dtype, out, "own-lines")


@pytest.mark.parametrize("offset", (16, 48, 112))
@pytest.mark.parametrize("out", ("e4m3fn", "e2m1"))
def test_output_pointers_off_a_line(out, offset):
    """Data and scale buffers that start `offset` bytes into a 128-byte line:
    the line ownership follows the absolute addresses; nothing is written
    before or after either buffer."""
    P, F = 64, 1032
    x = workloads.random_bits(P, F, "bf16", seed=offset, specials=True)
    xt = to_device(x, "bf16")
    nbytes = mxq.data_bytes(P, F, out)
    buf = torch.full((offset + nbytes + GUARD,), 0xEE, dtype=torch.uint8, device="cuda")
    data = buf[offset:offset + nbytes].view(mxq.data_shape(P, F, out))
    sbytes = P * (F // 4)
    sbuf = torch.full((offset + sbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
    image = sbuf[offset:offset + sbytes].view(P, F // 4)
    progress("pointer offset %d bf16->%s %dx%d" % (offset, out, P, F))
    mxq.quantize(xt, out, data_out=data, scale_out=image)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    sb = sbuf.cpu().numpy()
    assert np.all(b[:offset] == 0xEE) and np.all(b[offset + nbytes:] == 0xEE)
    assert np.all(sb[:offset] == SENTINEL) and np.all(sb[offset + sbytes:] == SENTINEL)
    fill = np.full((P, F // 4), SENTINEL, np.uint8)
    d_ref, im_ref = oracle.quantize(x, "bf16", out, image=fill)
    assert np.array_equal(b[offset:offset + nbytes].reshape(d_ref.shape), d_ref)
    assert np.array_equal(sb[offset:offset + sbytes].reshape(P, F // 4), im_ref)


@pytest.mark.parametrize("F,out", [(8200, "e4m3fn"), (8208, "e5m2"), (8188, "e4m3fn"), (8200, "e2m1")])
def test_misaligned_pitch_16384_rows_whole(F, out):
    """16384 rows on misaligned pitches (line-owning FP8 path; one-block
    strips at F % 8 == 4; FP4), every output byte compared."""
    P = 16384
    progress("bf16-%dx%d: generate on device" % (P, F))
    xt = workloads.colscaled_bf16_device(P, F, seed=F)
    _whole_tensor_check(xt, out, "bf16-%dx%d->%s" % (P, F, out))


# --------------------------------------------------------------- other checks

def test_bare_c_entry_point_on_device():
    """mxq_quantize itself, called through ctypes with raw device pointers
    and a raw stream handle (no binding logic), on the hand-placed
    128 x 512 workload: bit-exact against the oracle, both outputs."""
    import ctypes

    lib = mxq.load()
    x = workloads.handplaced_bf16_128x512()
    P, F = x.shape
    xt = to_device(x, "bf16")
    data = torch.full((P, F), 0xEE, dtype=torch.uint8, device="cuda")
    image = torch.full((P, F // 4), SENTINEL, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    progress("bare mxq_quantize 128x512 bf16->e4m3fn")
    rc = lib.mxq_quantize(ctypes.c_void_p(xt.data_ptr()), ctypes.c_int64(P), ctypes.c_int64(F), 0, 0,
                          ctypes.c_void_p(data.data_ptr()), ctypes.c_void_p(image.data_ptr()),
                          ctypes.c_void_p(s.cuda_stream))
    assert rc == 0, lib.mxq_status_string(rc)
    s.synchronize()
    fill = np.full((P, F // 4), SENTINEL, np.uint8)
    d_ref, im_ref = oracle.quantize(x, "bf16", "e4m3fn", image=fill)
    assert np.array_equal(data.cpu().numpy(), d_ref)
    assert np.array_equal(image.cpu().numpy(), im_ref)
    # an invalid call through the same symbol returns its status and writes nothing
    rc = lib.mxq_quantize(ctypes.c_void_p(xt.data_ptr()), ctypes.c_int64(P - 4), ctypes.c_int64(F), 0, 0,
                          ctypes.c_void_p(data.data_ptr()), ctypes.c_void_p(image.data_ptr()), None)
    assert rc == 3
    torch.cuda.synchronize()
    assert np.array_equal(data.cpu().numpy(), d_ref)



def test_deterministic_across_runs_and_streams():
    x = workloads.random_bits(1024, 4096, "bf16", seed=9, specials=True)
    xt = to_device(x, "bf16")
    ref = gpu_quantize(xt, "e4m3fn")
    s = torch.cuda.Stream()
    for k in range(5):
        got = gpu_quantize(xt, "e4m3fn", stream=s if k % 2 else None)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_empty_and_misaligned_on_device():
    for shape in ((0, 8), (8, 0)):
        xt = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        d, im = mxq.quantize(xt, "e4m3fn")
        assert d.numel() == 0 or im.numel() == 0
    flat = torch.zeros(8 * 8 + 1, dtype=torch.bfloat16, device="cuda")
    xt = flat[1:].view(8, 8)
    with pytest.raises(mxq.MXQError) as ei:
        mxq.quantize(xt, "e4m3fn")
    assert ei.value.status == 6


def test_outputs_on_caller_stream():
    """The kernel is enqueued on the given stream: work queued behind a
    long-running op on that stream sees the op's result."""
    x = workloads.random_bits(512, 2048, "f16", seed=10)
    xt = to_device(x, "f16")
    s = torch.cuda.Stream()
    src = torch.zeros_like(xt)
    with torch.cuda.stream(s):
        src.copy_(xt)        # queued on s before the quantize
        d, im = mxq.quantize(src, "e5m2")
    s.synchronize()
    d_ref, _ = oracle.quantize(x, "f16", "e5m2")
    assert np.array_equal(d.cpu().numpy(), d_ref)


def test_binding_uses_the_current_stream():
    """Without a stream argument the binding enqueues on the device's current
    stream, whichever way it reads it: the handle it passes equals torch's,
    on the default stream and inside a stream context."""
    dev = torch.device("cuda", torch.cuda.current_device())
    assert mxq._stream_handle(None, dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert mxq._stream_handle(None, dev) == s.cuda_stream != torch.cuda.default_stream(dev).cuda_stream
    assert mxq._stream_handle(s, dev) == s.cuda_stream


def test_concurrent_host_threads():
    """The library keeps no state: host threads calling it at the same time,
    each on its own stream, get the bytes a serial call gives."""
    import concurrent.futures

    cases = [(workloads.random_bits(256 + 64 * k, 1024, "bf16", seed=40 + k, specials=True), out)
             for k, out in enumerate(("e4m3fn", "e5m2", "e2m1", "e4m3fn"))]
    inputs = [(to_device(x, "bf16"), out) for x, out in cases]
    serial = []
    for xt, out in inputs:
        d, im = mxq.quantize(xt, out)
        torch.cuda.synchronize()
        serial.append((d.cpu().numpy(), im.cpu().numpy()))
    progress("quantize from 4 host threads, 4 streams, 8 rounds")

    def work(k):
        xt, out = inputs[k]
        s = torch.cuda.Stream()
        got = []
        for _ in range(8):
            with torch.cuda.stream(s):
                d, im = mxq.quantize(xt, out, stream=s)
            got.append((d, im))
        s.synchronize()
        return [(d.cpu().numpy(), im.cpu().numpy()) for d, im in got]

    with concurrent.futures.ThreadPoolExecutor(4) as ex:
        results = list(ex.map(work, range(4)))
    for k, rounds in enumerate(results):
        for d, im in rounds:
            assert np.array_equal(d, serial[k][0])
            # only the placed rows are defined (the image was allocated empty)
            P = inputs[k][0].shape[0]
            placed = (np.arange(P // 8) % 4) + 32 * (np.arange(P // 8) // 4)
            assert np.array_equal(im[placed], serial[k][1][placed])


@pytest.mark.parametrize("F,out", [(4096, "e4m3fn"), (4104, "e5m2"), (4100, "e2m1"), (8200, "e4m3fn")])
def test_grid_shape_invariance(F, out):
    """The same rows give the same bytes whatever grid covers them: the whole
    tensor in one call against slabs of whole 32-row bands in separate calls
    (each a different grid), with dense scales so the slabs' scale rows are
    the whole tensor's rows; the dequantize likewise. Ten repeats of the whole
    call are identical."""
    P = 1024
    x = workloads.random_bits(P, F, "bf16", seed=F, specials=True)
    xt = to_device(x, "bf16")
    d_all, s_all = mxq.quantize(xt, out, dense_scale=True)
    r_all = mxq.dequantize(d_all, s_all, out, torch.float32, dense_scale=True)
    torch.cuda.synchronize()
    for _ in range(9):
        d2, s2 = mxq.quantize(xt, out, dense_scale=True)
        assert torch.equal(d2, d_all) and torch.equal(s2, s_all)
    for r0, r1 in ((0, 32), (32, 288), (288, 800), (800, 1024)):
        d, s = mxq.quantize(xt[r0:r1].contiguous(), out, dense_scale=True)
        r = mxq.dequantize(d, s, out, torch.float32, dense_scale=True)
        torch.cuda.synchronize()
        assert torch.equal(d, d_all[r0:r1]), "data rows [%d, %d)" % (r0, r1)
        assert torch.equal(s, s_all[r0 // 8:r1 // 8]), "scale rows [%d, %d)" % (r0 // 8, r1 // 8)
        assert torch.equal(r.view(torch.int32), r_all[r0:r1].view(torch.int32)), "dequantized rows"
