"""The quantize and dequantize launch nothing but their kernel, so a caller
can capture them in a HIP graph. Each replay is checked against the eager
result, with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import mx_microscaling_quantization_amd as mxq
import workloads

pytestmark = pytest.mark.gpu


def test_graph_capture_and_replay():
    P, F = 1024, 4096
    x = workloads.random_bits(P, F, "bf16", seed=91, specials=True)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    data = torch.zeros((P, F), dtype=torch.uint8, device="cuda")
    image = torch.zeros((P, F // 4), dtype=torch.uint8, device="cuda")
    back = torch.zeros((P, F), dtype=torch.bfloat16, device="cuda")

    # eager reference
    d_ref, im_ref = mxq.quantize(xt, "e4m3fn", scale_out=image.clone())
    b_ref = mxq.dequantize(d_ref, im_ref, "e4m3fn", torch.bfloat16)
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm the binding on the capture stream
        mxq.quantize(xt, "e4m3fn", data_out=data, scale_out=image)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.quantize(xt, "e4m3fn", data_out=data, scale_out=image)
        mxq.dequantize(data, image, "e4m3fn", torch.bfloat16, out=back)

    for rep in range(4):
        data.zero_()
        back.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(data, d_ref), "replay %d data" % rep
        assert torch.equal(image.view(P // 32, 32, F // 4)[:, :4], im_ref.view(P // 32, 32, F // 4)[:, :4])
        assert torch.equal(back.view(torch.int16), b_ref.view(torch.int16)), "replay %d dequantize" % rep
        # unrelated eager work between replays
        _ = (xt.float() * 2).sum().item()


def test_graph_capture_every_entry_point():
    """Axis quantize (both axes), scaled matmul, quantize-on-produce and a
    quantize large enough for the occupancy-capped launch (its traffic
    exceeds the cache, so the launch reserves LDS): all captured in one
    graph, every replay equal to the eager results."""
    g_ = torch.Generator(device="cuda")
    g_.manual_seed(11)
    big = torch.randn((8192, 16384), generator=g_, device="cuda").to(torch.bfloat16)
    X = torch.randn((264, 512), generator=g_, device="cuda").to(torch.bfloat16)
    W = torch.randn((512, 136), generator=g_, device="cuda").to(torch.bfloat16)

    def run(outs=None):
        o = outs or {}
        d_big, s_big = mxq.quantize(big, "e4m3fn", data_out=o.get("d_big"), scale_out=o.get("s_big"))
        dl, sl = mxq.quantize_axis(X, "e4m3fn", -1, data_out=o.get("dl"), scale_out=o.get("sl"))
        dr, sr = mxq.quantize_axis(W, "e4m3fn", -2, data_out=o.get("dr"), scale_out=o.get("sr"))
        mm = mxq.scaled_matmul(dl, sl, dr, sr, "e4m3fn", torch.float32, out=o.get("mm"))
        qd, qs = mxq.scaled_matmul_quantize(dl, sl, dr, sr, "e4m3fn", "e4m3fn", data_out=o.get("qd"),
                                            scale_out=o.get("qs"))
        return {"d_big": d_big, "s_big": s_big, "dl": dl, "sl": sl, "dr": dr, "sr": sr, "mm": mm, "qd": qd,
                "qs": qs}

    ref = {k: v.clone() for k, v in run().items()}
    torch.cuda.synchronize()
    bufs = {k: torch.zeros_like(v) for k, v in ref.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(bufs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(bufs)
    for rep in range(4):
        for v in bufs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("d_big", "dl", "dr", "qd"):
            assert torch.equal(bufs[k], ref[k]), "replay %d: %s" % (rep, k)
        assert torch.equal(bufs["mm"].view(torch.int32), ref["mm"].view(torch.int32)), "replay %d: matmul" % rep
        # scale images: compare the placed rows (the others are never written)
        for k in ("s_big", "sl", "sr", "qs"):
            P = bufs[k].shape[0]
            rows = torch.tensor([(i % 4) + 32 * (i // 4) for i in range(P // 8)], device="cuda")
            assert torch.equal(bufs[k][rows], ref[k][rows]), "replay %d: %s" % (rep, k)
        _ = (X.float() * 2).sum().item()


def test_graph_capture_line_owning_launches():
    """The line-owning launches on row pitches that are not a multiple of
    128 bytes (FP8 quantize, dequantize to bf16 and f32, quantize down the
    columns): captured in one graph, every replay equal to the eager
    results."""
    g_ = torch.Generator(device="cuda")
    g_.manual_seed(12)
    P, F = 512, 8200
    x = torch.randn((P, F), generator=g_, device="cuda").to(torch.bfloat16)
    W = torch.randn((256, 1000), generator=g_, device="cuda").to(torch.bfloat16)
    data = torch.zeros((P, F), dtype=torch.uint8, device="cuda")
    image = torch.zeros((P, F // 4), dtype=torch.uint8, device="cuda")
    bf = torch.zeros((P, F), dtype=torch.bfloat16, device="cuda")
    f32 = torch.zeros((P, F), dtype=torch.float32, device="cuda")
    VP, VF = mxq.axis_view_shape(256, 1000, -2)
    wd = torch.zeros(mxq.data_shape(VP, VF, "e4m3fn"), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(mxq.scale_image_shape(VP, VF), dtype=torch.uint8, device="cuda")

    def calls():
        mxq.quantize(x, "e4m3fn", data_out=data, scale_out=image)
        mxq.dequantize(data, image, "e4m3fn", torch.bfloat16, out=bf)
        mxq.dequantize(data, image, "e4m3fn", torch.float32, out=f32)
        mxq.quantize_axis(W, "e4m3fn", -2, data_out=wd, scale_out=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (data, image, bf, f32, wd, ws)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for t in (data, bf, f32, wd):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("data", "image", "bf16", "f32", "axis data", "axis scale"),
                                   (data, image, bf, f32, wd, ws), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), "replay %d: %s" % (rep, name)
        _ = (x.float() * 2).sum().item()
