#!/usr/bin/env python3
"""Throughput of the MX quantize on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--op quantize|dequantize|matmul|matmul_quantize|quantize_axis]
                    [--dim -1|-2] [--res bf16|f32] [--cache hot|flushed]
                    [--no-cpu-baseline] [--copy-calibration]

A step is one full quantize of the workload tensor (one kernel launch: block
scales, prescale, narrow, packing and scale placement). The input is
generated on the device before timing and stays resident in HBM. The timed
region is K back-to-back steps on one stream, bracketed by device
synchronisation and by two HIP events on that stream; with one launch per
step, the span over K is also the kernel's average launch duration for the
roofline. (An event pair around every launch would add about 7 us per step
to a 475 us quantize.)

Prints one JSON line. ``value`` is algorithmic GB/s over the timed region:
bytes per step = input (2 B/element) + data (1 B/element FP8, 0.5 B FP4) +
logical scale (1/32 B/element); the never-written scale-image rows are not
counted.

``--op dequantize`` times the inverse instead: the workload is quantized once
(untimed) and each step decodes it back to ``--res`` (bytes per step = data +
logical scale + result).

``--op matmul`` times the block-scaled matmul of two quantized e4m3fn
operands (M = N = 8192, K = 4P = 8192 by default; ``--mm M N K``) in
TFLOP/s against the matrix cores' dense FP8 peak.

``--op quantize_axis [--dim -1|-2]`` times the quantize of the same input as
a plain row-major tensor with its blocks along rows (-1) or down columns
(-2), written in the partition-major layout the matmul reads (same bytes
per step as the quantize).

``--op matmul_quantize`` times the same product with its result quantized
in the kernel's epilogue (format ``--out``, default e4m3fn), and reports the
unfused pair (bf16 matmul, then quantize) on the same operands beside it.

The matmul ops warm up with 200 untimed launches by default (the streaming
ops with 5): under sustained FP8 MFMA work the GPU clock first drops below
its steady value and takes some 30 ms of load to settle, so a short
warm-up would time that transient rather than the sustained rate.

With the CPU baseline on (the default), the quantize line carries two
figures for the oracle on the same input: ``cpu_baseline`` (one thread on
leading row slabs, about 12 s of oracle time) and ``cpu_baseline_all_cores``
(the whole tensor split into whole 32-row bands over up to 16 threads,
wall-clock time).

``--cache flushed`` (streaming ops) reads a 512 MiB buffer, twice the
Infinity Cache, before every launch, so no launch finds its operands cached;
each launch then gets its own pair of HIP events, and ``value`` and
``ms_per_step`` cover the launches alone (the sum of those spans), not the
flushes between them. The default, ``hot``,
runs the launches back to back on the same buffers: a workload under the
cache size is then served largely from the cache.

The streaming ops' lines also carry ``per_call`` (the median and minimum of
20 more calls, each between its own event pair) and ``copy_reference``: a
plain 1 GiB device copy timed after the measured steps, and the line's value
over its rate.

``--copy-calibration`` instead times a plain device copy of 2 GiB (read 2 GiB,
write 2 GiB); its hardware counters give the factor that turns FETCH_SIZE /
WRITE_SIZE readings into bytes. ``--floors`` times plain linear read, write
and copy streams (torch's own kernels) for comparison. ``--vendor-gemm`` times
the vendor's per-tensor-scaled FP8 product at the ``--mm`` sizes, for context
beside the block-scaled matmul.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MX quantize GB/s (in+out bytes) and % of HBM peak, 1 MI355X"
METRIC_DEQUANT = "MX dequantize GB/s (in+out bytes) and % of HBM peak, 1 MI355X"
METRIC_AXIS = "MX quantize along a tensor axis GB/s (in+out bytes) and % of HBM peak, 1 MI355X"
METRIC_MATMUL = "MX scaled matmul TFLOP/s (fp32 accumulate), 1 MI355X"
METRIC_MATMUL_QUANTIZE = "MX scaled matmul with quantized result TFLOP/s (fp32 accumulate), 1 MI355X"
MFMA_FP8_PEAK_TFLOPS = 5000.0
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "bf16-131072x8192-colscaled"
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "mx_microscaling_quantization_amd/csrc/"
# What determines each op's kernel and launch: its kernel header(s), its
# launch file and the shared host helpers.
KERNEL_SOURCES = {
    "quantize": [_CSRC + f for f in ("mxq_quantize_kernels.hpp", "mxq_quantize_api.hip", "mxq_host.hpp")],
    "dequantize": [_CSRC + f for f in ("mxq_quantize_kernels.hpp", "mxq_dequantize_kernels.hpp",
                                       "mxq_dequantize_api.hip", "mxq_host.hpp")],
    "matmul": [_CSRC + f for f in ("mxq_quantize_kernels.hpp", "mxq_matmul_kernels.hpp", "mxq_matmul_api.hip",
                                   "mxq_host.hpp")],
    "quantize_axis": [_CSRC + f for f in ("mxq_quantize_kernels.hpp", "mxq_axis_kernels.hpp", "mxq_axis_api.hip",
                                          "mxq_host.hpp")],
}
KERNEL_SOURCES["matmul_quantize"] = KERNEL_SOURCES["matmul"]


def algorithmic_bytes(P: int, F: int, out: str) -> int:
    n = P * F
    data = n // 2 if out == "e2m1" else n
    return 2 * n + data + n // 32


def dequant_bytes(P: int, F: int, fmt: str, res: str) -> int:
    n = P * F
    data = n // 2 if fmt == "e2m1" else n
    return data + n // 32 + n * (4 if res == "f32" else 2)


def kernel_source_digest(op: str = "quantize") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[op]:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, out: str, op: str = "quantize", res: str = ""):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources, and where that figure comes from:
    (bytes, source) or (None, source) -- the counters are read in runs of
    their own (rocprofv3 --pmc), never inside this timed run."""
    tag = "%s_%s_%s" % (op, workload, out) + ("_" + res if res else "")
    path = os.path.join(PROFILES, "%s_hbm_traffic.txt" % tag)
    digest = kernel_source_digest(op)
    source = {"kind": "committed rocprofv3 --pmc summary (FETCH_SIZE, WRITE_SIZE runs)",
              "file": os.path.relpath(path, ROOT), "kernel_source_sha256_16": digest,
              "matches_current_sources": False}
    if not os.path.exists(path):
        source["file"] = None
        return None, source
    text = open(path).read()
    m_src = re.search(r"^kernel_source_sha256_16:\s*(\S+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_src or not m_b or m_src.group(1) != digest:
        return None, source
    source["matches_current_sources"] = True
    return float(m_b.group(1)), source


def make_input(workload: str, device):
    import numpy as np
    import torch

    import workloads

    spec = workloads.WORKLOADS[workload]
    P, F = spec["P"], spec["F"]
    if workload in workloads.DEVICE_DRAWN:
        xt = workloads.colscaled_bf16_device(P, F, seed=spec["seed"], device=str(device))
    else:
        x = workloads.make_host(workload)
        tdt = torch.bfloat16 if spec["in_dtype"] == "bf16" else torch.float16
        xt = torch.from_numpy(x.view(np.int16)).view(tdt).to(device)
    return xt, spec


def host_cpu() -> dict:
    """The host the CPU baselines ran on: its processor model (from
    /proc/cpuinfo), the logical CPUs it reports and the ones this process
    may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count() or 1, "usable_cpus": usable}


def cpu_baseline(xt, out: str, in_dtype: str, budget_s: float = 12.0, slab_rows: int = 4096, dim: int | None = None):
    """The CPU oracle (single thread, as it stands) on leading row slabs of
    the same input until about budget_s seconds of oracle time (with dim,
    its quantize along that axis; slabs stay multiples of 32 rows)."""
    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    P, F = xt.shape
    done_rows, spent = 0, 0.0
    while done_rows < P and spent < budget_s:
        rows = min(slab_rows, P - done_rows)
        x = xt[done_rows:done_rows + rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        if dim is None:
            oracle.quantize(x, in_dtype, out)
        else:
            oracle.quantize_axis(x, in_dtype, out, dim)
        spent += time.perf_counter() - t0
        done_rows += rows
    nbytes = algorithmic_bytes(done_rows, F, out)
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host": host_cpu(),
            "sample": "first %d of %d rows (%d x %d, %.3g s of single-thread oracle time)"
                      % (done_rows, P, done_rows, F, spent)}


def cpu_baseline_all_cores(xt, out: str, in_dtype: str, max_threads: int = 16):
    """The same CPU oracle, unchanged, on every host core the run may use
    (at most max_threads): the whole input split into one slab of whole
    32-row bands per thread, each slab quantized by its own call (ctypes
    releases the interpreter lock during the call). Wall-clock time."""
    import concurrent.futures

    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    oracle.quantize(np.zeros((8, 4), np.uint16), in_dtype, out)   # load the library before the threads
    P, F = xt.shape
    host = xt.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    n = max(1, min(max_threads, os.cpu_count() or 1, P // 32))
    bands = P // 32
    cuts = [32 * (bands * t // n) for t in range(n)] + [P]

    def work(t):
        oracle.quantize(host[cuts[t]:cuts[t + 1]], in_dtype, out)

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        list(ex.map(work, range(n)))
    spent = time.perf_counter() - t0
    return {"value": round(algorithmic_bytes(P, F, out) / spent / 1e9, 4), "unit": "GB/s", "cores": n,
            "kind": "oracle", "host": host_cpu(),
            "sample": "all %d rows (%d x %d) in %d slabs on %d threads, %.3g s wall" % (P, P, F, n, n, spent)}


def cpu_baseline_dequant(data, image, fmt: str, res: str, budget_s: float = 12.0, slab_rows: int = 4096):
    """The CPU oracle's dequantize (single thread) on leading row slabs."""
    import oracle

    oracle.build(force=False)
    P = data.shape[0]
    F = image.shape[1] * 4
    done_rows, spent = 0, 0.0
    while done_rows < P and spent < budget_s:
        rows = min(slab_rows, P - done_rows)
        d = data[done_rows:done_rows + rows].cpu().numpy()
        im = image[done_rows:done_rows + rows].cpu().numpy()   # slabs start at multiples of 32 rows
        t0 = time.perf_counter()
        oracle.dequantize(d, im, rows, F, fmt, res)
        spent += time.perf_counter() - t0
        done_rows += rows
    nbytes = dequant_bytes(done_rows, F, fmt, res)
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host": host_cpu(),
            "sample": "first %d of %d rows (%d x %d, %.3g s of single-thread oracle time)"
                      % (done_rows, P, done_rows, F, spent)}


def cpu_baseline_matmul(dl, sl, dr, sr, fmt: str, budget_s: float = 10.0, block: int = 16,
                        quantize_out: str | None = None):
    """The CPU oracle's scaled matmul (single thread) on block x block output
    tiles along the diagonal until about budget_s seconds; with quantize_out,
    the oracle's matmul followed by its quantize of the tile."""
    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    P = dl.shape[0]
    M, N = dl.shape[1] // 4, dr.shape[1] // 4
    done, spent = 0, 0.0
    while spent < budget_s and (done + 1) * block <= min(M, N):
        c0 = done * block
        hl = dl[:, 4 * c0:4 * (c0 + block)].contiguous().cpu().numpy()
        hr = dr[:, 4 * c0:4 * (c0 + block)].contiguous().cpu().numpy()
        hsl = sl[:, c0:c0 + block].contiguous().cpu().numpy()
        hsr = sr[:, c0:c0 + block].contiguous().cpu().numpy()
        t0 = time.perf_counter()
        if quantize_out:
            oracle.scaled_matmul_quantize(hl, hsl, hr, hsr, fmt, quantize_out)
        else:
            oracle.scaled_matmul(hl, hsl, hr, hsr, fmt)
        spent += time.perf_counter() - t0
        done += 1
    flops = 2.0 * done * block * block * 4 * P
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "host": host_cpu(),
            "sample": "%d diagonal %dx%d output tiles at K=%d (%.3g s of single-thread oracle time)"
                      % (done, block, block, 4 * P, spent)}


MATMUL_WARMUP = 200


def default_warmup(op: str, warmup: int | None) -> int:
    """The warm-up to use: the one given, else 200 launches for the matmul
    ops (whose clock takes that long to settle under FP8 MFMA load) and 5
    for the streaming ops."""
    if warmup is not None:
        return warmup
    return MATMUL_WARMUP if op in ("matmul", "matmul_quantize") else 5


def _time_steps(step, steps: int, warmup: int, stream, pre=None):
    """Time `steps` calls of `step` on `stream` after `warmup` untimed ones.

    Without `pre` the steps run back to back between two HIP events, and the
    span over `steps` is both the step time and, one launch per step, the
    kernel's average launch duration. With `pre` (work that must not be
    timed, such as a cache flush) `pre()` runs before every step, and each
    step gets its own pair of events: the total is the sum of those spans.
    Returns (total_ms, avg_ms)."""
    import torch

    for _ in range(warmup):
        if pre is not None:
            pre()
        step()
    torch.cuda.synchronize()
    if pre is None:
        t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_begin.record(stream)
        for _ in range(steps):
            step()
        t_end.record(stream)
        torch.cuda.synchronize()
        total_ms = t_begin.elapsed_time(t_end)
        return total_ms, total_ms / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        pre()
        starts[k].record(stream)
        step()
        ends[k].record(stream)
    torch.cuda.synchronize()
    total_ms = sum(s.elapsed_time(e) for s, e in zip(starts, ends))
    return total_ms, total_ms / steps


def bench_matmul(args) -> int:
    """--op matmul: the scaled matmul (bf16 or f32 result). --op
    matmul_quantize: the same product with its result quantized in the
    kernel (format --out, default e4m3fn); the unfused pair (bf16 matmul,
    then quantize) is timed on the same operands for comparison."""
    import torch

    import mx_microscaling_quantization_amd as mxq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, N, K = args.mm
    P = K // 4
    fmt = "e4m3fn"
    fused = args.op == "matmul_quantize"
    qout = args.out or "e4m3fn"
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    xl = torch.randn((P, 4 * M), generator=g, device=dev).to(torch.bfloat16)
    xr = torch.randn((P, 4 * N), generator=g, device=dev).to(torch.bfloat16)
    dl, sl = mxq.quantize(xl, fmt)
    dr, sr = mxq.quantize(xr, fmt)
    del xl, xr
    stream = torch.cuda.current_stream(dev)
    res_t = torch.bfloat16 if (args.res == "bf16" or fused) else torch.float32
    out = torch.empty((M, N), dtype=res_t, device=dev)
    compare = None
    if fused:
        qd = torch.empty(mxq.data_shape(M, N, qout), dtype=torch.uint8, device=dev)
        qs = torch.zeros(mxq.scale_image_shape(M, N), dtype=torch.uint8, device=dev)

        def step():
            mxq.scaled_matmul_quantize(dl, sl, dr, sr, fmt, qout, data_out=qd, scale_out=qs, stream=stream)

        def unfused():
            mxq.scaled_matmul(dl, sl, dr, sr, fmt, torch.bfloat16, out=out, stream=stream)
            mxq.quantize(out, qout, data_out=qd, scale_out=qs, stream=stream)

        u_total, u_avg = _time_steps(unfused, args.steps, args.warmup, stream)
        compare = {"unfused_ms_per_step": round(u_total / args.steps, 5),
                   "unfused": "scaled_matmul (bf16 result) then quantize",
                   "result_bytes_not_written_or_read": 2 * 2 * M * N}
    else:
        def step():
            mxq.scaled_matmul(dl, sl, dr, sr, fmt, res_t, out=out, stream=stream)

    total_ms, avg_ms = _time_steps(step, args.steps, args.warmup, stream)
    traffic, traffic_source = recorded_traffic("%s-%dx%dx%d" % (fmt, M, N, K), qout if fused else args.res, args.op)
    flops = 2.0 * M * N * K
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    achieved = flops / (avg_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC_MATMUL_QUANTIZE if fused else METRIC_MATMUL, "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True, "vs_baseline": None, "dtype": fmt, "data": "synthetic",
        "config": {"workload": "%s-%dx%dx%d-scaled-matmul%s" % (fmt, M, N, K, "-quantized-%s" % qout if fused else ""),
                   "M": M, "N": N, "K": K, "out": qout if fused else args.res, "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_source, "kernel_avg_us": round(avg_ms * 1e3, 3)},
        "cpu_baseline": None,
    }
    if compare:
        result["compare"] = compare
    result["env"] = run_env(args.op)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_matmul(dl, sl, dr, sr, fmt, quantize_out=qout if fused else None)
    print(json.dumps(result), flush=True)
    return 0


def copy_calibration(steps: int, warmup: int) -> None:
    import torch

    n = 1 << 30  # 2 GiB of bf16
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "ms_per_copy": round(ms, 4),
                      "copy_GBps": round(4 * n / ms / 1e6, 1)}), flush=True)


def run_env(op: str) -> dict:
    """Where the line was measured: HIP and torch versions, the device and
    its gfx architecture, and the digest of the op's kernel sources (the
    same digest that gates the committed traffic summaries)."""
    import torch

    props = torch.cuda.get_device_properties(0)
    return {"hip": torch.version.hip, "torch": torch.__version__, "device": props.name,
            "gfx_arch": getattr(props, "gcnArchName", None), "kernel_source_sha256_16": kernel_source_digest(op)}


def launch_stats(step, stream, n: int = 20, pre=None) -> dict:
    """`n` more calls, each between its own pair of HIP events (with `pre`,
    e.g. a cache flush, before each and outside its events), after the timed
    region: the median and minimum per call. An event pair around one launch
    also holds the launch's dispatch, so at small sizes these sit above the
    back-to-back average."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for k in range(n):
        if pre is not None:
            pre()
        starts[k].record(stream)
        step()
        ends[k].record(stream)
    torch.cuda.synchronize()
    us = sorted(starts[k].elapsed_time(ends[k]) * 1e3 for k in range(n))
    return {"n": n, "median_us": round(us[n // 2], 3), "min_us": round(us[0], 3),
            "timing": "one event pair per call, after the timed region"}


def copy_reference(stream, steps: int = 20, warmup: int = 3) -> dict:
    """A plain device-to-device copy of 1 GiB (torch's copy kernel: 1 GiB
    read, 1 GiB written) timed on the same box right after the measured
    op, so its line can be read against the copy rate as well as against
    the 8 TB/s peak. Its buffers are allocated and freed here, outside any
    timed region of the op."""
    import torch

    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    total_ms, avg_ms = _time_steps(lambda: dst.copy_(src), steps, warmup, stream)
    nbytes = 2 << 30
    del src, dst
    return {"kernel": "torch copy_ (device to device), 1 GiB read + 1 GiB written", "bytes_per_copy": nbytes,
            "us_per_copy": round(avg_ms * 1e3, 2), "GBps": round(nbytes / (avg_ms * 1e-3) / 1e9, 1)}


def floors(steps: int, warmup: int) -> None:
    """Plain linear streams with torch's own kernels, for comparison with
    the library's kernels: a read of 2 GiB (a sum), writes of 1 GiB and
    2 GiB (a fill) and a 2 GiB copy; each timed over `steps` back-to-back
    launches between two events on the current stream."""
    import torch

    stream = torch.cuda.current_stream()
    src = torch.ones(1 << 30, dtype=torch.bfloat16, device="cuda")      # 2 GiB
    dst1 = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")       # 1 GiB
    dst2 = torch.empty(1 << 30, dtype=torch.bfloat16, device="cuda")    # 2 GiB
    cases = [("read_2GiB_sum", lambda: src.sum(dtype=torch.float32), 2 << 30),
             ("write_1GiB_fill", lambda: dst1.fill_(7), 1 << 30),
             ("write_2GiB_fill", lambda: dst2.fill_(3.0), 2 << 30),
             ("copy_2GiB", lambda: dst2.copy_(src), 4 << 30)]
    out = {}
    for name, fn, nbytes in cases:
        total_ms, avg_ms = _time_steps(fn, steps, warmup, stream)
        out[name] = {"us": round(avg_ms * 1e3, 2), "GBps": round(nbytes / (avg_ms * 1e-3) / 1e9, 1)}
    print(json.dumps({"floors": out, "steps": steps, "warmup": warmup}), flush=True)


def vendor_gemm(args) -> None:
    """Context only, not the library: the vendor's per-tensor-scaled FP8
    product (torch._scaled_mm, e4m3fn operands, one fp32 scale each, bf16
    result) at the --mm sizes, timed like the matmul ops (warm-up launches,
    then `steps` back-to-back launches between two events). It does no
    per-block scale work, so it bounds what a block-scaled product of the
    same sizes could reach on this device."""
    import torch

    M, N, K = args.mm
    gen = torch.Generator(device="cuda").manual_seed(11)
    a = (torch.randn(M, K, device="cuda", generator=gen) * 0.5).to(torch.float8_e4m3fn)
    b = (torch.randn(N, K, device="cuda", generator=gen) * 0.5).to(torch.float8_e4m3fn).t()   # K x N, column-major
    one = torch.ones((), device="cuda")
    stream = torch.cuda.current_stream()
    total_ms, avg_ms = _time_steps(lambda: torch._scaled_mm(a, b, one, one, out_dtype=torch.bfloat16),
                                   args.steps, args.warmup, stream)
    flops = 2.0 * M * N * K
    print(json.dumps({"vendor_gemm": {"op": "torch._scaled_mm, per-tensor e4m3fn, bf16 result", "M": M, "N": N,
                                      "K": K, "us_per_call": round(avg_ms * 1e3, 2),
                                      "TFLOPs": round(flops / (avg_ms * 1e-3) / 1e12, 1)},
                      "steps": args.steps, "warmup": args.warmup}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default 5; 200 for the matmul ops)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--out", default=None, help="output format (default: the workload's first)")
    ap.add_argument("--op", choices=("quantize", "dequantize", "matmul", "matmul_quantize", "quantize_axis"),
                    default="quantize")
    ap.add_argument("--dim", type=int, choices=(-1, -2), default=-2,
                    help="quantize_axis: block axis of the row-major input (-1 along rows, -2 down columns)")
    ap.add_argument("--mm", type=int, nargs=3, default=(8192, 8192, 8192), metavar=("M", "N", "K"),
                    help="matmul sizes (M, N multiples of 4, K a multiple of 32)")
    ap.add_argument("--res", choices=("bf16", "f32"), default="bf16", help="dequantize result type")
    ap.add_argument("--cache", choices=("hot", "flushed"), default="hot",
                    help="flushed: read 512 MiB between launches and time the launches alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--floors", action="store_true",
                    help="time plain linear read / write / copy streams (torch kernels) instead")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the vendor's per-tensor FP8 product at the --mm sizes instead (context only)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this path runs on one GPU only; --gpus %d is not supported "
              "(rows shard with no exchange, see the design notes)" % args.gpus, file=sys.stderr)
        return 2
    args.warmup = default_warmup("matmul" if args.vendor_gemm else args.op, args.warmup)
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    import mx_microscaling_quantization_amd as mxq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration(args.steps, args.warmup)
        return 0
    if args.floors:
        floors(args.steps, args.warmup)
        return 0
    if args.vendor_gemm:
        vendor_gemm(args)
        return 0
    if args.op in ("matmul", "matmul_quantize"):
        return bench_matmul(args)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xt, spec = make_input(args.workload, dev)
    out = args.out or spec["outs"][0]
    P, F = xt.shape
    data = torch.empty(mxq.data_shape(P, F, out), dtype=torch.uint8, device=dev)
    image = torch.zeros(mxq.scale_image_shape(P, F), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.op == "quantize":
        def step():
            mxq.quantize(xt, out, data_out=data, scale_out=image, stream=stream)
        nbytes = algorithmic_bytes(P, F, out)
    elif args.op == "quantize_axis":
        VP, VF = mxq.axis_view_shape(P, F, args.dim)
        data = torch.empty(mxq.data_shape(VP, VF, out), dtype=torch.uint8, device=dev)
        image = torch.zeros(mxq.scale_image_shape(VP, VF), dtype=torch.uint8, device=dev)

        def step():
            mxq.quantize_axis(xt, out, args.dim, data_out=data, scale_out=image, stream=stream)
        nbytes = algorithmic_bytes(P, F, out)
    else:
        mxq.quantize(xt, out, data_out=data, scale_out=image, stream=stream)
        torch.cuda.synchronize()
        del xt
        res_t = torch.bfloat16 if args.res == "bf16" else torch.float32
        result = torch.empty((P, F), dtype=res_t, device=dev)

        def step():
            mxq.dequantize(data, image, out, res_t, out=result, stream=stream)
        nbytes = dequant_bytes(P, F, out, args.res)

    flushed = args.cache == "flushed"
    flush = None
    if flushed:
        # a read of twice the Infinity Cache's size before each launch, so the
        # launch finds none of its operands cached; a read leaves the caches
        # clean (a write would leave dirty lines whose write-back lands in
        # the next launch); it stays outside the timed spans
        flush_buf = torch.ones(64 << 20, dtype=torch.int64, device=dev)

        def flush():
            flush_buf.sum()

    total_ms, avg_launch_ms = _time_steps(step, args.steps, args.warmup, stream, pre=flush)
    value = nbytes * args.steps / (total_ms * 1e-3) / 1e9
    achieved = nbytes / (avg_launch_ms * 1e-3) / 1e9
    if args.op == "quantize":
        traffic, traffic_source = recorded_traffic(args.workload, out)
    elif args.op == "quantize_axis":
        traffic, traffic_source = recorded_traffic(args.workload, out, "quantize_axis", "dim%d" % args.dim)
    else:
        traffic, traffic_source = recorded_traffic(args.workload, out, "dequantize", args.res)

    config = {"workload": args.workload, "P": P, "F": F, "in": spec["in_dtype"], "out": out,
              "bytes_per_step": nbytes, "elements_per_step": P * F}
    if flushed:
        config["cache"] = "flushed"
    if args.op == "quantize_axis":
        config = {"workload": "%s-axis%d" % (args.workload, args.dim), "R": P, "C": F, "dim": args.dim,
                  "in": spec["in_dtype"], "out": out, "bytes_per_step": nbytes, "elements_per_step": P * F}
    if args.op == "dequantize":
        config = {"workload": args.workload + "-dequantize", "P": P, "F": F, "in": out, "out": args.res,
                  "bytes_per_step": nbytes, "elements_per_step": P * F}
    result = {
        "metric": {"quantize": METRIC, "quantize_axis": METRIC_AXIS}.get(args.op, METRIC_DEQUANT),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": out if args.op == "dequantize" else spec["in_dtype"],
        "data": "synthetic",
        "config": config,
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "elements_per_s": round(P * F * args.steps / (total_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_source": traffic_source, "kernel_avg_us": round(avg_launch_ms * 1e3, 3)},
        "cpu_baseline": None,
    }
    result["env"] = run_env(args.op)
    result["per_call"] = launch_stats(step, stream, pre=flush)
    ref = copy_reference(stream)
    ref["value_over_copy"] = round(value / ref["GBps"], 4)
    result["copy_reference"] = ref
    if not args.no_cpu_baseline:
        if args.op == "quantize":
            result["cpu_baseline"] = cpu_baseline(xt, out, spec["in_dtype"])
            result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(xt, out, spec["in_dtype"])
        elif args.op == "quantize_axis":
            result["cpu_baseline"] = cpu_baseline(xt, out, spec["in_dtype"], dim=args.dim)
        else:
            result["cpu_baseline"] = cpu_baseline_dequant(data, image, out, args.res)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
