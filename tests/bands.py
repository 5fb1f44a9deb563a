"""Run the CPU oracle over a large tensor in whole 32-row bands on the
host's threads and compare each band with the GPU's bytes.

A band of 32 rows is 4 row groups, so its scale-image rows are the global
image's rows shifted by the band's first row (the placement of logical row
i0 + k is row (k mod 4) + 32 floor(k / 4) + 8 i0 for i0 a multiple of 4), and
the oracle can quantize or decode it on its own. ctypes releases the
interpreter lock during each oracle call, so the bands run in parallel.
"""
from __future__ import annotations

import concurrent.futures
import os


def cuts(P: int, slabs: int) -> list[int]:
    """Row boundaries of `slabs` slabs of whole 32-row bands covering P rows."""
    bands = P // 32
    n = max(1, min(slabs, bands))
    return [32 * (bands * t // n) for t in range(n)] + [P]


def run_bands(P: int, check, slabs: int = 64, threads: int | None = None) -> list[str]:
    """Call check(r0, r1) for every slab (in parallel); it returns None or a
    message describing a mismatch. Returns the messages, in row order."""
    c = cuts(P, slabs)
    n = threads or max(1, min(16, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        out = list(ex.map(lambda t: check(c[t], c[t + 1]), range(len(c) - 1)))
    return [m for m in out if m]
