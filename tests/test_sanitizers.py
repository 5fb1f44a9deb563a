"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code
(CPU only; no kernel runs).

* The CPU oracle (plain C) with a driver that calls every entry point on
  every 16-bit input pattern, all type pairs, layouts and EMAX modes, plus
  the matmul under every E8M0 byte and the rejected calls.
* The library's host code (validation, size helpers, status strings) with a
  driver that makes every rejected and empty call through the C ABI. The
  device code is built as usual; only the host side is instrumented.

Each run must exit 0 with no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "mx_microscaling_quantization_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe: str) -> str:
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-4000:]
    return text


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", *SAN, "-o", exe, os.path.join(HERE, "oracle_main.c"),
                    os.path.join(ROOT, "oracle", "mxq_oracle.c"), "-lm"], check=True, timeout=300)
    assert "ok" in _run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_library_host_code_under_sanitizers(tmp_path):
    import concurrent.futures

    host_san = []
    for flag in SAN:
        host_san += ["-Xarch_host", flag]    # instrument the host side only
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, "-I", os.path.join(ROOT, "include"),
                        "-I", CSRC, "-c", src, "-o", obj], check=True, timeout=600, capture_output=True)
        return obj

    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    main_o = str(tmp_path / "abi_main.o")
    cc = CLANG if os.path.exists(CLANG) else shutil.which("clang") or "gcc"
    subprocess.run([cc, "-std=c99", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(HERE, "abi_main.c"), "-o", main_o], check=True, timeout=300)
    exe = str(tmp_path / "abi_san")
    subprocess.run([HIPCC, "--offload-arch=gfx950", *host_san, "-o", exe, *objs, main_o], check=True, timeout=600,
                   capture_output=True)
    assert "ok" in _run(exe)
