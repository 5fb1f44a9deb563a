"""The oracle's pins catch planted mistakes (CPU only).

Each case copies ``oracle/mxq_oracle.c``, plants one plausible mistake in
the copy (a wrong constant, a dropped term, a wrong index or rounding rule),
builds it with the oracle's own flags, and runs the pin suite against that
build (``MXQ_ORACLE_LIB``). The pins must fail for every mutant. A control
run on an unmodified copy must pass, so a failure is the mutant's doing.
The exhaustive sweeps are left out to keep the run short; every mutant here
is caught without them.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mxq_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")
FAST = "not exhaustive and not dense_fp32_range"

# (name, text in the oracle, planted replacement); the text must occur once
MUTANTS = [
    ("emax e4m3fn 8 -> 7", "case ORC_OUT_E4M3FN: return 8;", "case ORC_OUT_E4M3FN: return 7;"),
    ("emax e2m1 2 -> 3", "case ORC_OUT_E2M1: return 2;", "case ORC_OUT_E2M1: return 3;"),
    ("e8m0 zero not raised to 1", "int_max(1, int_max(0,", "int_max(0, int_max(0,"),
    ("e8m0 negative mirrored, not floored", "int_max(0, (int)max_exponent - emax_bias)",
     "abs((int)max_exponent - emax_bias)"),
    ("block exponent byte shifted by 24", "(bits_of(row[dc]) >> 23) & 0xFFu",
     "(bits_of(row[dc]) >> 24) & 0xFFu"),
    ("block drops its last row", "dr < 8; dr++)", "dr < 7; dr++)"),
    ("block drops its last column", "dc < 4; dc++)", "dc < 3; dc++)"),
    ("prescale exponent field 253 - e", "(254 - (int)e8m0)", "(253 - (int)e8m0)"),
    ("ties round up, not to even", "(rest == 0.5 && fmod(n, 2.0) != 0.0)", "(rest == 0.5)"),
    ("e4m3fn largest code 0x7D", "narrow_fp8(y, 3, -6, 448.0, 0x7E)", "narrow_fp8(y, 3, -6, 448.0, 0x7D)"),
    ("e4m3fn minimum normal exponent -7", "narrow_fp8(y, 3, -6,", "narrow_fp8(y, 3, -7,"),
    ("e5m2 with three mantissa bits", "narrow_fp8(y, 2, -14,", "narrow_fp8(y, 3, -14,"),
    ("FP8 NaN loses its sign", "(b >> 31) << 7);\n    if (isnan(y))\n        return sign;",
     "(b >> 31) << 7);\n    if (isnan(y))\n        return 0;"),
    ("FP4 NaN loses its sign", "(b >> 31) << 3);\n    if (isnan(y))\n        return sign;",
     "(b >> 31) << 3);\n    if (isnan(y))\n        return 0;"),
    ("lane remap without the byte mirror", "first + (stride - 1 - b % stride);", "first + b % stride;"),
    ("lane remap mirrors across the whole window of nibbles", "return 2 * mirrored + t;",
     "return 2 * mirrored + (1 - t);"),
    ("FP4 nibble parity 0", "#define ORC_FP4_PARITY 1", "#define ORC_FP4_PARITY 0"),
    ("scale slot stride 16", "(i & 3) + 32 * (i >> 2)", "(i & 3) + 16 * (i >> 2)"),
    ("f16 subnormal step 2^-25", "mag = ldexp((double)frac, -24);", "mag = ldexp((double)frac, -25);"),
    ("f16 normal bias off by one", "ldexp((double)(1024 + frac), ef - 25)", "ldexp((double)(1024 + frac), ef - 24)"),
    ("bf16 widen sets the low bit", "return float_of((uint32_t)h << 16);", "return float_of((uint32_t)h << 16 | 1u);"),
    ("e2m1 halves rounded up at ties", "round_half_even(fabs((double)y) * 2.0)", "floor(fabs((double)y) * 2.0 + 0.5)"),
    ("alternative EMAX subtracts 2", "int emax_bias = emax - (alt_emax ? 1 : 0);",
     "int emax_bias = emax - (alt_emax ? 2 : 0);"),
    ("dequantize scale 2^(e - 126)", "(float)ldexp(v, (int)srow[f / 4] - 127)", "(float)ldexp(v, (int)srow[f / 4] - 126)"),
    ("matmul reads a container backwards", "int64_t p = k / 4, j = k % 4;", "int64_t p = k / 4, j = 3 - k % 4;"),
    ("matmul scale 2^(e - 128)", "    return ldexp(v, e - 127);", "    return ldexp(v, e - 128);"),
    ("matmul reads E8M0 255 as NaN", "    return ldexp(v, e - 127);", "    return e == 255 ? NAN : ldexp(v, e - 127);"),
    ("axis view reverses each container", "                int64_t k = 4 * p + j;",
     "                int64_t k = 4 * p + (3 - j);"),
    ("bf16 rounding ties away from even", "(dropped == 0x8000u && (keep & 1u))", "(dropped == 0x8000u)"),
    ("FP4 decode of 0.5 as 0.25", "v = m ? 0.5 : 0.0;", "v = m ? 0.25 : 0.0;"),
    ("FP8 subnormals one binade low", "v = ldexp((double)m, 1 - bias - mbits);",
     "v = ldexp((double)m, -bias - mbits);"),
    ("e4m3fn NaN at 0x7E", "ef == 15 && m == 7)", "ef == 15 && m == 6)"),
    ("axis dim -2 mirrors the other axis", "in[k * C + o];", "in[k * C + (O - 1 - o)];"),
    ("fused result truncated to bf16", "res[k] = mxq_oracle_f32_to_bf16((float)sum[k]);",
     "res[k] = (uint16_t)(bits_of((float)sum[k]) >> 16);"),
    ("dense layout uses the image slot", "return layout == ORC_SCALE_DENSE ? i : mxq_oracle_scale_slot(i);",
     "return mxq_oracle_scale_slot(i);"),
]


def _build(text: str, out: str) -> None:
    src = out[:-3] + ".c"
    with open(src, "w") as fh:
        fh.write(text)
    subprocess.run(["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-w",
                    "-o", out, src, "-lm"], check=True)


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, MXQ_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-k", FAST, "-p", "no:cacheprovider",
                           "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Build the control copy and every mutant, then run the pins against
    all of them at once (a few processes at a time): name -> (exit status,
    end of the pytest report); a mutation site not found once maps to None."""
    import concurrent.futures

    text = open(SRC).read()
    work = tmp_path_factory.mktemp("mutants")
    jobs = {"control": text}
    sites = {}
    for k, (name, old, new) in enumerate(MUTANTS):
        sites[name] = text.count(old)
        if sites[name] == 1:
            jobs[name] = text.replace(old, new)
    libs = {}
    for k, (name, body) in enumerate(jobs.items()):
        libs[name] = str(work / ("m%02d.so" % k))
        _build(body, libs[name])

    def run(name):
        r = _run_pins(libs[name])
        return name, (r.returncode, r.stdout[-2000:])

    with concurrent.futures.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        done = dict(ex.map(run, list(jobs)))
    for name, count in sites.items():
        if count != 1:
            done[name] = None
    return done


def test_control_copy_passes(outcomes):
    rc, tail = outcomes["control"]
    assert rc == 0, tail


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_catch_mutant(outcomes, name):
    assert outcomes[name] is not None, "mutation site for %r not found exactly once" % name
    rc, tail = outcomes[name]
    # exit status 1: at least one pin failed (not a crash or a collection error)
    assert rc == 1, "the pins did not catch %r:\n%s" % (name, tail)
