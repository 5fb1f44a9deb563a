"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test checks the oracle against something it does not compute itself:
values the pages print (``tests/golden``), hand-worked tables, closed forms,
a brute-force definition checker (``defcheck``), and torch's own FP8 casts.
"""
import math

import numpy as np
import pytest
import torch

import defcheck
import oracle
import workloads

FMTS = ("e4m3fn", "e5m2", "e2m1")
INS = ("bf16", "f16")


def _golden_constants():
    return {k: v for k, v in defcheck.read_table("page_constants.txt")}


# ---------------------------------------------------------------- page facts

def test_emax_table_matches_page():
    c = _golden_constants()
    for fmt in FMTS:
        assert oracle.emax(fmt) == int(c["emax." + fmt])


def test_fp8_maxima_match_page():
    c = _golden_constants()
    for fmt in ("e4m3fn", "e5m2", "e2m1"):
        code = int(c["maxcode." + fmt], 16)
        val = float(c["maxval." + fmt])
        assert oracle.narrow(np.array([val], np.float32), fmt)[0] == code
        assert oracle.decode(np.array([code], np.uint8), fmt)[0] == val
        # anything larger saturates to the same code, with its sign
        big = np.array([val * 1.01, val * 1000, np.inf, -val * 3, -np.inf], np.float32)
        sb = 0x8 if fmt == "e2m1" else 0x80
        assert list(oracle.narrow(big, fmt)) == [code, code, code, code | sb, code | sb]


def test_e2m1_grid_matches_page():
    for nib, val in defcheck.read_table("e2m1_grid.txt"):
        n = int(nib, 16)
        v = float(val)
        got = oracle.decode(np.array([n], np.uint8), "e2m1")[0]
        assert got == v and math.copysign(1, got) == math.copysign(1, v)
        assert oracle.encode_e2m1(v) == n


def test_e2m1_hand_worked_ties():
    for val, code in defcheck.read_table("e2m1_rne_ties.txt"):
        assert oracle.encode_e2m1(float(val)) == int(code, 16), val


def test_e4m3fn_hand_worked_ties():
    for val, code in defcheck.read_table("e4m3fn_rne_ties.txt"):
        assert oracle.narrow(np.array([float(val)], np.float32), "e4m3fn")[0] == int(code, 16), val


def test_e8m0_clamps_match_page():
    c = _golden_constants()
    # all-zero (or all-denormal) block: max exponent byte 0 -> E8M0 1
    for fmt in FMTS:
        assert oracle.e8m0(0, oracle.emax(fmt)) == int(c["all_zero_block_e8m0"])
        # CLAMP-LOW then ZERO-FLOOR: anything at or below the bias gives 1
        for m in range(0, oracle.emax(fmt) + 2):
            assert oracle.e8m0(m, oracle.emax(fmt)) == 1
        for m in range(oracle.emax(fmt) + 1, 256):
            assert oracle.e8m0(m, oracle.emax(fmt)) == m - oracle.emax(fmt)


def test_prescale_is_power_of_two():
    c = _golden_constants()
    # E8M0 127 multiplies by exactly one
    x = workloads.bf16_bits_to_f32(np.arange(0, 0x7F80, 7, dtype=np.uint16))
    unit = int(c["unit_scale_e8m0"])
    assert np.array_equal(oracle.prescale(x, np.uint8(unit)).view(np.uint32), x.view(np.uint32))
    # the multiplier is 2^(127 - E8M0) for every reachable E8M0
    e = np.arange(1, 254, dtype=np.uint8)
    got = oracle.prescale(np.ones(e.size, np.float32), e).astype(np.float64)
    assert np.array_equal(got, np.ldexp(1.0, 127 - e.astype(np.int64)))


# ------------------------------------------------------------ widen (library)

def test_f16_widen_matches_numpy_all_patterns():
    h = np.arange(65536, dtype=np.uint16)
    got = oracle.widen(h, "f16")
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_bf16_widen_all_patterns():
    h = np.arange(65536, dtype=np.uint16)
    got = oracle.widen(h, "bf16")
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ----------------------------------------------- narrow: exhaustive + library

def _reachable_products(in_dtype: str):
    """Every finite input pattern times every prescale 2^(127-e), e in [1, 253],
    as fp32 (what the oracle narrows) and exactly (float64)."""
    h = np.arange(65536, dtype=np.uint16)
    x = defcheck.widen(h, in_dtype)
    x = x[np.isfinite(x)]
    e = np.arange(1, 254)
    exact = (x[None, :] * np.ldexp(1.0, 127 - e)[:, None]).ravel()
    with np.errstate(over="ignore"):      # unreachable huge pairs become inf: both saturate
        return exact.astype(np.float32), exact


@pytest.mark.parametrize("in_dtype", INS)
@pytest.mark.parametrize("fmt", FMTS)
def test_narrow_exhaustive_vs_bruteforce(in_dtype, fmt):
    y32, exact = _reachable_products(in_dtype)
    got = oracle.narrow(y32, fmt)
    # the same fp32 value through the brute-force nearest-code search
    assert np.array_equal(got, defcheck.narrow_bruteforce(y32.astype(np.float64), fmt))
    # and the exact product: rounding the product to fp32 first never
    # changes the code (double rounding is harmless for a power-of-two scale)
    assert np.array_equal(got, defcheck.narrow_bruteforce(exact, fmt))


@pytest.mark.parametrize("in_dtype", INS)
@pytest.mark.parametrize("fmt,tdtype,maxval", [("e4m3fn", torch.float8_e4m3fn, 448.0),
                                                ("e5m2", torch.float8_e5m2, 57344.0)])
def test_fp8_narrow_vs_torch_cast(in_dtype, fmt, tdtype, maxval):
    """torch's CPU float8 casts round to nearest-even but do not saturate, so
    clamping first gives the saturating narrow for finite inputs."""
    y32, _ = _reachable_products(in_dtype)
    t = torch.from_numpy(y32).clamp(-maxval, maxval).to(tdtype).view(torch.uint8).numpy()
    assert np.array_equal(oracle.narrow(y32, fmt), t)


def test_fp8_decode_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    for fmt, tdt in (("e4m3fn", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        ref = torch.from_numpy(codes.copy()).view(tdt).double().numpy()
        got = oracle.decode(codes, fmt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])


def test_e2m1_narrow_dense_fp32_range():
    """Every fp32 pattern with magnitude in [2^-3, 2^4) (all of e2m1's rounding
    boundaries), plus random patterns over the whole fp32 range."""
    lo = np.float32(0.125).view(np.uint32)
    hi = np.float32(16.0).view(np.uint32)
    for start in range(int(lo), int(hi), 1 << 23):
        u = np.arange(start, min(start + (1 << 23), int(hi)), dtype=np.uint32)
        y = u.view(np.float32)
        assert np.array_equal(oracle.narrow(y, "e2m1"), defcheck.narrow_bruteforce(y, "e2m1"))
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    y = u.view(np.float32)
    assert np.array_equal(oracle.narrow(y, "e2m1"), defcheck.narrow_bruteforce(y, "e2m1"))


@pytest.mark.parametrize("fmt", ("e4m3fn", "e5m2"))
def test_fp8_narrow_random_fp32(fmt):
    rng = np.random.default_rng(12)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    y = u.view(np.float32)
    assert np.array_equal(oracle.narrow(y, fmt), defcheck.narrow_bruteforce(y, fmt))


def test_nan_becomes_signed_zero():
    y = np.array([np.nan, -np.nan], np.float32)
    y[1] = -abs(y[1])
    assert list(oracle.narrow(y, "e2m1")) == [0x0, 0x8]
    assert list(oracle.narrow(y, "e4m3fn")) == [0x00, 0x80]
    assert list(oracle.narrow(y, "e5m2")) == [0x00, 0x80]


# ------------------------------------------------------------ E8M0 closed form

@pytest.mark.parametrize("in_dtype", INS)
@pytest.mark.parametrize("fmt", FMTS)
def test_e8m0_bit_trick_equals_closed_form(in_dtype, fmt):
    x = workloads.random_bits(64, 256, in_dtype, seed=21, specials=True)
    _, image = oracle.quantize(x, in_dtype, fmt)
    logical = image[defcheck.scale_slot(np.arange(64 // 8))]
    absmax = np.abs(defcheck.widen(x, in_dtype)).reshape(8, 8, 64, 4).max(axis=(1, 3))
    assert np.array_equal(logical, defcheck.e8m0_closed_form(absmax, fmt))


def test_e8m0_range_for_finite_blocks():
    for fmt in FMTS:
        x = workloads.random_bits(128, 512, "bf16", seed=22)
        _, image = oracle.quantize(x, "bf16", fmt)
        logical = image[defcheck.scale_slot(np.arange(16))]
        assert logical.min() >= 1 and logical.max() <= 254 - oracle.emax(fmt)


def test_block_max_exponent_is_sign_blind_and_denormal_zero():
    x = np.zeros((8, 4), np.float32)
    x[3, 2] = -3.0                      # biased exponent 128
    assert oracle.block_max_exponent(x, 0, 0) == 128
    x[:] = np.float32(1e-40)            # fp32 denormals read exponent 0
    assert oracle.block_max_exponent(x, 0, 0) == 0


# ------------------------------------------------------- packing and placement

def test_lane_remap_golden_and_involution():
    for k, r, _byte, _hi in defcheck.read_table("fp4_container_order.txt"):
        for q in range(5):
            assert oracle.lane_remap(4 * q + int(k), 2) == 4 * q + int(r)
    for stride in (1, 2, 3, 4, 8):
        for i in range(200):
            assert oracle.lane_remap(oracle.lane_remap(i, stride), stride) == i
    assert [oracle.lane_remap(i, 1) for i in range(32)] == list(range(32))


def test_scale_slot_golden_and_properties():
    for i, s in defcheck.read_table("scale_slots.txt"):
        assert oracle.scale_slot(int(i)) == int(s)
        assert defcheck.scale_slot(int(i)) == int(s)
    for P in (8, 16, 24, 32, 40, 64, 96, 128, 1024):
        slots = [oracle.scale_slot(i) for i in range(P // 8)]
        assert len(set(slots)) == len(slots) and max(slots) < P
    # a 32-row shard's slots are the whole tensor's shifted by 8 rows per group
    for i0 in range(0, 64, 4):
        for k in range(12):
            assert oracle.scale_slot(i0 + k) == oracle.scale_slot(k) + 8 * i0


def test_fp4_container_bytes_hand_worked():
    # one container per row: elements 0.5, 1, 1.5, 2 (codes 1, 2, 3, 4) at E8M0 127
    # -> byte0 = e2 | e3 << 4 = 0x43, byte1 = e0 | e1 << 4 = 0x21 (golden table)
    x = np.zeros((8, 4), np.uint16)
    vals = np.array([0.5, 1.0, 1.5, 2.0], np.float32)
    x[:] = workloads.f32_to_bf16_bits(vals)
    x[0, 0] = workloads.f32_to_bf16_bits(np.array([4.0], np.float32))[0]   # pilot: exp 129 -> E8M0 127
    data, image = oracle.quantize(x, "bf16", "e2m1")
    assert image[0, 0] == 127
    assert list(data[1]) == [0x43, 0x21]
    assert list(data[0]) == [0x43, 0x26]      # element 0 is 4.0 -> code 6


# ----------------------------------------------------- end to end, brute force

@pytest.mark.parametrize("in_dtype", INS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("P,F", [(8, 4), (16, 8), (32, 12), (40, 8), (40, 12), (64, 36)])
def test_oracle_equals_definitions_tiny(in_dtype, fmt, P, F):
    for seed in range(3):
        x = workloads.random_bits(P, F, in_dtype, seed=100 + seed, specials=True)
        fill = np.full((P, F // 4), 0xA5, np.uint8)
        d_or, im_or = oracle.quantize(x, in_dtype, fmt, image=fill)
        d_df, im_df = defcheck.quantize(x, in_dtype, fmt, image=fill)
        assert np.array_equal(d_or, d_df)
        assert np.array_equal(im_or, im_df)


@pytest.mark.parametrize("in_dtype", INS)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout", ("image", "dense"))
@pytest.mark.parametrize("alt", (False, True))
def test_oracle_equals_definitions_modes(in_dtype, fmt, layout, alt):
    for seed in range(3):
        x = workloads.random_bits(64, 36, in_dtype, seed=31 + seed, specials=True)
        d_or, im_or = oracle.quantize(x, in_dtype, fmt, alt_emax=alt, layout=layout)
        d_df, im_df = defcheck.quantize(x, in_dtype, fmt, alt=alt, layout=layout)
        assert np.array_equal(d_or, d_df) and np.array_equal(im_or, im_df)


def test_alt_emax_page_values_and_worked_example():
    # alternative mode: bias EMAX - 1 (7 for e4m3fn, 14 for e5m2)
    c = _golden_constants()
    for fmt in ("e4m3fn", "e5m2"):
        assert oracle.emax(fmt) - 1 == int(c["emax_alt." + fmt])
    # one block, max 256 (biased exponent 135): E8M0 135 - 7 = 128, multiplier
    # 2^-1, so 256 -> 128 = e4m3fn exponent field 14, mantissa 0 -> 0x70
    x = np.zeros((8, 4), np.uint16)
    x[0, 0] = workloads.f32_to_bf16_bits(np.array([256.0], np.float32))[0]
    data, image = oracle.quantize(x, "bf16", "e4m3fn", alt_emax=True)
    assert image[0, 0] == 128 and data[0, 0] == 0x70
    data, image = oracle.quantize(x, "bf16", "e4m3fn")
    assert image[0, 0] == 127 and data[0, 0] == 0x78


def test_alt_emax_fp4_nonfinite_block_reading():
    """E8M0 254: the page's multiplier is +0; every element of the block
    becomes a zero of its own sign (Inf * 0 read as a NaN of the Inf's sign)."""
    x = workloads.f32_to_bf16_bits(np.linspace(-3, 3, 32, dtype=np.float32)).reshape(8, 4)
    x[0, 0], x[0, 1], x[0, 2] = 0x7F80, 0xFF80, 0xFFC0      # +Inf, -Inf, -NaN
    data, image = oracle.quantize(x, "bf16", "e2m1", alt_emax=True)
    assert image[0, 0] == 254
    codes = defcheck.unpack_codes(data, 8, 4, "e2m1")
    signs = (x >> 15).astype(np.uint8)
    assert np.array_equal(codes, signs << 3)


def test_dense_layout_is_the_placed_rows():
    x = workloads.random_bits(256, 64, "f16", seed=33, specials=True)
    for fmt in FMTS:
        d_img, im = oracle.quantize(x, "f16", fmt)
        d_den, dense = oracle.quantize(x, "f16", fmt, layout="dense")
        assert np.array_equal(d_img, d_den)
        assert np.array_equal(dense, im[defcheck.scale_slot(np.arange(32))])
        for res in ("f32", "bf16"):
            a = oracle.dequantize(d_img, im, 256, 64, fmt, res)
            b = oracle.dequantize(d_den, dense, 256, 64, fmt, res, layout="dense")
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


# -------------------------------------------------------------- properties

@pytest.mark.parametrize("in_dtype", INS)
@pytest.mark.parametrize("fmt", FMTS)
def test_roundtrip_error_bound(in_dtype, fmt):
    """decode(q) * 2^(e-127) is within half a grid step of x unless x
    saturated, where it is +-max * 2^(e-127)."""
    P, F = 64, 128
    x = workloads.random_bits(P, F, in_dtype, seed=41)
    data, image = oracle.quantize(x, in_dtype, fmt)
    back = oracle.dequantize(data, image, P, F, fmt).astype(np.float64)
    v = defcheck.widen(x, in_dtype)
    e = np.repeat(np.repeat(image[defcheck.scale_slot(np.arange(P // 8))], 8, 0), 4, 1).astype(np.int64)
    y = v * np.ldexp(1.0, 127 - e)
    f = defcheck.FORMATS[fmt]
    maxval = defcheck.code_values(fmt)[-1]
    ay = np.abs(y)
    sat = ay >= maxval
    emin = 1 - f["bias"]
    binade = np.floor(np.log2(np.where(ay > 0, ay, 1.0)))
    step = np.ldexp(1.0, (np.maximum(binade, emin) - f["mbits"]).astype(np.int64))
    err = np.abs(back.astype(np.float64) * np.ldexp(1.0, 127 - e) - y)
    assert np.all(err[~sat] <= step[~sat] / 2)
    assert np.all(np.abs(back[sat]) == maxval * np.ldexp(1.0, e[sat] - 127))


@pytest.mark.parametrize("fmt", FMTS)
def test_prescaled_block_max_bounds(fmt):
    """Before the narrow the prescaled block max is below 2^(EMAX+1); after it
    every decoded magnitude is at most the format's largest value."""
    P, F = 128, 256
    x = workloads.random_bits(P, F, "bf16", seed=42)
    data, image = oracle.quantize(x, "bf16", fmt)
    e = np.repeat(np.repeat(image[defcheck.scale_slot(np.arange(P // 8))], 8, 0), 4, 1).astype(np.int64)
    y = defcheck.widen(x, "bf16") * np.ldexp(1.0, 127 - e)
    assert np.abs(y).max() < 2.0 ** (oracle.emax(fmt) + 1)
    if fmt == "e2m1":
        back = oracle.dequantize(data, image, P, F, fmt) * np.ldexp(1.0, 127 - e)
    else:
        back = oracle.decode(data, fmt)
    assert np.abs(back).max() <= defcheck.code_values(fmt)[-1]


def test_handplaced_workload_blocks():
    x = workloads.handplaced_bf16_128x512()
    data, image = oracle.quantize(x, "bf16", "e4m3fn")
    logical = image[defcheck.scale_slot(np.arange(16))]
    g, c = workloads.HANDPLACED["zero"]
    assert logical[g, c] == 1
    blk = data.reshape(16, 8, 128, 4)[g, :, c, :]
    assert set(blk.ravel().tolist()) == {0x00, 0x80} and (blk == 0x80).sum() == 1
    g, c = workloads.HANDPLACED["ties"]
    assert logical[g, c] == 127
    ties = {int(np.float32(float(v)).view(np.uint32)): int(code, 16)
            for v, code in defcheck.read_table("e4m3fn_rne_ties.txt")}
    vals = workloads.bf16_bits_to_f32(x.reshape(16, 8, 128, 4)[g, :, c, :]).ravel()
    codes = data.reshape(16, 8, 128, 4)[g, :, c, :].ravel()
    seen = 0
    for v, code in zip(vals.view(np.uint32), codes):
        if int(v) in ties:
            assert code == ties[int(v)], hex(int(v))
            seen += 1
    assert seen == 29          # pilot + 28 tie values (the three +0.0 fillers are not listed)
    g, c = workloads.HANDPLACED["outlier"]
    assert logical[g, c] == 147 - 8          # 2^20 has biased exponent 147
    g, c = workloads.HANDPLACED["subnormal"]
    assert logical[g, c] == 1
    # bf16 subnormal m * 2^-133 scaled by 2^126 is m * 2^-7: nonzero codes
    sub = data.reshape(16, 8, 128, 4)[g, :, c, :]
    assert np.all(sub & 0x7F > 0)


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((12, 8), np.uint16), "bf16", "e4m3fn")
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((8, 6), np.uint16), "bf16", "e4m3fn")


def test_empty_is_noop():
    d, im = oracle.quantize(np.zeros((0, 8), np.uint16), "bf16", "e4m3fn")
    assert d.size == 0 and im.size == 0


# ------------------------------------------------------------------ dequantize

def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(61)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    # plus every tie and near-tie pattern around a few binades, denormals and the top of the range
    base = np.array([0x3F800000, 0x00000000, 0x00010000, 0x7F7F0000, 0x80800000], np.uint32)
    extra = (base[:, None] + np.arange(0, 0x30000, 0x4000, dtype=np.uint32)[None, :]).ravel()
    extra = np.concatenate([extra, extra + 0x7FFF, extra + 0x8000, extra + 0x8001, extra + 0x18000])
    f = np.concatenate([u, extra]).view(np.float32)
    got = oracle.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7FFF) > 0x7F80)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("P,F", [(8, 4), (16, 12), (40, 8), (64, 64)])
def test_dequantize_equals_definition(fmt, P, F):
    rng = np.random.default_rng(P * 31 + F)
    data = rng.integers(0, 256, size=defcheck_data_bytes(P, F, fmt), dtype=np.uint8)
    image = rng.integers(0, 256, size=(P, F // 4), dtype=np.uint8)
    image[0, 0], image[min(1, P // 8 - 1) if P >= 16 else 0, -1] = 0, 255
    got = oracle.dequantize(data, image, P, F, fmt, "f32")
    ref = defcheck.dequantize(data, image, P, F, fmt)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    got16 = oracle.dequantize(data, image, P, F, fmt, "bf16")
    ref16 = torch.from_numpy(ref.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got16[~nan], ref16[~nan])
    assert np.all((got16[nan] & 0x7FFF) > 0x7F80)


def defcheck_data_bytes(P, F, fmt):
    return P * F // 2 if fmt == "e2m1" else P * F


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_inverts_quantize_on_grid_values(fmt):
    """Values already on the format's grid times 2^k, with the block max at
    the top binade, come back exactly."""
    P, F = 32, 32
    rng = np.random.default_rng(62)
    vals = defcheck.code_values(fmt)
    k = rng.integers(-20, 20, size=(P // 8, 1, F // 4, 1))
    pick = rng.integers(0, vals.size, size=(P // 8, 8, F // 4, 4))
    sign = np.where(rng.integers(0, 2, size=pick.shape) == 1, -1.0, 1.0)
    x = sign * vals[pick]
    x[:, 0, :, 0] = vals[-1]                       # block max = format max
    x = (x * np.ldexp(1.0, k)).reshape(P, F).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    assert np.array_equal(workloads.bf16_bits_to_f32(bits), x)   # exact in bf16
    data, image = oracle.quantize(bits, "bf16", fmt)
    back = oracle.dequantize(data, image, P, F, fmt, "f32")
    assert np.array_equal(back, x)


# ------------------------------------------------------------- scaled matmul

def _k_major(values_pf: np.ndarray, P: int, C: int) -> np.ndarray:
    """[P, 4C] element values -> the [K = 4P, C] matrix the reading gives:
    row k = 4p + j, column c holds element (p, 4c + j)."""
    return values_pf.reshape(P, C, 4).transpose(0, 2, 1).reshape(4 * P, C)


def _operand(rng, P, C, fmt, e_lo, e_hi):
    codes = rng.integers(0, 256, size=(P, 4 * C), dtype=np.uint8)
    nan = defcheck.FORMATS[fmt]["maxcode"]          # avoid NaN/Inf codes
    mag = codes & 0x7F
    codes = np.where(mag > nan, codes & 0x80 | nan, codes).astype(np.uint8)
    image = np.zeros((P, C), dtype=np.uint8)
    image[defcheck.scale_slot(np.arange(P // 8))] = rng.integers(e_lo, e_hi + 1, size=(P // 8, C))
    return codes, image


@pytest.mark.parametrize("fmt", ("e4m3fn", "e5m2"))
@pytest.mark.parametrize("P,M,N", [(8, 1, 1), (16, 3, 5), (40, 8, 4), (64, 16, 12)])
def test_scaled_matmul_equals_numpy_matmul_of_dequantized(fmt, P, M, N):
    """With scales in a narrow band every partial sum is exact in float64,
    so the triple loop must equal numpy's matmul of the independently
    dequantized operands bit for bit."""
    rng = np.random.default_rng(P * 100 + M * 10 + N)
    lhs, ls = _operand(rng, P, M, fmt, 124, 130)
    rhs, rs = _operand(rng, P, N, fmt, 124, 130)
    L = _k_major(defcheck.dequantize(lhs, ls, P, 4 * M, fmt).astype(np.float64), P, M)
    R = _k_major(defcheck.dequantize(rhs, rs, P, 4 * N, fmt).astype(np.float64), P, N)
    ref = np.matmul(L.T, R)
    got = oracle.scaled_matmul(lhs, ls, rhs, rs, fmt)
    assert np.array_equal(got, ref)


def test_scaled_matmul_integer_case():
    """Codes of small integers at E8M0 127: an exact integer matmul."""
    rng = np.random.default_rng(5)
    P, M, N = 16, 6, 7
    vals = np.array([0.0, 1.0, 2.0, 3.0, 4.0, -1.0, -2.0, -3.0])
    codes_of = {0.0: 0x00, 1.0: 0x38, 2.0: 0x40, 3.0: 0x44, 4.0: 0x48, -1.0: 0xB8, -2.0: 0xC0, -3.0: 0xC4}
    li = rng.integers(0, 8, size=(P, 4 * M))
    ri = rng.integers(0, 8, size=(P, 4 * N))
    lhs = np.vectorize(lambda i: codes_of[vals[i]])(li).astype(np.uint8)
    rhs = np.vectorize(lambda i: codes_of[vals[i]])(ri).astype(np.uint8)
    img_l = np.full((P, M), 127, np.uint8)
    img_r = np.full((P, N), 127, np.uint8)
    Lint = _k_major(vals[li], P, M).astype(np.int64)
    Rint = _k_major(vals[ri], P, N).astype(np.int64)
    got = oracle.scaled_matmul(lhs, img_l, rhs, img_r, "e4m3fn")
    assert np.array_equal(got, (Lint.T @ Rint).astype(np.float64))


def test_scaled_matmul_hand_worked_and_scale_shift():
    # K = 32 (one group), M = N = 1: lhs all 1.0 at E8M0 127, rhs all 2.0 at
    # E8M0 128 (x2): each product is 4, the sum 32 * 4 = 128
    lhs = np.full((8, 4), 0x38, np.uint8)
    rhs = np.full((8, 4), 0x40, np.uint8)
    got = oracle.scaled_matmul(lhs, np.full((8, 1), 127, np.uint8), rhs, np.full((8, 1), 128, np.uint8), "e4m3fn")
    assert got[0, 0] == 128.0
    # raising every lhs E8M0 by d multiplies the result by 2^d exactly
    rng = np.random.default_rng(6)
    lhs, ls = _operand(rng, 32, 4, "e5m2", 100, 150)
    rhs, rs = _operand(rng, 32, 3, "e5m2", 100, 150)
    base = oracle.scaled_matmul(lhs, ls, rhs, rs, "e5m2")
    placed = defcheck.scale_slot(np.arange(4))
    ls2 = ls.copy()
    ls2[placed] += 3
    assert np.array_equal(oracle.scaled_matmul(lhs, ls2, rhs, rs, "e5m2"), base * 8.0)
    # the dense layout reads the same scales
    assert np.array_equal(oracle.scaled_matmul(lhs, ls[placed], rhs, rs[placed], "e5m2", layout="dense"), base)


def test_scaled_matmul_e8m0_255_reading():
    """Reading: the numerics page gives the consumer's dequant as
    ldexpf(x, E8M0 - 127) with no exception, so a byte of 255 is the scale
    2^128 in the matmul too. With a lhs column whose only nonzero block sits
    under that byte, its results are exactly twice those under 254 (every
    product doubles, so every partial sum doubles exactly); the other
    columns do not change."""
    rng = np.random.default_rng(7)
    lhs, ls = _operand(rng, 16, 3, "e4m3fn", 125, 129)
    rhs, rs = _operand(rng, 16, 2, "e4m3fn", 125, 129)
    lhs[:8, 8:12] = 0                            # column 2 of lhs: row group 0 all zero
    slot1 = defcheck.scale_slot(1)
    ls[slot1, 2] = 254
    at254 = oracle.scaled_matmul(lhs, ls, rhs, rs, "e4m3fn")
    ls[slot1, 2] = 255                           # row group 1 of lhs column 2
    at255 = oracle.scaled_matmul(lhs, ls, rhs, rs, "e4m3fn")
    assert not np.isnan(at255).any() and np.any(at255[2] != 0)
    assert np.array_equal(at255[2], 2.0 * at254[2])
    assert np.array_equal(np.delete(at255, 2, axis=0), np.delete(at254, 2, axis=0))


@pytest.mark.parametrize("fmt", ("e4m3fn", "e5m2"))
def test_scaled_matmul_and_dequantize_agree_on_element_values(fmt):
    """Both consumers give an element the same value, decode(q) * 2^(E8M0 -
    127): a one-hot rhs (R[k][n] = 1 if k == n) makes the matmul return the
    lhs elements themselves, and rounded to fp32 they equal the dequantize's
    values -- under every E8M0 byte 0..255, including those whose values
    overflow fp32 (both then give the same infinity)."""
    P, M = 8, 64                                  # K = 32, one block per column
    rng = np.random.default_rng(70)
    lhs, ls = _operand(rng, P, M, fmt, 0, 255)
    ls[0, :] = np.arange(256)[rng.permutation(256)[:M]]
    ls[0, :4] = (0, 1, 254, 255)
    one = {"e4m3fn": 0x38, "e5m2": 0x3C}[fmt]
    rhs = np.zeros((P, 4 * 32), np.uint8)
    for k in range(32):
        rhs[k // 4, 4 * k + k % 4] = one          # R[k][n = k] = 1.0 at E8M0 127
    rs = np.zeros((P, 32), np.uint8)
    rs[0, :] = 127
    out = oracle.scaled_matmul(lhs, ls, rhs, rs, fmt)                # [M, K]
    deq = oracle.dequantize(lhs, ls, P, 4 * M, fmt, "f32")          # [P, 4M]
    L = _k_major(deq, P, M)                                          # [K, M]
    with np.errstate(over="ignore"):
        # compared as values: a sum of zeros is +0 where the element is -0
        assert np.array_equal(out.T.astype(np.float32), L)
    assert np.isinf(L[:, 3]).any() and np.isfinite(L[:, 0]).all() and (L[:, 0] != 0).any()


# ------------------------------------------------------ quantize-on-produce

@pytest.mark.parametrize("fmt,out", [("e4m3fn", "e4m3fn"), ("e5m2", "e5m2"), ("e4m3fn", "e2m1"),
                                     ("e5m2", "e4m3fn")])
@pytest.mark.parametrize("alt,layout", [(False, "image"), (True, "dense")])
def test_scaled_matmul_quantize_equals_definition_composition(fmt, out, alt, layout):
    """The fused oracle equals the definition checker's quantize of the
    product rounded to fp32 and then to bf16. The exact product comes from
    numpy's float64 matmul of the independently dequantized operands (scales
    in a narrow band keep every partial sum exact) and the bf16 rounding from
    torch's nearest-even cast, so no step is the oracle's own."""
    import torch

    P, M, N = 32, 16, 12
    rng = np.random.default_rng(sum(map(ord, fmt + out)) + 2 * alt)
    lhs, ls = _operand(rng, P, M, fmt, 124, 130)
    rhs, rs = _operand(rng, P, N, fmt, 124, 130)
    L = _k_major(defcheck.dequantize(lhs, ls, P, 4 * M, fmt).astype(np.float64), P, M)
    R = _k_major(defcheck.dequantize(rhs, rs, P, 4 * N, fmt).astype(np.float64), P, N)
    exact = np.matmul(L.T, R)
    b16 = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want_data, want_scale = defcheck.quantize(b16, "bf16", out, alt=alt, layout=layout)
    if layout == "dense":
        placed = defcheck.scale_slot(np.arange(P // 8))
        ls, rs = ls[placed], rs[placed]
    got_data, got_scale = oracle.scaled_matmul_quantize(lhs, ls, rhs, rs, fmt, out, alt_emax=alt, layout=layout)
    assert np.array_equal(got_data, want_data)
    assert np.array_equal(got_scale, want_scale)


def test_scaled_matmul_quantize_rounds_through_bf16():
    """Hand-worked, e4m3fn in and out, every E8M0 127 (scale 1). Column 0 of
    rhs holds 30 codes of 1.0, one 4.0 (0x48) and one 2^-4 (0x18); lhs is all
    1.0, so out[m][0] = 34.0625 for every m, and columns 1..3 are 0.
      bf16 keeps 8 significant bits: between 32 and 64 its step is 0.25, and
      34.0625 rounds to 34.0.
      Block max 34 has exponent 5, so E8M0 = 127 + 5 - 8 = 124 and the
      prescale multiplies by 2^(127 - 124) = 8: 34 -> 272, the midpoint of
      the e4m3fn neighbours 256 (0x78) and 288 (0x79); nearest-even gives
      0x78. Quantizing the fp32 value instead (272.5) would give 0x79."""
    lhs = np.full((8, 4 * 8), 0x38, np.uint8)                   # M = 8 columns of 1.0
    rhs = np.zeros((8, 4 * 4), np.uint8)                        # N = 4
    rhs[:, 0:4] = 0x38
    rhs[0, 0] = 0x48                                            # 4.0
    rhs[0, 1] = 0x18                                            # 2^-4
    ls = np.full((8, 8), 127, np.uint8)
    rs = np.full((8, 4), 127, np.uint8)
    exact = oracle.scaled_matmul(lhs, ls, rhs, rs, "e4m3fn")
    assert np.all(exact[:, 0] == 34.0625) and not exact[:, 1:].any()
    data, scale = oracle.scaled_matmul_quantize(lhs, ls, rhs, rs, "e4m3fn", "e4m3fn")
    assert scale[0, 0] == 124
    assert np.all(data[:, 0] == 0x78) and not data[:, 1:].any()
    assert oracle.narrow(np.float32([272.0, 272.5]), "e4m3fn").tolist() == [0x78, 0x79]


def test_scaled_matmul_quantize_empty_k_and_shapes():
    lhs = np.zeros((0, 32), np.uint8)
    rhs = np.zeros((0, 16), np.uint8)
    data, scale = oracle.scaled_matmul_quantize(lhs, np.zeros((0, 8), np.uint8), rhs, np.zeros((0, 4), np.uint8),
                                                "e4m3fn", "e5m2")
    assert data.shape == (8, 4) and not data.any()
    assert scale[defcheck.scale_slot(np.arange(1))].tolist() == [[1]]   # an all-zero block has E8M0 1
    with pytest.raises(ValueError):                                     # M % 8 != 0
        oracle.scaled_matmul_quantize(np.zeros((8, 16), np.uint8), np.zeros((8, 4), np.uint8),
                                      np.zeros((8, 16), np.uint8), np.zeros((8, 4), np.uint8), "e4m3fn", "e4m3fn")


# ------------------------------------------------------- quantize along an axis

def _device_view(x: np.ndarray, dim: int) -> np.ndarray:
    """numpy re-layout of a row-major [R, C] tensor into the [K/4, 4*O]
    partition-major view: element (p, 4o + j) = block-axis element 4p + j
    at other-axis index o."""
    d = dim + 2 if dim < 0 else dim
    if d == 1:                                   # blocks along rows: X[o][k]
        O, K = x.shape
        return x.reshape(O, K // 4, 4).transpose(1, 0, 2).reshape(K // 4, 4 * O)
    K, O = x.shape                               # blocks down columns: W[k][o]
    return x.reshape(K // 4, 4, O).transpose(0, 2, 1).reshape(K // 4, 4 * O)


@pytest.mark.parametrize("in_dtype,fmt", [("bf16", "e4m3fn"), ("f16", "e5m2"), ("bf16", "e2m1")])
@pytest.mark.parametrize("dim,R,C", [(-2, 32, 4), (0, 64, 36), (-2, 96, 64), (-1, 96, 64), (1, 4, 32),
                                     (-1, 13, 96)])
def test_quantize_axis_equals_definition(dim, in_dtype, fmt, R, C):
    x = workloads.random_bits(R, C, in_dtype, seed=R * 7 + C + dim, specials=True)
    for alt, layout in ((False, "image"), (True, "dense")):
        want = defcheck.quantize(_device_view(x, dim), in_dtype, fmt, alt=alt, layout=layout)
        got = oracle.quantize_axis(x, in_dtype, fmt, dim, alt_emax=alt, layout=layout)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_quantize_axis_hand_worked_positions():
    """One nonzero element 1.0 at block-axis index 5, other-axis index 1:
    block max 1.0 -> E8M0 127 - 8 = 119 -> prescale 2^8 -> 256 = 0x78, at
    device row 5 // 4 = 1, column 4 * 1 + 5 % 4 = 5; every other code 0."""
    one = np.uint16(0x3F80)                      # bf16 1.0
    w = np.zeros((32, 2), np.uint16)             # W[k][n], dim -2
    w[5, 1] = one
    x = np.zeros((2, 32), np.uint16)             # X[m][k], dim -1
    x[1, 5] = one
    for t, dim in ((w, -2), (x, -1)):
        data, scale = oracle.quantize_axis(t, "bf16", "e4m3fn", dim)
        assert data.shape == (8, 8)
        assert data[1, 5] == 0x78 and np.count_nonzero(data) == 1
        assert scale[0].tolist() == [1, 119]     # block of column 0 is all zero -> E8M0 1


@pytest.mark.parametrize("fmt", ("e4m3fn", "e5m2", "e2m1"))
def test_quantize_axis_grid_values_round_trip_through_the_layout(fmt):
    """Inputs on the format's grid at every block scale round-trip exactly:
    the dequantized device view equals numpy's re-layout of the input."""
    rng = np.random.default_rng(12)
    grid = {"e4m3fn": [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0], "e5m2": [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0],
            "e2m1": [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]}[fmt]
    for dim, shape in ((-1, (24, 64)), (-2, (96, 20))):
        v = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v = (v * np.ldexp(1.0, rng.integers(-20, 20, size=(1, shape[1]) if dim == -2 else (shape[0], 1)))
             ).astype(np.float32)
        bits = workloads.f32_to_bf16_bits(v)
        data, scale = oracle.quantize_axis(bits, "bf16", fmt, dim)
        P, F = _device_view(bits, dim).shape
        back = oracle.dequantize(data, scale, P, F, fmt, "f32")
        assert np.array_equal(back, _device_view(v, dim))


def test_quantize_axis_feeds_the_matmul_as_x_times_w():
    """Small integers are exact in e4m3fn at E8M0 127..: quantizing X [M, K]
    along its rows and W [K, N] down its columns gives operands whose scaled
    matmul is X @ W exactly -- the axis layout and the matmul's operand
    reading agree."""
    rng = np.random.default_rng(13)
    M, K, N = 12, 64, 20
    X = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    W = rng.integers(-4, 5, size=(K, N)).astype(np.float32)
    dl, sl = oracle.quantize_axis(workloads.f32_to_bf16_bits(X), "bf16", "e4m3fn", -1)
    dr, sr = oracle.quantize_axis(workloads.f32_to_bf16_bits(W), "bf16", "e4m3fn", -2)
    got = oracle.scaled_matmul(dl, sl, dr, sr, "e4m3fn")
    assert np.array_equal(got, X.astype(np.float64) @ W.astype(np.float64))


def test_quantize_axis_rejects_bad_axes():
    x = np.zeros((32, 32), np.uint16)
    for bad in (2, -3):
        with pytest.raises(ValueError):
            oracle.quantize_axis(x, "bf16", "e4m3fn", bad)
    with pytest.raises(ValueError):
        oracle.quantize_axis(np.zeros((32, 20), np.uint16), "bf16", "e4m3fn", -1)   # K = 20
