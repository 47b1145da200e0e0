"""Pins for the oracle's FP8 codec (CPU only).

Each check ties the oracle to something other than itself: the values the
pages print (tests/golden), library conversions of textbook IEEE formats
(numpy float16, torch bfloat16 / float8), a brute-force nearest-code search
and exhaustive enumeration of all 256 codes.
"""
import math

import numpy as np
import pytest
import torch

from conftest import golden_rows

STYLE = {"ieee": 0, "fn": 1}
FMT = {"float8_e4m3fn": 0, "float8_e5m2": 1}


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _close_printed(value, printed):
    """Equal to the page's decimal at the precision it was printed with."""
    s = printed.lower().replace("-", "")
    mant = s.split("e")[0]
    digits = len(mant.replace(".", "").lstrip("0")) or 1
    return math.isclose(value, float(printed), rel_tol=0.6 * 10 ** (1 - digits), abs_tol=0.0)


# ------------------------------------------------------------ page values ----

@pytest.mark.parametrize("row", golden_rows("fp8_finfo.txt"), ids=lambda r: r[0])
def test_finfo_extremes_match_page(oracle, row):
    name, ebits, mbits, style, bits, mx, mn, smallest_normal, eps = row
    ebits, mbits, st = int(ebits), int(mbits), STYLE[style]
    assert 1 + ebits + mbits == int(bits)
    vmax = oracle.mf_max(ebits, mbits, st)
    assert _close_printed(vmax, mx)
    # the most negative finite value is the max with the sign bit set
    maxcode = oracle.mf_encode(np.float32(min(vmax, 3.4028234e38)), ebits, mbits, st, 1)
    assert oracle.mf_decode(maxcode | (1 << (ebits + mbits)), ebits, mbits, st) == -vmax
    assert _close_printed(-vmax, mn)
    # smallest normal: exponent field 1, mantissa 0
    sn = oracle.mf_decode(1 << mbits, ebits, mbits, st)
    assert _close_printed(sn, smallest_normal)
    assert oracle.mf_decode((1 << mbits) - 1, ebits, mbits, st) < sn   # largest subnormal below it
    # eps: distance from 1.0 to the next representable value
    one = oracle.mf_encode(np.float32(1.0), ebits, mbits, st, 0)
    assert oracle.mf_decode(one, ebits, mbits, st) == 1.0
    assert _close_printed(oracle.mf_decode(one + 1, ebits, mbits, st) - 1.0, eps)


def test_fp8_extremes_codes(oracle):
    assert oracle.decode(0x7E, 0) == 448.0 and oracle.decode(0xFE, 0) == -448.0
    assert oracle.decode(0x7B, 1) == 57344.0 and oracle.decode(0xFB, 1) == -57344.0
    assert oracle.decode(0x08, 0) == 2.0 ** -6 and oracle.decode(0x04, 1) == 2.0 ** -14
    assert oracle.decode(0x01, 0) == 2.0 ** -9 and oracle.decode(0x01, 1) == 2.0 ** -16
    assert math.isnan(oracle.decode(0x7F, 0)) and math.isnan(oracle.decode(0xFF, 0))
    assert oracle.decode(0x7C, 1) == math.inf and oracle.decode(0xFC, 1) == -math.inf
    for c in (0x7D, 0x7E, 0x7F):
        assert math.isnan(oracle.decode(c, 1))
    assert oracle.fp8_max(0) == 448.0 and oracle.fp8_max(1) == 57344.0


def test_worked_cast_example_matches_page(oracle):
    rows = {r[0]: r[1:] for r in golden_rows("cast_example.txt")}
    x = np.array([float(v) for v in rows["float32"]], dtype=np.float32)
    for name, fmt in FMT.items():
        got = [oracle.decode(oracle.encode(v, fmt), fmt) for v in x]
        assert got == [float(v) for v in rows[name]], name
    # expected codes (derived from the format layout)
    assert [oracle.encode(v, 0) for v in x] == [0x40, 0xB5, 0xAF, 0xBB]
    assert [oracle.encode(v, 1) for v in x] == [0x40, 0xBA, 0xB8, 0xBD]
    bf = oracle.bf16_to_f64(oracle.bf16_from_f32(x))
    for v, p in zip(bf, rows["bfloat16"]):
        assert _close_printed(v, p)


# --------------------------------------------------- exhaustive over codes ----

@pytest.mark.parametrize("fmt", [0, 1])
def test_round_trip_all_codes(oracle, fmt):
    for c in range(256):
        v = oracle.decode(c, fmt)
        if math.isnan(v):
            continue
        if math.isinf(v):          # E5M2 Inf: the saturating cast clips it to max
            assert oracle.encode(v, fmt) == (0x7B | (c & 0x80))
            continue
        assert oracle.encode(np.float32(v), fmt) == c, hex(c)
    assert oracle.encode(np.float32(-0.0), fmt) == 0x80
    assert oracle.encode(np.float32(0.0), fmt) == 0x00


def test_e5m2_decode_is_fp16_decode_of_high_byte(oracle):
    for c in range(256):
        h = np.array([c << 8], dtype=np.uint16).view(np.float16)[0]
        v = oracle.decode(c, 1)
        if math.isnan(v):
            assert np.isnan(h)
        else:
            assert float(h) == v


def test_values_are_sorted_and_distinct(oracle):
    for fmt, maxc in ((0, 0x7E), (1, 0x7B)):
        vals = [oracle.decode(c, fmt) for c in range(maxc + 1)]
        assert all(a < b for a, b in zip(vals, vals[1:]))


# --------------------------------------------------- brute-force agreement ----

def _edge_inputs(oracle, fmt, maxc):
    """All midpoints of adjacent codes, their fp32 neighbours, and the codes."""
    vals = np.array([oracle.decode(c, fmt) for c in range(maxc + 1)])
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    assert np.all(pts.astype(np.float64) == np.concatenate([vals, mids]))   # exact in fp32
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(-np.inf))
    allp = np.concatenate([pts, up, dn])
    return np.concatenate([allp, -allp])


@pytest.mark.parametrize("fmt,maxc", [(0, 0x7E), (1, 0x7B)])
def test_encoder_matches_bruteforce(oracle, fmt, maxc):
    rng = np.random.default_rng(1234 + fmt)
    all_bf16 = _f32(np.arange(1 << 16, dtype=np.uint32) << 16)
    rnd = _f32(rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32))
    # random values concentrated in and around the format's range
    near = (rng.standard_normal(1 << 20) * np.exp2(rng.uniform(-20, 20, 1 << 20))).astype(np.float32)
    x = np.concatenate([all_bf16, rnd, near, _edge_inputs(oracle, fmt, maxc)])
    a = oracle.encode_array(x, fmt)
    b = oracle.encode_bruteforce_array(x, fmt)
    bad = np.nonzero(a != b)[0]
    assert bad.size == 0, [(float(x[i]), hex(a[i]), hex(b[i])) for i in bad[:5]]


@pytest.mark.parametrize("fmt,maxc", [(0, 0x7E), (1, 0x7B)])
def test_midpoints_round_to_even(oracle, fmt, maxc):
    for c in range(maxc):
        lo, hi = oracle.decode(c, fmt), oracle.decode(c + 1, fmt)
        mid = np.float32((lo + hi) / 2)
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode(mid, fmt) == even
        assert oracle.encode(np.nextafter(mid, np.float32(np.inf)), fmt) == c + 1
        assert oracle.encode(np.nextafter(mid, np.float32(-np.inf)), fmt) == c
        assert oracle.encode(-mid, fmt) == (even | 0x80)


@pytest.mark.parametrize("fmt,maxc,mx", [(0, 0x7E, 448.0), (1, 0x7B, 57344.0)])
def test_saturation(oracle, fmt, maxc, mx):
    rng = np.random.default_rng(7)
    lo, hi = int(_bits(np.float32(mx))), int(_bits(np.float32(np.inf)))
    b = np.concatenate([rng.integers(lo, hi + 1, size=1 << 18, dtype=np.uint64).astype(np.uint32),
                        np.array([lo, lo + 1, hi - 1, hi], dtype=np.uint32)])
    x = _f32(b)
    assert np.all(oracle.encode_array(x, fmt) == maxc)
    assert np.all(oracle.encode_array(-x, fmt) == (maxc | 0x80))
    assert oracle.encode(np.float32(1e30), fmt) == maxc
    assert oracle.encode(np.float32(-1e30), fmt) == maxc | 0x80
    for nan_bits in (0x7FC00000, 0x7F800001, 0x7FFFFFFF, 0xFFC00000):
        code = oracle.encode(_f32(np.array([nan_bits], dtype=np.uint32))[0], fmt)
        assert code == (0x7F | (0x80 if nan_bits >> 31 else 0))


@pytest.mark.parametrize("fmt,mx", [(0, 448.0), (1, 57344.0)])
def test_count_saturated(oracle, fmt, mx):
    """The saturated-element count: planted products at the boundary (exactly
    the maximum is exact, not clamped; one step above is clamped), +-Inf
    counted, NaN and zero not, for fp32 and bf16 inputs; then, on random
    data spanning the boundary, the count equals the number of products that
    the encoder maps to the top code while lying above the maximum, and the
    count of numpy's fp32 products above it."""
    s = np.float32(128.0)                        # power of two: the planted products are exact
    at = np.float32(mx / 128.0)                  # 3.5 (E4M3) and 448 (E5M2): bf16-exact
    above = np.float32(np.nextafter(at, np.float32(np.inf)))
    above_bf16 = np.float32(at + (2.0 ** (math.floor(math.log2(at)) - 7)))   # one bf16 step up
    planted = np.array([at, -at, above, -above, np.inf, -np.inf, np.nan, 0.0, -0.0, 1e30, 1.0], dtype=np.float32)
    assert oracle.count_saturated(planted, fmt, s) == 5          # +-above, +-inf, 1e30 (fp32 product 1.28e32)
    assert oracle.count_saturated(planted[:2], fmt, s) == 0
    planted16 = np.array([at, -at, above_bf16, -above_bf16, np.inf, np.nan, 0.0], dtype=np.float32)
    bits = oracle.bf16_from_f32(planted16)
    assert np.array_equal(oracle.bf16_to_f64(bits), planted16.astype(np.float64), equal_nan=True)
    assert oracle.count_saturated(bits, fmt, s) == 3
    assert oracle.count_saturated(np.zeros(0, dtype=np.float32), fmt, s) == 0
    rng = np.random.default_rng(19)
    x = (rng.standard_normal(1 << 16) * (mx / 3.0)).astype(np.float32)
    sc = np.float32(1.37)
    p = x * sc                                   # numpy's fp32 products (IEEE RNE)
    top = 0x7E if fmt == 0 else 0x7B
    codes = oracle.encode_array(p, fmt) & 0x7F
    want = int(np.count_nonzero(np.abs(p) > np.float32(mx)))
    assert want > 100
    assert oracle.count_saturated(x, fmt, sc) == want
    assert want == int(np.count_nonzero((codes == top) & (np.abs(p) > np.float32(mx))))
    assert int(np.count_nonzero(codes == top)) >= want


# ------------------------------------------- textbook formats via library ----

def _pattern_set(n_random, seed):
    rng = np.random.default_rng(seed)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x3000, 0x7FFF,
                     0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    structured = (hi[:, None] | lows[None, :]).ravel()
    rnd = rng.integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    # every fp32 exponent that lands in fp16's subnormal / lowest-normal range, strided mantissas
    sub = ((np.arange(100, 116, dtype=np.uint32)[:, None] << 23) |
           (np.arange(0, 1 << 23, 97, dtype=np.uint32)[None, :])).ravel()
    return np.concatenate([structured, rnd, sub, sub | 0x80000000])


def test_generic_codec_is_ieee_fp16(oracle):
    """(5 exponent, 10 mantissa) bits, IEEE style, no saturation == numpy float16 (RNE)."""
    b = _pattern_set(1 << 21, 11)
    x = _f32(b)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.mf_encode_array(x, 5, 10, 0, 0).astype(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan].view(np.float16)))
    # decode side: all 65536 fp16 codes
    codes = np.arange(1 << 16, dtype=np.uint32)
    dec = oracle.mf_decode_array(codes, 5, 10, 0)
    ref_dec = codes.astype(np.uint16).view(np.float16).astype(np.float64)
    same = (dec == ref_dec) | (np.isnan(dec) & np.isnan(ref_dec))
    assert same.all()


def test_generic_codec_is_bfloat16(oracle):
    """(8, 7) bits, IEEE style, no saturation == torch's float -> bfloat16 (RNE)."""
    b = _pattern_set(1 << 21, 12)
    x = _f32(b)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_f32(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(((got[nan] >> 7) & 0xFF) == 0xFF) and np.all(got[nan] & 0x7F)


def test_fp8_codec_matches_torch_in_range(oracle):
    """torch's float8 casts round to nearest-even but give NaN beyond the range,
    so they pin the in-range part of the saturating cast."""
    b = _pattern_set(1 << 21, 13)
    x = _f32(b)
    for dt, fmt, mx in ((torch.float8_e4m3fn, 0, 448.0), (torch.float8_e5m2, 1, 57344.0)):
        sel = np.abs(x) <= mx
        ref = torch.from_numpy(x[sel].copy()).to(dt).view(torch.uint8).numpy()
        got = oracle.encode_array(x[sel], fmt)
        assert np.array_equal(got, ref), dt


def test_f64_rounding_paths(oracle):
    rng = np.random.default_rng(5)
    d = rng.standard_normal(1 << 16) * np.exp2(rng.uniform(-140, 130, 1 << 16))
    assert np.array_equal(oracle.f32_from_f64(d), d.astype(np.float32))
    # bf16 from fp64 is one rounding: compare with rounding the exact value by hand
    got = oracle.bf16_to_f64(oracle.bf16_from_f64(d[:4096]))
    for v, g in zip(d[:4096], got):
        m, e = math.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
        q = max(e - 8, -133)                      # bf16: 8 significant bits, emin = -126
        n = v / 2.0 ** q                          # exact (power-of-two scaling)
        r = round(n)                              # Python round: ties to even
        want = r * 2.0 ** q
        if abs(want) > 3.3895313892515355e38:
            want = math.copysign(math.inf, v)
        assert g == want, (v, g, want)
