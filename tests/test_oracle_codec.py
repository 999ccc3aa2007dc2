"""Pins of the oracle's E4M3 codec against facts fixed outside the oracle.

* the OCP E4M3 value set written out from the format definition (1 sign,
  4 exponent bits with bias 7, 3 mantissa bits, subnormals m*2^-9, NaN at
  magnitude 0x7F) with exact rational arithmetic;
* brute-force nearest-value search over that value set (ties to the even
  code, saturation at 448) on every bf16 bit pattern and on random fp32;
* the constants and worked values the pages print (tests/golden/e4m3_pins.txt);
* the independent NumPy codec on all 2^16 bf16 inputs times several scales.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import np_codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_pins.txt")


def _exact_value(code: int):
    """E4M3 value of a code from the format definition, as a Fraction (None for NaN)."""
    sign = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return None
    if e == 0:
        mag = Fraction(m, 512)
    else:
        mag = Fraction(8 + m, 8) * (Fraction(2) ** (e - 7))
    return sign, mag


def _finite_table():
    """Sorted non-negative finite values (codes 0x00..0x7E); monotone in the code."""
    vals = np.array([float(_exact_value(c)[1]) for c in range(0x7F)], dtype=np.float64)
    assert np.all(np.diff(vals) > 0)
    return vals


def _bruteforce_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 value by search; ties go to the even code; >=448 saturates."""
    x = x.astype(np.float32)
    vals = _finite_table()
    a = np.abs(x).astype(np.float64)
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    out = np.zeros(x.shape, np.int64)
    fin = np.isfinite(a)
    af = np.where(fin, a, 0.0)
    hi = np.clip(np.searchsorted(vals, af, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dhi = np.abs(vals[hi] - af)
    dlo = np.abs(af - vals[lo])
    pick = np.where(dlo < dhi, lo, hi)
    tie = (dlo == dhi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    out[:] = pick
    out = np.where(af >= 448.0, 0x7E, out)
    out = np.where(np.isinf(a), 0x7E, out)
    out = np.where(np.isnan(a), 0x7F, out)
    return (out.astype(np.uint8) | sign).astype(np.uint8)


def _all_bf16_as_f32() -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    return bits.view(np.float32)


def test_decode_all_256_codes_match_format_definition(orc):
    codes = np.arange(256, dtype=np.uint8)
    dec = orc.e4m3_decode(codes)
    for c in range(256):
        ev = _exact_value(c)
        if ev is None:
            assert math.isnan(dec[c]), hex(c)
            continue
        sign, mag = ev
        assert Fraction(float(abs(dec[c]))) == mag, hex(c)
        assert math.copysign(1.0, float(dec[c])) == sign, hex(c)   # includes -0 for 0x80
    assert int(np.isnan(dec).sum()) == 2


def test_encode_decode_roundtrip_every_finite_code(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert codes.size == 254
    back = orc.e4m3_encode(orc.e4m3_decode(codes))
    assert np.array_equal(back, codes)


def test_encode_is_nearest_value_on_every_bf16_pattern(orc):
    x = _all_bf16_as_f32()
    got = orc.e4m3_encode(x)
    want = _bruteforce_encode(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    # NaN keeps its sign bit and maps to magnitude 0x7F
    assert np.all((got[nan] & 0x7F) == 0x7F)
    assert np.array_equal(got[nan] & 0x80, np.where(np.signbit(x[nan]), 0x80, 0).astype(np.uint8))


@pytest.mark.parametrize("seed", [0, 1])
def test_encode_is_nearest_value_on_random_fp32(orc, seed):
    rng = np.random.default_rng(seed)
    # log-uniform magnitudes spanning subnormal fp32 to beyond saturation, plus grid midpoints
    mags = np.exp2(rng.uniform(-140, 12, size=400_000)).astype(np.float32)
    vals = _finite_table()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    nudged = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    x = np.concatenate([mags, nudged]).astype(np.float32)
    x = np.where(rng.random(x.size) < 0.5, -x, x).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(x), _bruteforce_encode(x))


def _parse_real(tok: str) -> np.float32:
    if tok == "-0":
        return np.float32(-0.0)
    return np.float32(float(tok))


def test_golden_pins_from_pages(orc):
    n = 0
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            body = line.split("|")[0].split()
            op, inp, exp = body
            if op == "decode":
                got = orc.e4m3_decode(np.array([int(inp, 16)], np.uint8))[0]
                if exp == "nan":
                    assert math.isnan(got), line
                else:
                    want = _parse_real(exp)
                    assert got == want and math.copysign(1, got) == math.copysign(1, want), line
            else:
                got = orc.e4m3_encode(np.array([_parse_real(inp)], np.float32))[0]
                assert got == int(exp, 16), line
            n += 1
    assert n >= 30


SCALES = [1.0, 0.5, 0.02, 0.015, 0.03, 0.2087, 6.0 / 448.0, 2.0 ** -7, 2.0 ** -13, 1e-30, -0.125]


def test_numpy_codec_agrees_with_c_codec_on_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    a, b = orc.e4m3_decode(codes), np_codec.decode(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    m = ~np.isnan(a)
    assert np.array_equal(a[m].view(np.uint32), b[m].view(np.uint32))


@pytest.mark.parametrize("scale", SCALES)
def test_numpy_codec_agrees_with_c_codec_on_all_bf16_times_scale(orc, scale):
    x = _all_bf16_as_f32()
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (x * inv).astype(np.float32)
    y = np.where(np.isnan(x), x, y).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(y), np_codec.encode(y))


def test_tiny_negative_and_fp32_subnormals_keep_sign(orc):
    x = np.array([-1e-40, 1e-40, -2.0 ** -11, 2.0 ** -11, -np.float32(1.4e-45)], np.float32)
    assert list(orc.e4m3_encode(x)) == [0x80, 0x00, 0x80, 0x00, 0x80]
