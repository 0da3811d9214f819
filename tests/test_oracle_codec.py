"""Pins for the oracle's FP8 / INT8 / BF16 codecs (CPU only).

The pages fix the formats (AstrAI ops/fp8.py @5e76fbd, ``_fmt_dtype``:
torch.float8_e4m3fn and torch.float8_e5m2), round-half-to-even (POPCORNBENCH
"Kimi-K2.6 l2_p13", the nearbyintf discussion) and, through the quantize
contract, saturation.  These tests pin the oracle's codecs by brute-force
enumeration of all 256 codes, by the formats' limits, and against torch's
independent CPU casts wherever torch and the contract agree (finite values
below the format maximum; torch does not saturate above it).
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden

FMTS = [(0, torch.float8_e4m3fn, 448.0, 0x7E, -9), (1, torch.float8_e5m2, 57344.0, 0x7B, -16)]


def _finite_positive_codes(orc, fmt):
    return [c for c in range(0x80) if math.isfinite(orc.fp8_decode(c, fmt))]


@pytest.mark.parametrize("fmt,tdt,maxv,maxcode,minsub", FMTS)
def test_decode_matches_torch_all_codes(orc, fmt, tdt, maxv, maxcode, minsub):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(tdt).to(torch.float64).numpy()
    mine = np.array([orc.fp8_decode(c, fmt) for c in range(256)])
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(mine))
    assert np.array_equal(ref[~nan_ref], mine[~nan_ref])
    # signed zero
    assert math.copysign(1.0, orc.fp8_decode(0x80, fmt)) == -1.0


@pytest.mark.parametrize("fmt,tdt,maxv,maxcode,minsub", FMTS)
def test_limits(orc, fmt, tdt, maxv, maxcode, minsub):
    assert orc.fp8_decode(maxcode, fmt) == maxv
    assert orc.fp8_decode(maxcode | 0x80, fmt) == -maxv
    assert orc.fp8_decode(0x01, fmt) == 2.0 ** minsub
    assert orc.fp8_encode(2.0 ** minsub, fmt) == 0x01
    if fmt == 0:
        assert math.isnan(orc.fp8_decode(0x7F, fmt)) and math.isnan(orc.fp8_decode(0xFF, fmt))
    else:
        assert orc.fp8_decode(0x7C, fmt) == math.inf and orc.fp8_decode(0xFC, fmt) == -math.inf
        assert all(math.isnan(orc.fp8_decode(c, fmt)) for c in (0x7D, 0x7E, 0x7F))


@pytest.mark.parametrize("fmt,tdt,maxv,maxcode,minsub", FMTS)
def test_decode_encode_identity(orc, fmt, tdt, maxv, maxcode, minsub):
    for c in range(256):
        v = orc.fp8_decode(c, fmt)
        if math.isfinite(v):
            assert orc.fp8_encode(v, fmt) == c, hex(c)


@pytest.mark.parametrize("fmt,tdt,maxv,maxcode,minsub", FMTS)
def test_midpoints_round_to_even(orc, fmt, tdt, maxv, maxcode, minsub):
    codes = _finite_positive_codes(orc, fmt)
    vals = [orc.fp8_decode(c, fmt) for c in codes]
    for (c0, v0), (c1, v1) in zip(zip(codes, vals), zip(codes[1:], vals[1:])):
        mid = (v0 + v1) / 2.0
        even = c0 if c0 % 2 == 0 else c1
        assert orc.fp8_encode(mid, fmt) == even, (hex(c0), hex(c1))
        assert orc.fp8_encode(-mid, fmt) == even | 0x80
        assert orc.fp8_encode(np.nextafter(mid, -np.inf), fmt) == c0
        assert orc.fp8_encode(np.nextafter(mid, np.inf), fmt) == c1


@pytest.mark.parametrize("fmt,tdt,maxv,maxcode,minsub", FMTS)
def test_saturation_and_specials(orc, fmt, tdt, maxv, maxcode, minsub):
    for v in (maxv, maxv * 1.0001, maxv * 1.1, 1e30, math.inf):
        assert orc.fp8_encode(v, fmt) == maxcode
        assert orc.fp8_encode(-v, fmt) == maxcode | 0x80
    assert orc.fp8_encode(0.0, fmt) == 0x00
    assert orc.fp8_encode(-0.0, fmt) == 0x80
    # below half the minimum subnormal: signed zero
    assert orc.fp8_encode(2.0 ** (minsub - 1) * 0.999, fmt) == 0x00
    assert orc.fp8_encode(-(2.0 ** (minsub - 1)), fmt) == 0x80     # tie to even (0)
    assert orc.fp8_encode(math.nan, fmt) & 0x7F == 0x7F


@pytest.mark.parametrize("fmt,tdt,maxv,maxcode,minsub", FMTS)
def test_encode_monotone(orc, fmt, tdt, maxv, maxcode, minsub):
    xs = np.concatenate([-np.geomspace(maxv * 2, 2.0 ** (minsub - 3), 4000), [0.0],
                         np.geomspace(2.0 ** (minsub - 3), maxv * 2, 4000)])
    prev = -math.inf
    for x in xs:
        v = orc.fp8_decode(orc.fp8_encode(float(x), fmt), fmt)
        v = 0.0 if v == 0 else v
        assert v >= prev
        prev = v


@pytest.mark.parametrize("fmt,tdt,maxv,maxcode,minsub", FMTS)
def test_encode_matches_torch_below_max(orc, fmt, tdt, maxv, maxcode, minsub):
    """Every finite BF16 pattern plus 200k random FP32 values below the format
    maximum: the oracle's encode equals torch's independent cast."""
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    vals = bits.view(np.float32)
    rng = np.random.default_rng(1234)
    extra = (rng.standard_normal(200_000) * np.exp(rng.uniform(-14, 11, 200_000))).astype(np.float32)
    vals = np.concatenate([vals, extra])
    vals = vals[np.isfinite(vals) & (np.abs(vals) < maxv)]
    ref = torch.from_numpy(vals).to(tdt).view(torch.uint8).numpy()
    enc = np.frompyfunc(lambda v: orc.fp8_encode(float(v), fmt), 1, 1)
    mine = enc(vals).astype(np.uint8)
    bad = np.nonzero(ref != mine)[0]
    assert bad.size == 0, [(float(vals[i]), hex(ref[i]), hex(mine[i])) for i in bad[:5]]


def test_int8_ties_from_the_pages(orc):
    """The six ties worked on the POPCORNBENCH trace page (round half to even)."""
    rows = list(read_golden("int8_rne_ties.txt"))
    assert len(rows) == 6
    for x, code in rows:
        assert orc.int8_encode(float(x)) == int(code)


def test_int8_encode_matches_torch_round(orc):
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-140, 140, 100_000).astype(np.float32),
                        np.arange(-140, 140.5, 0.5, dtype=np.float32)])
    ref = torch.clamp(torch.round(torch.from_numpy(v)), -127, 127).numpy().astype(np.int64)
    mine = np.array([orc.int8_encode(float(x)) for x in v])
    assert np.array_equal(ref, mine)
    assert orc.int8_encode(-1e9) == -127 and orc.int8_encode(1e9) == 127


def test_bf16_decode_all_patterns(orc):
    """Oracle BF16 input decode (via amax of single elements) equals torch's."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(t)
    x = bits[finite].reshape(-1, 1)
    got = orc.amax_raw(x, orc.PER_ROW)
    assert np.array_equal(got, np.abs(t[finite]))


def test_div_f32_correctly_rounded(orc):
    """fl32(x/s) equals torch's FP32 division (IEEE, correctly rounded)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20_000) * np.exp(rng.uniform(-20, 20, 20_000))).astype(np.float32)
    s = (np.exp(rng.uniform(-30, 30, 20_000))).astype(np.float32)
    ref = (torch.from_numpy(x) / torch.from_numpy(s)).numpy()
    mine = np.array([orc.div_f32(a, b) for a, b in zip(x, s)], dtype=np.float32)
    assert np.array_equal(ref.view(np.uint32), mine.view(np.uint32))
