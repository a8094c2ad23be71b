"""Pins for the oracle's value codecs (CPU only)."""
import math
import os

import numpy as np
import pytest

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_table_matches_format_definition_points():
    for code, value in _golden():
        got = codecs.e4m3_value(code)
        if math.isnan(value):
            assert math.isnan(got), hex(code)
        else:
            assert got == value, hex(code)
            assert math.copysign(1.0, got) == math.copysign(1.0, value), hex(code)


def test_e4m3_table_is_monotone_and_has_two_nans():
    t = codecs.E4M3_TABLE
    assert np.isnan(t).sum() == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -pos)


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.E4M3_TABLE[codes].astype(np.float32)
    assert np.array_equal(codecs.f32_to_e4m3(vals), codes)


def test_e4m3_encode_ties_to_even_and_saturates():
    # midpoint of 1.0 (0x38, even) and 1.125 (0x39) -> 0x38
    assert codecs.f32_to_e4m3(np.float32(1.0625)) == 0x38
    # midpoint of 1.125 (0x39) and 1.25 (0x3A, even) -> 0x3A
    assert codecs.f32_to_e4m3(np.float32(1.1875)) == 0x3A
    # just above a midpoint rounds up, just below rounds down
    assert codecs.f32_to_e4m3(np.nextafter(np.float32(1.0625), np.float32(2))) == 0x39
    assert codecs.f32_to_e4m3(np.nextafter(np.float32(1.1875), np.float32(0))) == 0x39
    # subnormal midpoint between 0 and 2^-9 -> 0 (even); 1.5 * 2^-9 -> 2 * 2^-9
    assert codecs.f32_to_e4m3(np.float32(2.0 ** -10)) == 0x00
    assert codecs.f32_to_e4m3(np.float32(1.5 * 2.0 ** -9)) == 0x02
    # saturation: 448 and anything larger -> 0x7E; sign kept
    for v in (448.0, 449.0, 464.0, 480.0, 1e6):
        assert codecs.f32_to_e4m3(np.float32(v)) == 0x7E
        assert codecs.f32_to_e4m3(np.float32(-v)) == 0xFE
    # negative value rounding to zero keeps the sign bit
    assert codecs.f32_to_e4m3(np.float32(-1e-4)) == 0x80


def test_e4m3_encode_is_nearest_value():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 100).astype(np.float32)
    codes = codecs.f32_to_e4m3(x)
    dec = codecs.E4M3_TABLE[codes]
    fin = codecs.E4M3_TABLE[np.isfinite(codecs.E4M3_TABLE)]
    xm = np.clip(x.astype(np.float64), -448, 448)
    best = np.min(np.abs(fin[None, :] - xm[:, None]), axis=1)
    assert np.array_equal(np.abs(dec - xm), best)


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    got = codecs.bf16_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -1.0
    assert got[2] == 3.140625
    assert got[3] == 0.0 and math.copysign(1, got[4]) == -1
    assert got[5] == (2 - 2 ** -7) * 2.0 ** 127
