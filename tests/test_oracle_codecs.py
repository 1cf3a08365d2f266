"""Pins of the oracle's number formats (CPU only).

Each format is checked against something other than the oracle itself:
library casts (numpy's float16, torch's bfloat16 / float8_e4m3fn /
float8_e5m2), the OCP specification's closed forms
(tests/golden/e4m3_ocp_codes.txt; E5M2 codes are the upper bytes of binary16
codes) and the round-to-nearest-even rule on every midpoint.
"""

import os

import numpy as np
import pytest
import torch

from oracle import codecs

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
ALL8 = np.arange(256, dtype=np.uint16).astype(np.uint8)


def same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


def test_f16_decode_matches_numpy_float16_on_every_code():
    ref = ALL16.view(np.float16).astype(np.float64)
    assert same(codecs.decode("f16", ALL16), ref)


def test_bf16_decode_matches_torch_on_every_code():
    t = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16)
    assert same(codecs.decode("bf16", ALL16), t.double().numpy())


def test_e4m3_decode_matches_torch_on_every_code():
    t = torch.from_numpy(ALL8.copy()).view(torch.float8_e4m3fn)
    assert same(codecs.decode("e4m3", ALL8), t.double().numpy())


def test_e5m2_is_the_upper_byte_of_binary16():
    # OCP E5M2 shares binary16's sign, exponent and bias; its two mantissa
    # bits are binary16's top two, so code c decodes as the binary16 c << 8.
    ref = (ALL8.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    assert same(codecs.decode("e5m2", ALL8), ref)
    t = torch.from_numpy(ALL8.copy()).view(torch.float8_e5m2)
    assert same(codecs.decode("e5m2", ALL8), t.double().numpy())
    assert codecs.max_finite("e5m2") == 57344.0


def test_e4m3_spec_table(golden_dir):
    with open(os.path.join(golden_dir, "e4m3_ocp_codes.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for code_hex, val in rows:
        got = float(codecs.decode("e4m3", np.array([int(code_hex, 16)]))[0])
        if val == "nan":
            assert np.isnan(got), code_hex
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), code_hex
    assert codecs.max_finite("e4m3") == 448.0
    assert codecs.max_finite("f16") == 65504.0
    assert codecs.max_finite("bf16") == float(torch.finfo(torch.bfloat16).max)


@pytest.mark.parametrize("fmt,codes", [("f16", ALL16), ("bf16", ALL16), ("e4m3", ALL8),
                                       ("e5m2", ALL8)])
def test_encode_inverts_decode(fmt, codes):
    vals = codecs.decode(fmt, codes)
    finite = ~np.isnan(vals)
    back = codecs.encode(fmt, vals[finite])
    assert np.array_equal(back, codes[finite])


@pytest.mark.parametrize("fmt,codes", [("f16", ALL16), ("bf16", ALL16), ("e4m3", ALL8),
                                       ("e5m2", ALL8)])
def test_encode_rounds_midpoints_to_even(fmt, codes):
    ebits, bias, mbits, has_inf, _ = codecs.FORMATS[fmt]
    sign_bit = 1 << (ebits + mbits)
    pos = codes[(codes.astype(np.int64) & sign_bit) == 0].astype(np.int64)
    vals = codecs.decode(fmt, pos)
    ok = np.isfinite(vals)
    lo, v = pos[ok][:-1], vals[ok]
    hi_v, lo_v = v[1:], v[:-1]
    mid = (lo_v + hi_v) / 2                     # exact in float64
    got = codecs.encode(fmt, mid).astype(np.int64)
    expect_even = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect_even)
    # Just off the midpoint the nearer neighbour wins.
    gap = hi_v - lo_v
    assert np.array_equal(codecs.encode(fmt, mid - gap / 8).astype(np.int64), lo)
    assert np.array_equal(codecs.encode(fmt, mid + gap / 8).astype(np.int64), lo + 1)


@pytest.mark.parametrize("fmt,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16),
                                     ("e4m3", torch.float8_e4m3fn),
                                     ("e5m2", torch.float8_e5m2)])
def test_encode_matches_torch_cast_on_random_floats(fmt, tdt):
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 300)])
    x = x.astype(np.float32)
    if fmt == "e4m3":
        x = x[np.abs(x) < 440]
    ref = torch.from_numpy(x).to(tdt)
    ref_codes = ref.view(torch.uint8 if fmt in ("e4m3", "e5m2") else torch.int16).numpy()
    got = codecs.encode(fmt, x.astype(np.float64))
    assert np.array_equal(got.view(ref_codes.dtype), ref_codes)


def test_overflow_rules():
    assert np.isinf(codecs.decode("f16", codecs.encode("f16", [65520.0]))[0])
    assert codecs.decode("f16", codecs.encode("f16", [65519.0]))[0] == 65504.0
    # e4m3 saturates (reading R21): beyond 448 stays 448, never NaN.
    assert codecs.decode("e4m3", codecs.encode("e4m3", [470.0, 1e6, -1e6])).tolist() == [448.0, 448.0, -448.0]
    assert codecs.decode("e4m3", codecs.encode("e4m3", [464.0]))[0] == 448.0
    # e5m2 overflows to inf like binary16 (IEEE rounding: at and beyond the
    # midpoint 61440 between 57344 and the next binade).
    assert np.isinf(codecs.decode("e5m2", codecs.encode("e5m2", [61440.0]))[0])
    assert codecs.decode("e5m2", codecs.encode("e5m2", [61439.0]))[0] == 57344.0
    t = torch.tensor([61440.0, 61439.0]).to(torch.float8_e5m2).double().numpy()
    assert np.isinf(t[0]) and t[1] == 57344.0


def test_e8m0_every_code_against_torch():
    # The OCP MX shared-scale format, all 256 codes, against torch's own
    # float8_e8m0fnu decoding (a library routine).
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = codecs.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[126] == 0.5
