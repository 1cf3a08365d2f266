"""Number formats used by the engine's operands and outputs (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Formats, each a sign bit, ``E`` exponent bits with bias ``B`` and ``M``
stored mantissa bits:

* ``f16``   -- IEEE-754 binary16: E=5, B=15, M=10, infinities and NaNs.
* ``bf16``  -- bfloat16: E=8, B=127, M=7, infinities and NaNs.
* ``e4m3``  -- OCP 8-bit floating point, E4M3 variant: E=4, B=7, M=3.  No
               infinities; the single NaN pattern per sign is exponent 1111
               with mantissa 111; the largest finite value is 448.  This is the
               fp8 encoding gfx950 uses (the "gemm_rowcolquant dispatcher
               bridge" PR, round-3 fixes: OCP on gfx950, FNUZ on gfx942).
* ``e5m2``  -- OCP 8-bit floating point, E5M2 variant ("bf8" on that PR):
               E=5, B=15, M=2, infinities and NaNs as in IEEE-754; its codes
               are the upper bytes of binary16 codes.

* ``e8m0``  -- the OCP Microscaling (MX) shared block scale: an unsigned
               8-bit exponent with bias 127 and no mantissa, value
               2^(code - 127) for codes 0..254; code 255 is NaN (decode only,
               ``decode_e8m0``: scales are drawn as codes, never rounded).

Decoding is exact in float64.  Encoding rounds to nearest, ties to even.
Values beyond the largest finite number become +/-inf for f16 / bf16 / e5m2
(IEEE overflow under round-to-nearest) and saturate to +/-448 for e4m3 (our reading:
the pages only name the OCP encoding; saturation is the conventional
"satfinite" conversion and never triggers on the workloads, whose fp8 data is
quantised N(0,1)).
"""

import numpy as np

# name -> (exponent bits, bias, mantissa bits, has_inf, storage bytes)
FORMATS = {
    "f16": (5, 15, 10, True, 2),
    "bf16": (8, 127, 7, True, 2),
    "e4m3": (4, 7, 3, False, 1),
    "e5m2": (5, 15, 2, True, 1),
}


def storage_dtype(fmt):
    """numpy unsigned integer type that holds one code of ``fmt``."""
    return np.uint16 if FORMATS[fmt][4] == 2 else np.uint8


def decode(fmt, codes):
    """Exact float64 value of every code in ``codes`` (any integer array)."""
    ebits, bias, mbits, has_inf, _ = FORMATS[fmt]
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> (ebits + mbits)) & 1
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    mag = np.where(
        e == 0,
        np.ldexp(m.astype(np.float64), 1 - bias - mbits),           # subnormal
        np.ldexp((m + (1 << mbits)).astype(np.float64), e - bias - mbits),
    )
    if has_inf:
        mag = np.where((e == emax_field) & (m == 0), np.inf, mag)
        mag = np.where((e == emax_field) & (m != 0), np.nan, mag)
    else:
        # OCP E4M3: only S.1111.111 is NaN; the rest of exponent 1111 is finite.
        mag = np.where((e == emax_field) & (m == (1 << mbits) - 1), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def max_finite(fmt):
    ebits, bias, mbits, has_inf, _ = FORMATS[fmt]
    emax_field = (1 << ebits) - 1
    if has_inf:
        return float(np.ldexp((1 << (mbits + 1)) - 1, emax_field - 1 - bias - mbits))
    return float(np.ldexp((1 << (mbits + 1)) - 2, emax_field - bias - mbits))


def encode(fmt, x):
    """Round float64 values to the nearest ``fmt`` code (ties to even)."""
    ebits, bias, mbits, has_inf, _ = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.int64)
    a_in = np.abs(x)
    a = np.where(np.isfinite(a_in), a_in, 0.0)   # inf / NaN patched in below
    emin = 1 - bias                      # exponent of the smallest normal
    # Exponent of the binade holding a (clamped to the subnormal binade).
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    # log2 of values just below a power of two can round up; fix both ways.
    e = np.where(np.ldexp(1.0, e) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= a, e + 1, e)
    e = np.maximum(e, emin)
    # Number of quanta of size 2^(e - mbits); exact scaling by a power of two.
    n = np.rint(np.ldexp(a, -(e - mbits)))            # rint = ties to even
    # A carry out of the mantissa moves the value to the next binade.
    carry = n >= (1 << (mbits + 1))
    e = np.where(carry, e + 1, e)
    n = np.where(carry, n / 2, n).astype(np.int64)
    is_normal = n >= (1 << mbits)
    efield = np.where(is_normal, e + bias, 0)
    mfield = np.where(is_normal, n - (1 << mbits), n)
    code = (efield << mbits) | mfield
    emax_field = (1 << ebits) - 1
    if has_inf:
        overflow = efield >= emax_field
        code = np.where(overflow, emax_field << mbits, code)
        nan_code = (emax_field << mbits) | (1 << (mbits - 1))
        code = np.where(np.isinf(a_in), emax_field << mbits, code)
    else:
        max_code = (emax_field << mbits) | ((1 << mbits) - 2)
        code = np.where((efield > emax_field) | (code > max_code), max_code, code)
        code = np.where(np.isinf(a_in), max_code, code)
        nan_code = (emax_field << mbits) | ((1 << mbits) - 1)
    code = np.where(np.isnan(x), nan_code, code)
    code = code | (sign << (ebits + mbits))
    return code.astype(storage_dtype(fmt))


def decode_e8m0(codes):
    """Exact float64 value of OCP MX E8M0 scale codes: 2^(code - 127), NaN
    for 255."""
    c = np.asarray(codes).astype(np.int64)
    if ((c < 0) | (c > 255)).any():
        raise ValueError("e8m0 codes are bytes")
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))
