"""Number formats the oracle reads and writes, in fp64.

TEST INFRASTRUCTURE ONLY (see the package header).

* bf16: the upper 16 bits of an IEEE-754 binary32.
* OCP E4M3 per the OCP 8-bit Floating Point Specification (OFP8), rev. 1.0,
  section "E4M3": 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
  is subnormal; S.1111.111 is NaN; there is no infinity; the largest finite
  magnitude is 448 (S.1111.110).

Parity pins (tests/test_oracle_formats.py): every one of the 256 E4M3 codes
against PyTorch's ``float8_e4m3fn`` dtype and against the spec's named values
(tests/golden/e4m3_ocp_values.json); the encoder against PyTorch's cast on
dense grids and random values, plus brute-force nearest search at midpoints.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode OCP E4M3 codes: value = (-1)^s * 2^(E-7) * (1 + M/8), or 2^-6 * M/8 if E == 0."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def _e4m3_positive_table():
    codes = np.arange(0x7F)                 # 0x00 .. 0x7E, all finite, increasing
    return codes, e4m3_to_f64(codes)


def e4m3_encode(x) -> np.ndarray:
    """fp64 -> OCP E4M3 code: round to the nearest representable value, ties to the
    code with an even mantissa, magnitudes past 448 saturate to 448, NaN -> 0x7F.
    The sign bit is kept (a negative value rounding to zero gives 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _e4m3_positive_table()
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)   # vals[hi] >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    c = np.where(pick_hi, codes[hi], codes[lo])
    c = np.where(np.signbit(x), c | 0x80, c)
    return np.where(np.isnan(x), E4M3_NAN_CODE, c).astype(np.uint8)
