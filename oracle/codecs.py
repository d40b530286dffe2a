"""Number formats, written from their definitions (oracle; test infrastructure only).

bf16: 1 sign bit, 8 exponent bits (bias 127, the fp32 exponent range), 7
fraction bits.  Rounding is IEEE round-to-nearest, ties to even, done here by
scaling to the unit in the last place and calling rint (which rounds half to
even); all arithmetic is exact in fp64.

E4M3 (OCP 8-bit floating point, the "FN" variant): 1 sign bit, 4 exponent bits
(bias 7), 3 fraction bits; exponent field 0 holds subnormals m * 2^-9; the
code S.1111.111 is NaN; there are no infinities; the largest finite magnitude
is 1.75 * 2^8 = 448.  Encoding here is round-to-nearest, ties to the code with
an even fraction, saturating: magnitudes above 448 (and infinities) map to 448.
The pages use NVFP4 on Blackwell; fp8 E4M3 is the substitute format of this
build (no passage of the pages defines it).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------------------------
# bf16

def bf16_round(x) -> np.ndarray:
    """Round fp32/fp64 numbers to the nearest bf16 value (ties to even); returns float64 values."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)              # xf = m * 2^e with 0.5 <= |m| < 1, so the leading bit is 2^(e-1)
    lead = e - 1
    lead = np.maximum(lead, -126)    # below the smallest normal the spacing stays 2^-133
    ulp = np.ldexp(1.0, lead - 7)
    r = np.rint(xf / ulp) * ulp      # exact: xf/ulp has at most ~53 significant bits
    r[np.abs(r) >= 2.0 ** 128] = np.inf * np.sign(r[np.abs(r) >= 2.0 ** 128])
    out[fin] = r
    return out


def bf16_bits(x) -> np.ndarray:
    """bf16 storage bits (uint16) of the bf16 rounding of x."""
    v = bf16_round(x).astype(np.float32)   # exact: bf16 values are fp32 values
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    """float64 values of bf16 storage bits."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# E4M3

E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        ef = (code >> 3) & 0xF
        m = code & 0x7
        if ef == 0xF and m == 0x7:
            vals[code] = np.nan
        elif ef == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (ef - 7)
    return vals


E4M3_VALUES = _e4m3_table()                  # value of every code (NaN for 0x7F, 0xFF)
_POS = E4M3_VALUES[:0x7F]                    # codes 0x00..0x7E: 0 .. 448, strictly increasing


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Encode numbers to E4M3 codes: nearest value, ties to even fraction, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    hi = np.searchsorted(_POS, a, side="left")          # first table value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.where(_POS[hi] > a, hi - 1, hi)             # last table value <= a
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    return code
